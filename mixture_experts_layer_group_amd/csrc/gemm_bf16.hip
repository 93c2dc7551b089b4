// Grouped expert GEMMs on CDNA4 matrix cores (fp32 accumulation) over the
// ragged per-expert row groups that the dispatch produced: all routed
// experts are evaluated by one launch per projection instead of a loop over
// experts (dockyard_rl "Mixture-of-Experts" page, "The pipeline", grouped
// GEMM), with the two products per expert of the "Mixture of Experts" blog
// page's third program (moe_forward).
//
//   up   (GEMM1): H[r, f] = act(x[tok(r)] . W_gate[e][f] (, x . W_up[e][f]))
//                 SwiGLU = silu(gate) * up (Edge0 "MoE Spec and Routing",
//                 _swiglu); ReLU ("Mixture of Experts" blog, expert_forward)
//                 bf16 x bf16 products, H stored as fp16
//   down (GEMM2): Y[r, n] = H[r] . W_down[e][n]   fp16 x fp16 products (the
//                 bf16 weights are converted in registers), Y kept in fp32
//
// H is held in fp16 rather than bf16: its 3 extra mantissa bits keep the
// rounding between the two products 8x smaller, which the layer's
// max-norm output tolerance needs when drops leave a few tokens far above
// the output RMS; the hidden activations are O(1), well inside fp16 range
// (the conversion saturates at +-65504).
//
// Kernel shape (gfx950):
//   * a 256 x 256 output tile per 512-thread workgroup, K steps of 64;
//     each of the 8 waves (2 per SIMD, so one fills the other's issue gaps)
//     owns a 128 x 64 sub-tile = 4 x 2 blocks of v_mfma_f32_32x32x16;  The weight tile is the MFMA A operand
//     (rows = output columns) and the activation tile the B operand, so a
//     lane's accumulators hold 4 consecutive output columns of one row;
//   * both operands are K-contiguous in HBM (weights are [out, in]) and go
//     straight from HBM to LDS (buffer_load_dwordx4 ... lds, no staging
//     registers) into double-buffered tiles (2 x 64 KiB); the next K step is
//     in flight while the current one is multiplied.  The 16-byte chunks of
//     each 128-byte LDS row are XOR-swizzled (conflict-free for 8- and
//     16-lane LDS phases); the swizzle is applied on the global side, since
//     a direct load writes LDS at lane*16;
//   * activation rows are gathered on load through sorted_token (no
//     permuted copy of x);
//   * SwiGLU: a tile's 256 weight rows are 128 gate rows then the same 128
//     up rows; each wave holds gate and up accumulators of the same
//     (row, column) in the same lanes, so the epilogue fuses silu(g) * u;
//   * ragged groups without a host sync: the grid is an upper bound on the
//     tile count; each workgroup reads the per-expert M-tile prefix written
//     by the dispatch and exits if surplus.  Workgroup ids are remapped so
//     that each of the 8 XCDs (hardware dispatch is round-robin over XCDs)
//     gets a contiguous range of tiles, ordered 8 N-tiles fastest inside an
//     expert's M-tiles, so concurrently running tiles on one XCD share
//     weight and activation tiles in its L2.
#include <algorithm>
#include <type_traits>

#include "moe_internal.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kRowBytes = BK * 2;           // 128
constexpr int kTileBytes = BM * kRowBytes;  // 32 KiB per operand per stage
constexpr int kNG = 8;                      // N-tiles per scheduling column group
constexpr int kWaves = 8;                   // 2 waves per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kWavesN = 4;                  // waves along N (2 along M)
constexpr int MB = 4, NB = 2;               // 32x32 blocks per wave: 128 x 64
constexpr int kLoads = 32 / kWaves;         // 1 KiB direct loads per operand per wave
static_assert(BM == kGemm1BM && BM == kGemm2BM, "tile prefix BM mismatch");

enum Mode { kSwiGLU = 0, kReLU = 1, kDown = 2 };

struct GemmArgs {
  const uint16_t* a;            // activation rows (x or H)
  const int32_t* sorted_token;  // gather table (nullptr: row = group row)
  const int32_t* offsets;       // [E+1] group row offsets (nullptr: one group)
  const int32_t* tiles;         // [E+1] group M-tile prefix (nullptr: one group)
  int E;
  int32_t single_rows;          // rows of the single group
  const uint16_t* w0;           // gate / in / down  [E][N][K]
  const uint16_t* w1;           // up (SwiGLU)
  int N;                        // weight rows per expert
  int K;                        // reduction length (row length of a and w)
  void* out;                    // [rows][ldo]: bf16 H (up), fp32 Y (down)
  int ldo;                      // output row length (F or d)
  int NT;                       // N tiles
};

// byte offset of 16-byte chunk c (0..7) of row r inside a swizzled tile.
// The XOR pattern keeps the 32 rows read by one MFMA fragment load on
// distinct banks whether the LDS serves 8 lanes (32 banks) or 16 lanes (64
// banks) of a 16-byte read per cycle.
__device__ __forceinline__ int swz(int r, int c) {
  return r * kRowBytes + ((c ^ ((r ^ (r >> 3)) & 7)) << 4);
}

__device__ __forceinline__ int largest_le(const int32_t* __restrict__ p, int E,
                                          int32_t v) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p[mid] <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float silu(float z) { return z / (1.f + __expf(-z)); }

// hidden activation -> fp16, round to nearest even, saturating at +-65504
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  a = fminf(fmaxf(a, -65504.f), 65504.f);
  b = fminf(fmaxf(b, -65504.f), 65504.f);
  const _Float16 ha = static_cast<_Float16>(a), hb = static_cast<_Float16>(b);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ha)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hb)) << 16);
}

// 8 bf16 weights -> 8 fp16 (exact for normal fp16 values; v_cvt_pkrtz
// saturates instead of overflowing)
__device__ __forceinline__ half8 bf16x8_to_f16x8(bf16x8 v) {
  const uint4 u = __builtin_bit_cast(uint4, v);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(
                                            __uint_as_float(w[j] << 16),
                                            __uint_as_float(w[j] & 0xffff0000u)));
  return __builtin_bit_cast(half8, make_uint4(o[0], o[1], o[2], o[3]));
}

template <int MODE, bool GATHER>
__global__ void __launch_bounds__(kThreads, 1)
grouped_gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kTileBytes];
  uint8_t* sA = smem;                   // [2][BM rows][128 B]
  uint8_t* sW = smem + 2 * kTileBytes;  // [2][BN rows][128 B]

  // ---------------- tile scheduling
  const int total_mt = g.tiles ? g.tiles[g.E] : (g.single_rows + BM - 1) / BM;
  const int real = total_mt * g.NT;
  const int share = (real + 7) >> 3;
  const int bid = blockIdx.x;
  const int local = bid >> 3;
  if (local >= share) return;
  const int L = (bid & 7) * share + local;
  if (L >= real) return;
  int gm, nt;
  {
    const int full = g.NT / kNG;
    const int colgrp = L / (total_mt * kNG);
    if (colgrp < full) {
      const int rem = L - colgrp * total_mt * kNG;
      gm = rem / kNG;
      nt = colgrp * kNG + rem % kNG;
    } else {
      const int ng = g.NT - full * kNG;
      const int rem = L - full * total_mt * kNG;
      gm = rem / ng;
      nt = full * kNG + rem % ng;
    }
  }
  int e = 0, row0, cnt, mt;
  if (g.tiles) {
    e = largest_le(g.tiles, g.E, gm);
    mt = gm - g.tiles[e];
    row0 = g.offsets[e];
    cnt = g.offsets[e + 1] - row0;
  } else {
    mt = gm;
    row0 = 0;
    cnt = g.single_rows;
  }
  const int m0 = mt * BM;  // first row of this tile inside the group

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;

  // ---------------- direct-to-LDS load descriptors
  // Each wave-wide buffer_load_dwordx4 ... lds fills 1 KiB of LDS (8 rows of
  // 128 B) at lane*16; lane l therefore fetches the global chunk that the
  // swizzle places at position l%8 of row l/8.  Wave w issues blocks
  // j*kWaves + w of each 32 KiB operand tile.
  const int64_t K = g.K;
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(g.a), (short)0, -1, 0x00020000);
  const uint16_t* wbase0 = g.w0 + static_cast<int64_t>(e) * g.N * K;
  const uint16_t* wbase1 = (MODE == kSwiGLU ? g.w1 : g.w0) + static_cast<int64_t>(e) * g.N * K;
  const __amdgpu_buffer_rsrc_t rsW0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(wbase0), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsW1 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(wbase1), (short)0, -1, 0x00020000);
  uint32_t voffA[kLoads], voffW[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int r = (j * kWaves + wave) * 8 + (lane >> 3);  // tile row
    const int c = (lane & 7) ^ ((r ^ (r >> 3)) & 7);     // chunk at position lane%8
    int m = m0 + r;
    if (m > cnt - 1) m = cnt - 1;  // clamp ragged tail to a valid row
    const int64_t arow = GATHER ? static_cast<int64_t>(g.sorted_token[row0 + m])
                                : static_cast<int64_t>(row0 + m);
    voffA[j] = static_cast<uint32_t>(arow * K * 2 + c * 16);
    int n = (MODE == kSwiGLU) ? nt * (BN / 2) + (r & 127) : nt * BN + r;
    if (n > g.N - 1) n = g.N - 1;
    voffW[j] = static_cast<uint32_t>(static_cast<int64_t>(n) * K * 2 + c * 16);
  }

  // ---------------- per-lane fragment offsets
  // MFMA 32x32x16: lane l supplies row (l % 32), K elements 8*(l/32)..+8.
  // A wave owns 128 activation rows (4 blocks) and 64 weight rows (2
  // blocks); for SwiGLU those are 32 gate rows and the matching 32 up rows.
  const int fr = lane & 31;
  const int fh = lane >> 5;
  int wrow[NB], arow_l[MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (MODE == kSwiGLU)
      wrow[nb] = (nb ? 128 : 0) + wn * 32 + fr;
    else
      wrow[nb] = wn * 64 + nb * 32 + fr;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) arow_l[mb] = wm * 128 + mb * 32 + fr;

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = g.K / BK;
  auto issue = [&](int kt, int buf) {
    const int soff = kt * kRowBytes;  // K advance in bytes
    uint8_t* a = sA + buf * kTileBytes;
    uint8_t* w = sW + buf * kTileBytes;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int blk = (j * kWaves + wave) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsA, (__attribute__((address_space(3))) void*)(a + blk), 16, voffA[j],
          soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          j < kLoads / 2 ? rsW0 : rsW1,
          (__attribute__((address_space(3))) void*)(w + blk), 16, voffW[j], soff,
          0, 0);
    }
  };

  // fragments are double-buffered in registers: the LDS reads for K
  // sub-step s+1 are in flight while the MFMAs of sub-step s run.  The next
  // K tile's first fragments are read right after the barrier that
  // publishes it, ahead of the current tile's last MFMAs.  On the fp16 path
  // the weight fragments are read raw (bf16) and converted later in the
  // sub-step, so no conversion waits on its LDS read.
  using frag_t = typename std::conditional<MODE == kDown, half8, bf16x8>::type;
  frag_t wf[2][NB], af[2][MB];
  bf16x8 wraw[2][NB];
  auto read_frags = [&](int buf, int ks, int fb) {
    const uint8_t* a = sA + buf * kTileBytes;
    const uint8_t* w = sW + buf * kTileBytes;
    const int ch = ks * 2 + fh;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (MODE == kDown)
        wraw[fb][nb] = *reinterpret_cast<const bf16x8*>(w + swz(wrow[nb], ch));
      else
        wf[fb][nb] = *reinterpret_cast<const bf16x8*>(w + swz(wrow[nb], ch));
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      af[fb][mb] = *reinterpret_cast<const frag_t*>(a + swz(arow_l[mb], ch));
  };
  auto convert = [&](int fb) {
    if constexpr (MODE == kDown) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wf[fb][nb] = bf16x8_to_f16x8(wraw[fb][nb]);
    }
  };
  auto mfmas = [&](int fb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (MODE == kDown)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              wf[fb][nb], af[fb][mb], acc[nb][mb], 0, 0, 0);
        else
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              wf[fb][nb], af[fb][mb], acc[nb][mb], 0, 0, 0);
      }
  };

  // Instruction pacing (8 MFMAs and 6 fragment reads per sub-step).  Plain
  // sub-step: each fragment read of the next sub-step sits between MFMAs of
  // the current one.  Sub-step 0 also issues the next K tile's direct loads;
  // a direct load writes LDS, so the compiler keeps fragment reads and
  // direct loads in program order -- there the reads go first and the loads
  // are paired with the MFMAs.  The fp16 path places the weight
  // conversions (about 12 VALU ops per fragment) in the second half.
  auto pace = [&]() {
#pragma unroll
    for (int i = 0; i < NB + MB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
#pragma unroll
    for (int i = NB + MB; i < NB * MB; ++i) {
      if (MODE == kDown) __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
  };
  auto pace_loads = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, NB + MB, 0);  // DS read
#pragma unroll
    for (int i = 0; i < NB * MB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x020, 2 * kLoads / (NB * MB), 0);  // VMEM
      if (MODE == kDown) __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
  };
  auto tile = [&](int kt, auto last_tag) {
    constexpr bool last = decltype(last_tag)::value;
    const int cur = kt & 1;
    read_frags(cur, 1, 1);
    if constexpr (!last) {
      issue(kt + 1, cur ^ 1);
      mfmas(0);
      convert(1);
      pace_loads();
    } else {
      mfmas(0);
      convert(1);
      pace();
    }
    read_frags(cur, 2, 0);
    mfmas(1);
    convert(0);
    pace();
    read_frags(cur, 3, 1);
    mfmas(0);
    convert(1);
    pace();
    if constexpr (!last) {
      // every read of this tile is issued: wait for them and for the next
      // tile's loads, publish the next tile, and read its first fragments
      // ahead of this tile's last MFMAs
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __syncthreads();
      read_frags(cur ^ 1, 0, 0);
      mfmas(1);
      convert(0);
      pace();
    } else {
      mfmas(1);
    }
  };

  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  read_frags(0, 0, 0);
  convert(0);
  for (int kt = 0; kt + 1 < KT; ++kt) tile(kt, std::false_type{});
  tile(KT - 1, std::true_type{});

  // ---------------- epilogue
  // lane holds, for block (nb, mb) and item v: output column
  //   colbase(nb) + 8*(v/4) + 4*(lane/32) + v%4, row arow_l[mb].
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + arow_l[mb];
    if (m >= cnt) continue;
    const int64_t orow_off = static_cast<int64_t>(row0 + m) * g.ldo;
    uint16_t* orow = static_cast<uint16_t*>(g.out) + orow_off;
    float* orow_f = static_cast<float*>(g.out) + orow_off;
    if (MODE == kSwiGLU) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = nt * (BN / 2) + wn * 32 + 8 * q + 4 * fh;
        if (col >= g.N) continue;
        float h[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          h[v] = silu(acc[0][mb][4 * q + v]) * acc[1][mb][4 * q + v];
        uint2 pk;
        pk.x = pack_h2(h[0], h[1]);
        pk.y = pack_h2(h[2], h[3]);
        *reinterpret_cast<uint2*>(orow + col) = pk;
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nt * BN + wn * 64 + nb * 32 + 8 * q + 4 * fh;
          if (col >= g.N) continue;
          if (MODE == kDown) {
            *reinterpret_cast<float4*>(orow_f + col) =
                make_float4(acc[nb][mb][4 * q], acc[nb][mb][4 * q + 1],
                            acc[nb][mb][4 * q + 2], acc[nb][mb][4 * q + 3]);
          } else {
            float h[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float z = acc[nb][mb][4 * q + v];
              h[v] = z > 0.f ? z : 0.f;
            }
            uint2 pk;
            pk.x = pack_h2(h[0], h[1]);
            pk.y = pack_h2(h[2], h[3]);
            *reinterpret_cast<uint2*>(orow + col) = pk;
          }
        }
      }
    }
  }
}

int ntiles(int mode, int N) {
  const int cols = mode == kSwiGLU ? BN / 2 : BN;
  return (N + cols - 1) / cols;
}

hipError_t launch_one(int mode, bool gather, const GemmArgs& g, int64_t mt_upper,
                      hipStream_t s) {
  int64_t n = mt_upper * g.NT;
  n = (n + 7) / 8 * 8;
  if (n <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(n)), block(kThreads);
  if (mode == kSwiGLU && gather)
    hipLaunchKernelGGL((grouped_gemm_kernel<kSwiGLU, true>), grid, block, 0, s, g);
  else if (mode == kSwiGLU)
    hipLaunchKernelGGL((grouped_gemm_kernel<kSwiGLU, false>), grid, block, 0, s, g);
  else if (mode == kReLU && gather)
    hipLaunchKernelGGL((grouped_gemm_kernel<kReLU, true>), grid, block, 0, s, g);
  else if (mode == kReLU)
    hipLaunchKernelGGL((grouped_gemm_kernel<kReLU, false>), grid, block, 0, s, g);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<kDown, false>), grid, block, 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_shared_bf16(const Dims& D, const void* x,
                              const moe_expert_weights& w, void* Hs, void* Ys,
                              hipStream_t s) {
  const int up_mode = D.swiglu ? kSwiGLU : kReLU;
  const int64_t mt = (D.T + BM - 1) / BM;
  for (int sh = 0; sh < D.S; ++sh) {
    const int64_t wo = static_cast<int64_t>(sh) * D.Fs * D.d;
    GemmArgs g{};
    g.a = static_cast<const uint16_t*>(x);
    g.E = 1;
    g.single_rows = static_cast<int32_t>(D.T);
    g.w0 = static_cast<const uint16_t*>(w.shared_gate) + wo;
    g.w1 = D.swiglu ? static_cast<const uint16_t*>(w.shared_up) + wo : nullptr;
    g.N = D.Fs;
    g.K = D.d;
    g.out = Hs;
    g.ldo = D.Fs;
    g.NT = ntiles(up_mode, D.Fs);
    hipError_t err = launch_one(up_mode, false, g, mt, s);
    if (err != hipSuccess) return err;
    GemmArgs h{};
    h.a = static_cast<const uint16_t*>(Hs);
    h.E = 1;
    h.single_rows = static_cast<int32_t>(D.T);
    h.w0 = static_cast<const uint16_t*>(w.shared_down) + wo;
    h.N = D.d;
    h.K = D.Fs;
    h.out = static_cast<float*>(Ys) + static_cast<int64_t>(sh) * D.T * D.d;
    h.ldo = D.d;
    h.NT = ntiles(kDown, D.d);
    err = launch_one(kDown, false, h, mt, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_ffn_bf16(const Dims& D, const int32_t* offsets,
                           const int32_t* tiles1, const int32_t* tiles2,
                           const int32_t* sorted_token, const void* x,
                           const moe_expert_weights& w, void* H, void* Hs,
                           void* Y, void* Ys, hipStream_t s) {
  const int up_mode = D.swiglu ? kSwiGLU : kReLU;
  // kept rows are at most min(T*k, E*capacity); cap is already <= T*k
  const int64_t nmax = std::min<int64_t>(D.slots, D.cap * D.E);
  {
    GemmArgs g{};
    g.a = static_cast<const uint16_t*>(x);
    g.sorted_token = sorted_token;
    g.offsets = offsets;
    g.tiles = tiles1;
    g.E = D.E;
    g.w0 = static_cast<const uint16_t*>(w.gate);
    g.w1 = D.swiglu ? static_cast<const uint16_t*>(w.up) : nullptr;
    g.N = D.F;
    g.K = D.d;
    g.out = H;
    g.ldo = D.F;
    g.NT = ntiles(up_mode, D.F);
    hipError_t err = launch_one(up_mode, true, g, nmax / BM + D.E, s);
    if (err != hipSuccess) return err;
  }
  {
    GemmArgs g{};
    g.a = static_cast<const uint16_t*>(H);
    g.offsets = offsets;
    g.tiles = tiles2;
    g.E = D.E;
    g.w0 = static_cast<const uint16_t*>(w.down);
    g.N = D.d;
    g.K = D.F;
    g.out = Y;
    g.ldo = D.d;
    g.NT = ntiles(kDown, D.d);
    hipError_t err = launch_one(kDown, false, g, nmax / BM + D.E, s);
    if (err != hipSuccess) return err;
  }
  if (D.S > 0) return launch_shared_bf16(D, x, w, Hs, Ys, s);
  return hipSuccess;
}

}  // namespace moe
