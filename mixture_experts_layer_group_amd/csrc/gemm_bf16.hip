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
//     owns a 128 x 64 sub-tile = 4 x 2 blocks of v_mfma_f32_32x32x16.  The
//     weight tile is the MFMA A operand (rows = output columns) and the
//     activation tile the B operand, so a lane's accumulators hold 4
//     consecutive output columns of one row;
//   * both operands are K-contiguous in HBM (weights are [out, in]) and go
//     straight from HBM to LDS (buffer_load_dwordx4 ... lds, no staging
//     registers) into double-buffered tiles (2 x 64 KiB).  The loads of K
//     step t+1 start right after the barrier that ends step t-1 (half
//     there, half in step t's first sub-step), so the memory pipe is busy
//     across the barrier.  The 16-byte chunks of each 128-byte LDS row are
//     XOR-swizzled (conflict-free for 8- and 16-lane LDS phases); the
//     swizzle is applied on the global side, since a direct load writes LDS
//     at lane*16;
//   * activation rows are gathered on load through sorted_token (no
//     permuted copy of x); rows past the end of a group are given an
//     out-of-range offset, so a ragged tile fetches only its real rows;
//   * SwiGLU: a tile's 256 weight rows are 128 gate rows then the same 128
//     up rows; each wave holds gate and up accumulators of the same
//     (row, column) in the same lanes, so the epilogue fuses silu(g) * u;
//   * ragged groups without a host sync: the grid is an upper bound on the
//     tile count; each workgroup reads the per-expert M-tile prefix written
//     by the dispatch and exits if surplus.  Workgroup ids are remapped so
//     that each of the 8 XCDs (hardware dispatch is round-robin over XCDs)
//     gets a contiguous range of tiles, ordered per expert in groups of 8
//     N-tiles with the expert's M-tiles fastest, so the tiles running
//     together on one XCD share weight and activation lines in its L2;
//   * the down projection may split its reduction in two K halves (more,
//     shorter tiles when the tile count would leave the last round of
//     workgroups mostly idle); the second half goes to a partial buffer.
#include <algorithm>
#include <type_traits>

#include "moe_internal.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = kGemm1BM, BN = 256, BK = 64;
constexpr int kRowBytes = BK * 2;            // 128
constexpr int kTileBytesA = BM * kRowBytes;  // activation tile per stage
constexpr int kTileBytesW = BN * kRowBytes;  // weight tile per stage (32 KiB)
constexpr int kNG = 8;                      // N-tiles per scheduling column group
constexpr int kWaves = 8;                   // 2 waves per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kWavesN = 4;                  // waves along N (2 along M)
constexpr int MB = BM / 64, NB = 2;         // 32x32 blocks per wave: (BM/2) x 64
constexpr int kLoadsA = kTileBytesA / 1024 / kWaves;  // 1 KiB direct loads per wave
constexpr int kLoadsW = kTileBytesW / 1024 / kWaves;
static_assert(BM == kGemm2BM && BM % 64 == 0, "tile prefix BM mismatch");
static_assert(kTileBytesA % (1024 * kWaves) == 0, "whole direct loads per wave");

enum Mode { kSwiGLU = 0, kReLU = 1, kDown = 2 };

struct GemmArgs {
  const uint16_t* a;            // activation rows (x or H)
  uint32_t a_bytes;             // size of the activation buffer in bytes
  const int32_t* sorted_token;  // gather table (nullptr: row = group row)
  const int32_t* offsets;       // [E+1] group row offsets (nullptr: one group)
  const int32_t* tiles;         // [E+1] group M-tile prefix (nullptr: one group)
  int E;
  int32_t single_rows;          // rows of the single group
  const uint16_t* w0;           // gate / in / down of expert 0, [N][K]
  const uint16_t* w1;           // up (SwiGLU) of expert 0
  int64_t wstride;              // elements from one expert's matrix to the
                                // next (N*K; 2*N*K for fused gate/up)
  int N;                        // weight rows per expert
  int K;                        // reduction length (row length of a and w)
  void* out;                    // [rows][ldo]: bf16 H (up), fp32 Y (down)
  float* part;                  // down, second K split: fp32 partial rows
  int ksplit;                   // K splits (1 or 2; 2 only for down)
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

// silu with the hardware reciprocal (about 1 ulp of fp32) instead of an
// IEEE division: H is rounded to fp16 right after, 2^-11 relative, far above
// that error, and the epilogue of a tile runs 64 of these per lane.
// Large negative z: exp overflows to inf, the reciprocal gives 0, silu -> -0.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __expf(-z));
}

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
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (kTileBytesA + kTileBytesW)];
  uint8_t* sA = smem;                    // [2][BM rows][128 B]
  uint8_t* sW = smem + 2 * kTileBytesA;  // [2][BN rows][128 B]

  // ---------------- tile scheduling
  const int total_mt = g.tiles ? g.tiles[g.E] : (g.single_rows + BM - 1) / BM;
  const int real = total_mt * g.NT;
  const int share = (real * g.ksplit + 7) >> 3;
  const int bid = blockIdx.x;
  const int local = bid >> 3;
  if (local >= share) return;
  int L = (bid & 7) * share + local;
  if (L >= real * g.ksplit) return;
  const int split = L / real;  // K split (slowest, so each split's tiles keep their order)
  L -= split * real;
  int e = 0, row0, cnt, mt, nt;
  {
    // expert-major order: per expert, groups of kNG N-tiles; inside a group
    // the expert's M-tiles run fastest, so the workgroups that run together
    // on one XCD share each weight tile and the expert's activation rows
    const int32_t* tp = g.tiles;
    int t0 = 0, t1 = total_mt;
    if (tp) {
      e = largest_le(tp, g.E, L / g.NT);
      t0 = tp[e];
      t1 = tp[e + 1];
    }
    const int mte = t1 - t0;
    const int rem = L - t0 * g.NT;
    const int full = g.NT / kNG;
    const int grp = rem / (mte * kNG);
    if (grp < full) {
      const int r2 = rem - grp * mte * kNG;
      nt = grp * kNG + r2 / mte;
      mt = r2 % mte;
    } else {
      const int r2 = rem - full * mte * kNG;
      nt = full * kNG + r2 / mte;
      mt = r2 % mte;
    }
    if (tp) {
      row0 = g.offsets[e];
      cnt = g.offsets[e + 1] - row0;
    } else {
      row0 = 0;
      cnt = g.single_rows;
    }
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
  // The activation descriptor carries the buffer size: rows past the end
  // of the group get the offset a_bytes, which the buffer range check turns
  // into loads that fetch nothing (the LDS rows they would fill only feed
  // output rows that are never stored).
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(g.a), (short)0, static_cast<int>(g.a_bytes), 0x00020000);
  const uint16_t* wbase0 = g.w0 + static_cast<int64_t>(e) * g.wstride;
  const uint16_t* wbase1 = (MODE == kSwiGLU ? g.w1 : g.w0) + static_cast<int64_t>(e) * g.wstride;
  const __amdgpu_buffer_rsrc_t rsW0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(wbase0), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsW1 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(wbase1), (short)0, -1, 0x00020000);
  uint32_t voffA[kLoadsA], voffW[kLoadsW];
#pragma unroll
  for (int j = 0; j < kLoadsA; ++j) {
    const int r = (j * kWaves + wave) * 8 + (lane >> 3);  // tile row
    const int c = (lane & 7) ^ ((r ^ (r >> 3)) & 7);     // chunk at position lane%8
    const int m = m0 + r;
    if (m < cnt) {
      const int64_t arow = GATHER ? static_cast<int64_t>(g.sorted_token[row0 + m])
                                  : static_cast<int64_t>(row0 + m);
      voffA[j] = static_cast<uint32_t>(arow * K * 2 + c * 16);
    } else {
      voffA[j] = g.a_bytes;  // past the group: out of range, no fetch
    }
  }
#pragma unroll
  for (int j = 0; j < kLoadsW; ++j) {
    const int r = (j * kWaves + wave) * 8 + (lane >> 3);  // tile row
    const int c = (lane & 7) ^ ((r ^ (r >> 3)) & 7);     // chunk at position lane%8
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
  for (int mb = 0; mb < MB; ++mb) arow_l[mb] = wm * (MB * 32) + mb * 32 + fr;

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = g.K / BK / g.ksplit;  // K steps of this split
  const int kbase = split * KT;
  auto issue = [&](int kt, int buf) {
    const int soff = (kbase + kt) * kRowBytes;  // K advance in bytes
    uint8_t* a = sA + buf * kTileBytesA;
    uint8_t* w = sW + buf * kTileBytesW;
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsA, (__attribute__((address_space(3))) void*)(a + (j * kWaves + wave) * 1024), 16,
          voffA[j], soff, 0, 0);
#pragma unroll
    for (int j = 0; j < kLoadsW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          j < kLoadsW / 2 ? rsW0 : rsW1,
          (__attribute__((address_space(3))) void*)(w + (j * kWaves + wave) * 1024), 16,
          voffW[j], soff, 0, 0);
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
    const uint8_t* a = sA + buf * kTileBytesA;
    const uint8_t* w = sW + buf * kTileBytesW;
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
  // the sub-step that issues a K step's direct loads: fragment reads first,
  // then the loads spread evenly over its MFMAs
  auto pace_loads = [&]() {
    constexpr int kV = kLoadsA + kLoadsW;  // direct loads in this sub-step
    constexpr int NM = NB * MB;
    static_assert(kV <= 2 * NM, "load spread");
    __builtin_amdgcn_sched_group_barrier(0x100, NB + MB, 0);  // DS read
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int n_here = ((i + 1) * kV) / NM - (i * kV) / NM;
      if (n_here >= 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM
      if (n_here >= 2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM
      if (MODE == kDown) __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
  };
  // Load pipeline.  The loads of K tile t+1 go into the buffer that tile
  // t-1 used: they are issued right after the barrier that ends tile t-1
  // (that buffer is free from then on), during tile t-1's last MFMAs, so
  // the memory pipe never idles across the barrier and tile t+1 has nearly
  // a whole tile of MFMAs to arrive in.
  auto tile = [&](int kt, auto kind_tag) {
    constexpr int kind = decltype(kind_tag)::value;  // 0 full, 1 no loads, 2 last
    const int cur = kt & 1;
    read_frags(cur, 1, 1);
    mfmas(0);
    convert(1);
    pace();
    read_frags(cur, 2, 0);
    mfmas(1);
    convert(0);
    pace();
    read_frags(cur, 3, 1);
    mfmas(0);
    convert(1);
    pace();
    if constexpr (kind != 2) {
      // every read of this tile is issued: wait for them and for the next
      // tile's loads, publish the next tile, read its first fragments ahead
      // of this tile's last MFMAs, and start the loads of the tile after it
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __syncthreads();
      // down projection: the waves that leave the barrier first issue the
      // next loads and their last sub-step at raised priority (5% faster on
      // the Mixtral-shaped layer; the gate/up product is 1% slower with it)
      if constexpr (MODE == kDown) __builtin_amdgcn_s_setprio(1);
      read_frags(cur ^ 1, 0, 0);
      if constexpr (kind == 0) {
        issue(kt + 2, cur);
        mfmas(1);
        convert(0);
        pace_loads();
        if constexpr (MODE == kDown) __builtin_amdgcn_s_setprio(0);
      } else {
        mfmas(1);
        convert(0);
        pace();
        if constexpr (MODE == kDown) __builtin_amdgcn_s_setprio(0);
      }
    } else {
      mfmas(1);
    }
  };

  issue(0, 0);
  if (KT > 1) issue(1, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  read_frags(0, 0, 0);
  convert(0);
  for (int kt = 0; kt + 2 < KT; ++kt) tile(kt, std::integral_constant<int, 0>{});
  if (KT > 1) tile(KT - 2, std::integral_constant<int, 1>{});
  tile(KT - 1, std::integral_constant<int, 2>{});

  // ---------------- epilogue
  // lane holds, for block (nb, mb) and item v: output column
  //   colbase(nb) + 8*(v/4) + 4*(lane/32) + v%4, row arow_l[mb].
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + arow_l[mb];
    if (m >= cnt) continue;
    const int64_t orow_off = static_cast<int64_t>(row0 + m) * g.ldo;
    uint16_t* orow = static_cast<uint16_t*>(g.out) + orow_off;
    float* orow_f = (split ? g.part : static_cast<float*>(g.out)) + orow_off;
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
  int64_t n = mt_upper * g.NT * g.ksplit;
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

int down_splits(const Dims& D) {
  if (!D.bf16 || D.u4) return 1;
  const int KT = D.F / BK;
  if (KT % 2 != 0 || KT < 16) return 1;
  const int64_t nmax = std::min<int64_t>(D.slots, D.cap * D.E);
  const int64_t t = (nmax / BM + D.E) * ntiles(kDown, D.d);  // tile upper bound
  constexpr int64_t kCUs = 256;
  const int64_t half_rounds1 = (t + kCUs - 1) / kCUs * 2;
  const int64_t half_rounds2 = (2 * t + kCUs - 1) / kCUs;
  return half_rounds2 * 10 < half_rounds1 * 9 ? 2 : 1;
}

hipError_t launch_shared_bf16(const Dims& D, const void* x,
                              const moe_expert_weights& w, void* Hs, void* Ys,
                              hipStream_t s) {
  const int up_mode = D.swiglu ? kSwiGLU : kReLU;
  const int64_t mt = (D.T + BM - 1) / BM;
  const int64_t mat = static_cast<int64_t>(D.Fs) * D.d;  // one [Fs][d] matrix
  for (int sh = 0; sh < D.S; ++sh) {
    const int64_t wo = static_cast<int64_t>(sh) * mat;
    GemmArgs g{};
    g.a = static_cast<const uint16_t*>(x);
    g.a_bytes = static_cast<uint32_t>(D.T * D.d * 2);
    g.E = 1;
    g.single_rows = static_cast<int32_t>(D.T);
    if (D.fused) {  // [S][2Fs][d]: gate rows, then up rows
      g.w0 = static_cast<const uint16_t*>(w.shared_gate) + 2 * wo;
      g.w1 = g.w0 + mat;
    } else {
      g.w0 = static_cast<const uint16_t*>(w.shared_gate) + wo;
      g.w1 = D.swiglu ? static_cast<const uint16_t*>(w.shared_up) + wo : nullptr;
    }
    g.wstride = 0;  // a single expert
    g.N = D.Fs;
    g.K = D.d;
    g.out = Hs;
    g.ldo = D.Fs;
    g.NT = ntiles(up_mode, D.Fs);
    g.ksplit = 1;
    hipError_t err = launch_one(up_mode, false, g, mt, s);
    if (err != hipSuccess) return err;
    GemmArgs h{};
    h.a = static_cast<const uint16_t*>(Hs);
    h.a_bytes = static_cast<uint32_t>(D.T * D.Fs * 2);
    h.E = 1;
    h.single_rows = static_cast<int32_t>(D.T);
    h.w0 = static_cast<const uint16_t*>(w.shared_down) + wo;
    h.wstride = 0;
    h.N = D.d;
    h.K = D.Fs;
    h.out = static_cast<float*>(Ys) + static_cast<int64_t>(sh) * D.T * D.d;
    h.ldo = D.d;
    h.NT = ntiles(kDown, D.d);
    h.ksplit = 1;
    err = launch_one(kDown, false, h, mt, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_ffn_bf16(const Dims& D, const int32_t* offsets,
                           const int32_t* tiles1, const int32_t* tiles2,
                           const int32_t* sorted_token, const void* x,
                           const moe_expert_weights& w, void* H, void* Hs,
                           void* Y, float* Ypart, void* Ys, hipStream_t s) {
  const int up_mode = D.swiglu ? kSwiGLU : kReLU;
  // kept rows are at most min(T*k, E*capacity); cap is already <= T*k
  const int64_t nmax = std::min<int64_t>(D.slots, D.cap * D.E);
  {
    GemmArgs g{};
    g.a = static_cast<const uint16_t*>(x);
    g.a_bytes = static_cast<uint32_t>(D.T * D.d * 2);
    g.sorted_token = sorted_token;
    g.offsets = offsets;
    g.tiles = tiles1;
    g.E = D.E;
    const int64_t mat = static_cast<int64_t>(D.F) * D.d;  // one [F][d] matrix
    g.w0 = static_cast<const uint16_t*>(w.gate);
    if (D.fused) {  // [E][2F][d]: each expert's gate rows, then its up rows
      g.w1 = g.w0 + mat;
      g.wstride = 2 * mat;
    } else {
      g.w1 = D.swiglu ? static_cast<const uint16_t*>(w.up) : nullptr;
      g.wstride = mat;
    }
    g.N = D.F;
    g.K = D.d;
    g.out = H;
    g.ldo = D.F;
    g.NT = ntiles(up_mode, D.F);
    g.ksplit = 1;
    hipError_t err = launch_one(up_mode, true, g, nmax / BM + D.E, s);
    if (err != hipSuccess) return err;
  }
  {
    GemmArgs g{};
    g.a = static_cast<const uint16_t*>(H);
    g.a_bytes = static_cast<uint32_t>(D.slots * D.F * 2);
    g.offsets = offsets;
    g.tiles = tiles2;
    g.E = D.E;
    g.w0 = static_cast<const uint16_t*>(w.down);
    g.wstride = static_cast<int64_t>(D.d) * D.F;
    g.N = D.d;
    g.K = D.F;
    g.out = Y;
    g.ldo = D.d;
    g.NT = ntiles(kDown, D.d);
    g.ksplit = down_splits(D);
    g.part = Ypart;
    if (g.ksplit > 1 && Ypart == nullptr) return hipErrorInvalidValue;
    hipError_t err = launch_one(kDown, false, g, nmax / BM + D.E, s);
    if (err != hipSuccess) return err;
  }
  if (D.S > 0) return launch_shared_bf16(D, x, w, Hs, Ys, s);
  return hipSuccess;
}

}  // namespace moe
