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
//   * a BM x 256 output tile (BM = 256, or 128 for 4-bit layers with few
//     rows per expert) per 512-thread workgroup, K steps of 64; each of the
//     8 waves (2 per SIMD, so one fills the other's issue gaps) owns a
//     BM/2 x 64 sub-tile = BM/64 x 2 blocks of v_mfma_f32_32x32x16.  The
//     weight tile is the MFMA A operand (rows = output columns) and the
//     activation tile the B operand, so a lane's accumulators hold 4
//     consecutive output columns of one row;
//   * both operands are K-contiguous in HBM (weights are [out, in]) and go
//     straight from HBM to LDS (buffer_load_dwordx4 ... lds, no staging
//     registers) into LDS stages: three of each operand where they fit
//     160 KiB, else (256-row bf16 tiles) two activation and three weight
//     stages, so the weights run two K steps ahead.  The loads of a later
//     step start right after the barrier that ends the step whose stage
//     they reuse, so the memory pipe is busy across the barrier.  The 16-byte chunks of each 128-byte LDS row are
//     XOR-swizzled (conflict-free for 8- and 16-lane LDS phases); the
//     swizzle is applied on the global side, since a direct load writes LDS
//     at lane*16;
//   * activation rows are gathered on load through sorted_token (no
//     permuted copy of x); rows past the end of a group are given an
//     out-of-range offset, so a ragged tile fetches only its real rows,
//     and a wave's K loop is compiled per number of its 32-row blocks
//     that hold rows (empty blocks get no fragment reads and no products);
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

constexpr int BN = 256, BK = 64;
constexpr int kRowBytes = BK * 2;            // 128
constexpr int kTileBytesW = BN * kRowBytes;  // weight tile per stage (32 KiB)
constexpr int kNG = 8;                      // N-tiles per scheduling column group
constexpr int kWaves = 8;                   // 2 waves per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kWavesN = 4;                  // waves along N (2 along M)
constexpr int NB = 2;                       // 32x32 weight blocks per wave (64 columns)
constexpr int kLoadsW = kTileBytesW / 1024 / kWaves;  // 1 KiB direct loads per wave
// 4-bit weights, per stage: the codes of the BN weight rows (32 B per row
// per K step of 64), then one dword per row holding its scale, then one
// holding its bias (the dword of the bf16 array that contains this K step's
// group: with an even number of groups per row the pair never crosses a row)
constexpr int kQCodeBytes = BN * 32;
constexpr int kTileBytesQ = kQCodeBytes + BN * 8;
static_assert(kQCodeBytes == kWaves * 1024 && BN == 4 * 64, "one code load per wave, "
              "four 64-row dword loads each for scales and biases");

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
  int32_t* err;                 // MOE_FLAG_H_SATURATED is OR-ed in (or nullptr)
  const float* row_scale;       // down: factor of each output row (nullptr: 1)
  bool y16;                     // down: rows (and K-split parts) stored as fp16
  // 4-bit affine weights (U4 kernels): packed codes [N][K/8] uint32 and bf16
  // scales / biases [N][K/64] of expert 0 (gate / in / down, and up)
  const uint8_t* q0;
  const uint8_t* q1;
  const uint16_t* s0;
  const uint16_t* s1;
  const uint16_t* b0;
  const uint16_t* b1;
  int64_t qstride;              // rows from one expert's matrix to the next
  uint32_t nibble_mask;         // 0x0F0F0F0F, passed in so it stays in a register
};

// byte offset of 16-byte chunk c (0..7) of row r inside a swizzled tile.
// The XOR pattern keeps the 32 rows read by one MFMA fragment load on
// distinct banks whether the LDS serves 8 lanes (32 banks) or 16 lanes (64
// banks) of a 16-byte read per cycle.
__device__ __forceinline__ int swz(int r, int c) {
  return r * kRowBytes + ((c ^ ((r ^ (r >> 3)) & 7)) << 4);
}

// The largest e < E with p[e] <= v, for a non-decreasing p with p[0] <= v,
// searched by the whole wave: each round the lanes read 64 evenly spaced
// entries of the remaining range at once and a ballot keeps the stretch after
// the last one not above v (one round up to 64 experts, two up to 4096),
// where a binary search made one dependent load per halving.
__device__ __forceinline__ int largest_le(const int32_t* __restrict__ p, int E,
                                          int32_t v) {
  const int lane = threadIdx.x & 63;
  int base = 0, span = E;
  while (span > 1) {
    const int step = (span + 63) >> 6;
    const int i = lane * step;
    const bool le = i < span && p[base + i] <= v;
    const int last = 63 - __builtin_clzll(__ballot(le));  // lane 0 always holds
    base += last * step;
    span = min(step, span - last * step);
  }
  return base;
}

// silu with the hardware reciprocal (about 1 ulp of fp32) instead of an
// IEEE division: H is rounded to fp16 right after, 2^-11 relative, far above
// that error, and the epilogue of a tile runs 64 of these per lane.
// Large negative z: exp overflows to inf, the reciprocal gives 0, silu -> -0.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __expf(-z));
}

// hidden activation -> fp16, round to nearest even, saturating at +-65504;
// `sat` records a value outside that range (or NaN, which the clamp turns
// into -65504)
__device__ __forceinline__ uint32_t pack_h2(float a, float b, bool& sat) {
  sat |= !(fabsf(a) <= 65504.f) || !(fabsf(b) <= 65504.f);
  a = fminf(fmaxf(a, -65504.f), 65504.f);
  b = fminf(fmaxf(b, -65504.f), 65504.f);
  const _Float16 ha = static_cast<_Float16>(a), hb = static_cast<_Float16>(b);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ha)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hb)) << 16);
}

// 8 bf16 weights -> 8 fp16, rounded to nearest (v_cvt_pk_f16_f32, one
// instruction per pair): exact for magnitudes from 2^-17 (where fp16's
// subnormal grid still holds bf16's 8 significant bits) up to 65504; smaller
// ones land on the nearest multiple of 2^-24, larger ones become +-inf
__device__ __forceinline__ half8 bf16x8_to_f16x8(bf16x8 v) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const uint4 u = __builtin_bit_cast(uint4, v);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f2 f = {__uint_as_float(w[j] << 16), __uint_as_float(w[j] & 0xffff0000u)};
    o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, h2));
  }
  return __builtin_bit_cast(half8, make_uint4(o[0], o[1], o[2], o[3]));
}

// 8 codes of one packed word (element i in nibble i) -> 8 weights s*q + b,
// formed in fp32 (exact for the 4-bit codes) and rounded once to the MFMA
// operand type (fp16 for the 4-bit products).  `mask` is 0x0F0F0F0F held in
// a register, so the nibble pairs become the bytes that v_cvt_f32_ubyte0..3
// read.
template <bool F16>
__device__ __forceinline__ uint4 dequant8(uint32_t w, float sc, float bi, uint32_t mask) {
  const uint32_t lo = w & mask;         // codes 0, 2, 4, 6 in bytes 0..3
  const uint32_t hi = (w >> 4) & mask;  // codes 1, 3, 5, 7
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = fmaf(sc, static_cast<float>((lo >> (8 * j)) & 0xffu), bi);
    v[2 * j + 1] = fmaf(sc, static_cast<float>((hi >> (8 * j)) & 0xffu), bi);
  }
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (F16) {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      const h2 p = {static_cast<_Float16>(v[2 * j]), static_cast<_Float16>(v[2 * j + 1])};
      o[j] = __builtin_bit_cast(uint32_t, p);
    } else {
      typedef __bf16 b2 __attribute__((ext_vector_type(2)));
      const b2 p = {static_cast<__bf16>(v[2 * j]), static_cast<__bf16>(v[2 * j + 1])};
      o[j] = __builtin_bit_cast(uint32_t, p);
    }
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Which tile a workgroup computes.  The grid is an upper bound on the tile
// count (ragged groups, no host sync): a workgroup reads the per-expert
// M-tile prefix that the dispatch wrote and returns false if surplus.
// Workgroup ids are remapped so each of the 8 XCDs (hardware dispatch is
// round-robin over XCDs) gets a contiguous range of tiles, in expert-major
// order: per expert, groups of kNG N-tiles; inside a group the expert's
// M-tiles run fastest, so the workgroups that run together on one XCD share
// each weight tile and the expert's activation rows.  For ragged groups the
// ranges are cut at equal estimated cost (XcdPlan; the dispatch wrote the
// boundaries after the M-tile prefix), for one group at equal count.
struct TileSched {
  int e, row0, cnt, mt, nt, split;
};

// One tile of the last quarters of the XCD ranges, claimed by thread 0 of a
// workgroup of XCD x: from the front of x's own quarter (own), else from
// the back of another XCD's (see XcdPlan); -1 when none is left.  Relaxed
// device-scope atomics: the counters only hand out distinct tiles.  A
// counter is read before it is incremented, so workgroups that come late
// do not queue increments on counters that are spent.
__device__ int claim_tile(const int32_t* xb, unsigned long long* claims, int x, bool own) {
  for (int j = own ? 0 : 1; j < (own ? 1 : kXcds); ++j) {
    const int y = (x + j) & (kXcds - 1);
    const int hi = xb[y + 1];
    const int q = (hi - xb[y]) >> 2;
    if (q <= 0) continue;
    unsigned long long* c = claims + kClaimStride / 2 * y;
    const unsigned long long now = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (static_cast<int>(now & 0xffffffffull) + static_cast<int>(now >> 32) >= q) continue;
    const unsigned long long old = __hip_atomic_fetch_add(
        c, own ? 1ull : 1ull << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int front = static_cast<int>(old & 0xffffffffull);
    const int back = static_cast<int>(old >> 32);
    if (front + back < q) return own ? hi - q + front : hi - 1 - back;
  }
  return -1;
}

__device__ __forceinline__ bool schedule_tile(const GemmArgs& g, int bm, TileSched& t,
                                              int* lds_word) {
  const int total_mt = g.tiles ? g.tiles[g.E] : (g.single_rows + bm - 1) / bm;
  const int real = total_mt * g.NT;
  const int bid = blockIdx.x;
  const int local = bid >> 3;
  int L;
  if (g.tiles) {
    // the XCD's range of equal estimated cost, written after the prefix; its
    // last quarter is claimed at run time (shared with the other XCDs)
    const int32_t* xb = g.tiles + g.E + 1;
    const int start = xb[bid & 7];
    const int size = xb[(bid & 7) + 1] - start;
    if (local < size - (size >> 2)) {
      L = start + local;
    } else {
      // the quarter's own claims, then at most kStealers claims elsewhere
      if (local >= size + kStealers) return false;
      if (threadIdx.x == 0)
        *lds_word = claim_tile(xb, reinterpret_cast<unsigned long long*>(
                                       const_cast<int32_t*>(g.tiles) + tile_claims_at(g.E)),
                               bid & 7, local < size);
      __syncthreads();
      L = *lds_word;
      __syncthreads();  // the word is LDS that the tile's loads reuse
      if (L < 0) return false;
    }
  } else {
    const int share = (real * g.ksplit + 7) >> 3;
    if (local >= share) return false;
    L = (bid & 7) * share + local;
  }
  if (L >= real * g.ksplit) return false;
  t.split = L / real;  // K split (slowest, so each split's tiles keep their order)
  L -= t.split * real;
  t.e = 0;
  const int32_t* tp = g.tiles;
  int t0 = 0, t1 = total_mt;
  if (tp) {
    t.e = largest_le(tp, g.E, L / g.NT);
    t0 = tp[t.e];
    t1 = tp[t.e + 1];
  }
  const int mte = t1 - t0;
  const int rem = L - t0 * g.NT;
  const int full = g.NT / kNG;
  const int grp = rem / (mte * kNG);
  const int r2 = rem - (grp < full ? grp : full) * mte * kNG;
  t.nt = (grp < full ? grp : full) * kNG + r2 / mte;
  t.mt = r2 % mte;
  if (tp) {
    t.row0 = g.offsets[t.e];
    t.cnt = g.offsets[t.e + 1] - t.row0;
  } else {
    t.row0 = 0;
    t.cnt = g.single_rows;
  }
  return true;
}

// the largest per-variant counts, for array sizes: arrays sized by a
// template-dependent count and captured by the kernel's lambdas lose the
// kernel's host-side launch stub
constexpr int kMaxMB = 4, kMaxLoadsA = 4;

// Sizes of one kernel variant: BMT-row tiles, bf16 or 4-bit weights, and
// its LDS stages.
template <int BMT, bool U4>
struct TileCfg {
  static constexpr int BM = BMT;                          // tile rows (activation rows)
  static constexpr int kTileBytesA = BM * kRowBytes;      // activation tile per stage
  static constexpr int MB = BM / 64;                      // 32x32 blocks per wave along M
  static constexpr int kLoadsA = kTileBytesA / 1024 / kWaves;  // 1 KiB direct loads per wave
  static constexpr int kWBytes = U4 ? kTileBytesQ : kTileBytesW;  // weight stage
  static constexpr int NST = (kTileBytesA + kWBytes) * 3 <= 160 * 1024 ? 3 : 2;
  // LDS stages of the activation and of the weight tiles: NST each, except
  // where three stages of both do not fit and a third weight stage does
  // (256-row bf16 tiles: 2 x 32 KiB + 3 x 32 KiB = 160 KiB), which puts the
  // weights -- streamed from HBM -- two steps ahead and the activations,
  // mostly served by the caches, one
  static constexpr int NSA = NST;
  static constexpr int NSW =
      NST == 2 && 2 * kTileBytesA + 3 * kWBytes <= 160 * 1024 ? 3 : NST;
  static constexpr int kLoadsWStep = U4 ? 2 : kLoadsW;
  // direct loads per K step and wave (vmcnt counts them in issue order)
  static constexpr int kStepLoads = kLoadsA + kLoadsWStep;
  static_assert(BM % 128 == 0 && kTileBytesA % (1024 * kWaves) == 0, "whole direct loads");
  static_assert(MB <= kMaxMB && kLoadsA <= kMaxLoadsA, "array bounds");
};

template <int MODE, bool GATHER, bool U4, int BMT>
__global__ void __launch_bounds__(kThreads, 1)
grouped_gemm_kernel(GemmArgs g) {
  using TC = TileCfg<BMT, U4>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[TC::NSA * TC::kTileBytesA + TC::NSW * TC::kWBytes];
  uint8_t* sA = smem;                              // [NSA][BM rows][128 B]
  uint8_t* sW = smem + TC::NSA * TC::kTileBytesA;  // [NSW][BN rows][128 B]; 4-bit: codes, scales, biases

  // ---------------- tile scheduling
  TileSched ts;
  if (!schedule_tile(g, TC::BM, ts, reinterpret_cast<int*>(smem))) return;
  const int e = ts.e, row0 = ts.row0, mt = ts.mt, nt = ts.nt, split = ts.split;
  // The group's rows spread evenly over its M tiles, in 32-row blocks (the
  // tile count stays ceil(rows / BM)): tiles that share a weight column then
  // step through K at the same pace and meet in the L2, where a full tile
  // beside a nearly empty one ran ahead of it and the weights were fetched
  // twice.  cnt is this tile's end inside the group.
  const int mte = (ts.cnt + TC::BM - 1) / TC::BM;
  const int tr = mte > 0 ? min(TC::BM, ((ts.cnt + mte - 1) / mte + 31) / 32 * 32) : TC::BM;
  const int m0 = mt * tr;  // first row of this tile inside the group
  const int cnt = min(ts.cnt, m0 + tr);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform to the compiler: descriptors and LDS addresses derived
  // from it stay in scalar registers (no per-lane waterfall loops)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  uint32_t voffA[kMaxLoadsA], voffW[kLoadsW];  // the first TC::kLoadsA used
#pragma unroll
  for (int j = 0; j < TC::kLoadsA; ++j) {
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
  // 4-bit weights: wave w loads the codes of tile rows 32w..32w+31 (lane l:
  // row 32w + l/2, bytes 16*(l%2).. of the row's 32 per K step), then a
  // quarter of the scales (waves 0-3) or biases (waves 4-7): 64 rows, one
  // dword each.  Every descriptor carries its matrix's exact size.
  const int64_t G = K / 64;  // groups per row (even)
  auto tile_row_n = [&](int r) {
    int n = (MODE == kSwiGLU) ? nt * (BN / 2) + (r & 127) : nt * BN + r;
    return n > g.N - 1 ? g.N - 1 : n;
  };
  const uint8_t* qptr = nullptr;
  const uint16_t* sbptr = nullptr;
  int qbytes = 0, sbbytes = 0;
  uint32_t voffQ = 0, voffSB = 0;
  if constexpr (U4) {
    const int64_t erow = static_cast<int64_t>(e) * g.qstride;  // expert's first row
    const int rq = wave * 32 + (lane >> 1);
    const bool up_q = MODE == kSwiGLU && wave >= 4;  // rq >= 128
    qptr = (up_q ? g.q1 : g.q0) + erow * (K / 2);
    qbytes = static_cast<int>(static_cast<int64_t>(g.N) * (K / 2));
    voffQ = static_cast<uint32_t>(static_cast<int64_t>(tile_row_n(rq)) * (K / 2) +
                                  (lane & 1) * 16);
    const int rs = (wave & 3) * 64 + lane;
    const bool up_s = MODE == kSwiGLU && (wave & 3) >= 2;  // rs >= 128
    sbptr = (wave < 4 ? (up_s ? g.s1 : g.s0) : (up_s ? g.b1 : g.b0)) + erow * G;
    sbbytes = static_cast<int>(static_cast<int64_t>(g.N) * G * 2);
    voffSB = static_cast<uint32_t>(static_cast<int64_t>(tile_row_n(rs)) * G * 2);
  }
  const __amdgpu_buffer_rsrc_t rsQ = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(qptr), (short)0, qbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsSB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(sbptr), (short)0, sbbytes, 0x00020000);

  // ---------------- per-lane fragment offsets
  // MFMA 32x32x16: lane l supplies row (l % 32), K elements 8*(l/32)..+8.
  // A wave owns 128 activation rows (4 blocks) and 64 weight rows (2
  // blocks); for SwiGLU those are 32 gate rows and the matching 32 up rows.
  const int fr = lane & 31;
  const int fh = lane >> 5;
  int wrow[NB], arow_l[kMaxMB];  // the first TC::MB used
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (MODE == kSwiGLU)
      wrow[nb] = (nb ? 128 : 0) + wn * 32 + fr;
    else
      wrow[nb] = wn * 64 + nb * 32 + fr;
  }
#pragma unroll
  for (int mb = 0; mb < TC::MB; ++mb) arow_l[mb] = wm * (TC::MB * 32) + mb * 32 + fr;

  f32x16 acc[NB][kMaxMB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < TC::MB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = g.K / BK / g.ksplit;  // K steps of this split
  const int kbase = split * KT;
  // the direct loads of K step kt: activations into stage kt % NSA,
  // weights into stage kt % NSW
  auto issue_a = [&](int kt) {
    const int soff = (kbase + kt) * kRowBytes;  // K advance in bytes
    uint8_t* a = sA + (kt % TC::NSA) * TC::kTileBytesA;
#pragma unroll
    for (int j = 0; j < TC::kLoadsA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsA, (__attribute__((address_space(3))) void*)(a + (j * kWaves + wave) * 1024), 16,
          voffA[j], soff, 0, 0);
  };
  auto issue_w = [&](int kt) {
    const int soff = (kbase + kt) * kRowBytes;  // K advance in bytes
    uint8_t* w = sW + (kt % TC::NSW) * TC::kWBytes;
    if constexpr (U4) {
      const int step = kbase + kt;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsQ, (__attribute__((address_space(3))) void*)(w + wave * 1024), 16, voffQ,
          step * 32, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsSB,
          (__attribute__((address_space(3))) void*)(w + kQCodeBytes + (wave >> 2) * (BN * 4) +
                                                    (wave & 3) * 256),
          4, voffSB, (step >> 1) * 4, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < kLoadsW; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            j < kLoadsW / 2 ? rsW0 : rsW1,
            (__attribute__((address_space(3))) void*)(w + (j * kWaves + wave) * 1024), 16,
            voffW[j], soff, 0, 0);
    }
  };

  // fragments are double-buffered in registers: the LDS reads for K
  // sub-step s+1 are in flight while the MFMAs of sub-step s run.  The next
  // K tile's first fragments are read right after the barrier that
  // publishes it, ahead of the current tile's last MFMAs.  On the fp16 path
  // the weight fragments are read raw (bf16) and converted later in the
  // sub-step, so no conversion waits on its LDS read.
  // fp16 operands for the down product and for every 4-bit product (the
  // activations of the 4-bit gate/up product are converted to fp16 before
  // it; dequantised weights then keep 11 bits instead of bf16's 8)
  constexpr bool kF16 = MODE == kDown || U4;
  using frag_t = typename std::conditional<kF16, half8, bf16x8>::type;
  frag_t wf[2][NB], af[2][kMaxMB];
  bf16x8 wraw[2][NB];
  // 4-bit weights: a lane's codes for the whole K step (4 words: K chunks
  // 4*fh .. 4*fh+3 of its row), and the step's scale and bias of its rows.
  // The K chunks of a step are taken in the order (sub-step ks, lane half
  // fh) -> chunk 4*fh + ks on both operands (instead of 2*ks + fh): the same
  // permutation of the reduction on both sides, so the product is
  // unchanged, and each lane's codes are one 16-byte LDS read.
  uint4 qw[NB];
  float qs[NB], qb[NB];
  // A wave's K loop is specialised to MBA, the number of its activation
  // blocks that hold rows of the group (the wave's share of the tile's
  // rows, in 32-row blocks): in a ragged last tile the empty blocks get no
  // fragment reads and no products, so their SIMD's matrix core takes the
  // other wave's products sooner.  Every wave still issues its share of the
  // direct loads and meets every barrier.
  auto run = [&](auto mba_tag) {
  constexpr int MBA = decltype(mba_tag)::value;
  constexpr bool kFull = MBA == TC::MB;
  // K step `step` (activations in stage sa, weights in stage sw)
  auto read_frags = [&](int sa, int sw, int step, int ks, int fb) {
    if constexpr (MBA == 0) return;
    const uint8_t* a = sA + sa * TC::kTileBytesA;
    const uint8_t* w = sW + sw * TC::kWBytes;
    const int ch = U4 ? fh * 4 + ks : ks * 2 + fh;
    if constexpr (U4) {
      if (ks == 0) {
        // the K step's parity selects the bf16 half of the scale / bias
        // dword
        const int hi = (kbase + step) & 1;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          qw[nb] = *reinterpret_cast<const uint4*>(w + wrow[nb] * 32 + fh * 16);
          const uint32_t sv = *reinterpret_cast<const uint32_t*>(w + kQCodeBytes + wrow[nb] * 4);
          const uint32_t bv =
              *reinterpret_cast<const uint32_t*>(w + kQCodeBytes + BN * 4 + wrow[nb] * 4);
          qs[nb] = __uint_as_float(hi ? (sv & 0xffff0000u) : (sv << 16));
          qb[nb] = __uint_as_float(hi ? (bv & 0xffff0000u) : (bv << 16));
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (MODE == kDown)
          wraw[fb][nb] = *reinterpret_cast<const bf16x8*>(w + swz(wrow[nb], ch));
        else
          wf[fb][nb] = *reinterpret_cast<const bf16x8*>(w + swz(wrow[nb], ch));
      }
    }
#pragma unroll
    for (int mb = 0; mb < MBA; ++mb)
      af[fb][mb] = *reinterpret_cast<const frag_t*>(a + swz(arow_l[mb], ch));
  };
  auto convert = [&](int fb, int ks) {
    if constexpr (MBA == 0) return;
    if constexpr (U4) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t word = ks == 0 ? qw[nb].x : ks == 1 ? qw[nb].y : ks == 2 ? qw[nb].z : qw[nb].w;
        wf[fb][nb] = __builtin_bit_cast(frag_t, dequant8<true>(word, qs[nb], qb[nb], g.nibble_mask));
      }
    } else if constexpr (MODE == kDown) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wf[fb][nb] = bf16x8_to_f16x8(wraw[fb][nb]);
    }
  };
  auto mfmas = [&](int fb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MBA; ++mb) {
        if constexpr (kF16)
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
  // 4-bit weights: the dequantisation (about 23 VALU ops per fragment, 2
  // fragments per sub-step) is spread evenly over the sub-step's MFMAs.
  // A wave with empty blocks (MBA < MB) runs short of products to pace
  // against and is left to the compiler's schedule.
  constexpr int kDeqValu = 6;
  auto pace = [&]() {
    if constexpr (!kFull) return;
    if constexpr (U4) {
#pragma unroll
      for (int i = 0; i < NB * TC::MB; ++i) {
        if (i < TC::MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, kDeqValu, 0);      // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // MFMA
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NB + TC::MB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
#pragma unroll
    for (int i = NB + TC::MB; i < NB * TC::MB; ++i) {
      if (MODE == kDown) __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
  };
  // the sub-step that issues a K step's direct loads: fragment reads first,
  // then the loads spread evenly over its MFMAs
  auto pace_loads = [&]() {
    if constexpr (!kFull) return;
    constexpr int kV = TC::kLoadsA + (U4 ? 2 : kLoadsW);  // direct loads in this sub-step
    constexpr int NM = NB * TC::MB;
    static_assert(kV <= 2 * NM, "load spread");
    __builtin_amdgcn_sched_group_barrier(0x100, U4 ? TC::MB + 3 * NB : NB + TC::MB, 0);  // DS read
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int n_here = ((i + 1) * kV) / NM - (i * kV) / NM;
      if (n_here >= 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM
      if (n_here >= 2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM
      if (U4) __builtin_amdgcn_sched_group_barrier(0x002, kDeqValu, 0);     // VALU
      else if (MODE == kDown) __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
  };
  // Load pipeline: K step t's activations live in stage t % NSA, its
  // weights in stage t % NSW (NSA <= NSW).  Right after the barrier that
  // ends step t-1 (from then on both of its stages are free) a wave issues
  // the activations of step t-1+NSA, then the weights of step t-1+NSW,
  // during step t-1's last MFMAs, so the memory pipe never idles across a
  // barrier.  The prologue issues steps 0.. in the same order (activations
  // before weights within a step).  Before the barrier that publishes step
  // t+1, a wave waits until only the loads issued after step t+1's are
  // pending: those of step t+2 (NSA = NSW = 3), or the weights of step t+2
  // (NSA = 2, NSW = 3); vector-memory loads retire in issue order.
  constexpr int kLaterLoads = TC::NSW == 3 ? (TC::NSA == 3 ? TC::kStepLoads : TC::kLoadsWStep) : 0;
  auto wait_publish = [&](bool later_in_flight) {
    if (kLaterLoads > 0 && later_in_flight)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kLaterLoads) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  };
  auto tile = [&](int kt, auto kind_tag) {
    // 0 issues both operands' loads, 3 the activations' only, 1 none, 2 last
    constexpr int kind = decltype(kind_tag)::value;
    const int ca = kt % TC::NSA, cw = TC::NSA == TC::NSW ? ca : kt % TC::NSW;
    read_frags(ca, cw, kt, 1, 1);
    mfmas(0);
    convert(1, 1);
    pace();
    read_frags(ca, cw, kt, 2, 0);
    mfmas(1);
    convert(0, 2);
    pace();
    read_frags(ca, cw, kt, 3, 1);
    mfmas(0);
    convert(1, 3);
    pace();
    if constexpr (kind != 2) {
      // every read of this step is issued: wait for them and for the next
      // step's loads, publish the next step, read its first fragments ahead
      // of this step's last MFMAs, and start the loads of later steps
      wait_publish(kt + 2 < KT);
      __syncthreads();
      // down projection: the waves that leave the barrier first issue the
      // next loads and their last sub-step at raised priority (5% faster on
      // the Mixtral-shaped layer; the gate/up product is 1% slower with it)
      if constexpr (MODE == kDown) __builtin_amdgcn_s_setprio(1);
      const int na = (kt + 1) % TC::NSA;
      read_frags(na, TC::NSA == TC::NSW ? na : (kt + 1) % TC::NSW, kt + 1, 0, 0);
      if constexpr (kind == 0) {
        issue_a(kt + TC::NSA);
        issue_w(kt + TC::NSW);
        mfmas(1);
        convert(0, 0);
        pace_loads();
      } else {
        if constexpr (kind == 3) issue_a(kt + TC::NSA);
        mfmas(1);
        convert(0, 0);
        pace();
      }
      if constexpr (MODE == kDown) __builtin_amdgcn_s_setprio(0);
    } else {
      mfmas(1);
    }
  };

  issue_a(0);
  issue_w(0);
  if (KT > 1) {
    issue_a(1);
    issue_w(1);
  }
  if (KT > 2) {
    if constexpr (TC::NSA > 2) issue_a(2);
    if constexpr (TC::NSW > 2) issue_w(2);
  }
  // step 0's loads: the later prologue steps' may stay in flight
  constexpr int kPro2 = (TC::NSA > 2 ? TC::kLoadsA : 0) + (TC::NSW > 2 ? TC::kLoadsWStep : 0);
  if (kPro2 > 0 && KT > 2)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(TC::kStepLoads + kPro2) : "memory");
  else if (KT > 1)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(TC::kStepLoads) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  read_frags(0, 0, 0, 0, 0);
  convert(0, 0);
  int kt = 0;
  for (; kt + TC::NSW < KT; ++kt) tile(kt, std::integral_constant<int, 0>{});
  if constexpr (TC::NSA < TC::NSW)
    for (; kt + TC::NSA < KT; ++kt) tile(kt, std::integral_constant<int, 3>{});
  for (; kt + 1 < KT; ++kt) tile(kt, std::integral_constant<int, 1>{});
  tile(KT - 1, std::integral_constant<int, 2>{});

  };
  // this wave's rows of the tile, in 32-row blocks
  const int wave_rows = cnt - m0 - wm * (TC::MB * 32);
  const int mba = wave_rows <= 0 ? 0 : (wave_rows + 31) / 32;
  if (mba >= TC::MB) {
    run(std::integral_constant<int, TC::MB>{});
  } else if (mba == 0) {
    run(std::integral_constant<int, 0>{});
  } else if constexpr (TC::MB == 4) {
    if (mba == 1)
      run(std::integral_constant<int, 1>{});
    else if (mba == 2)
      run(std::integral_constant<int, 2>{});
    else
      run(std::integral_constant<int, 3>{});
  } else {
    static_assert(TC::MB == 2, "tile rows");
    run(std::integral_constant<int, 1>{});
  }

  // ---------------- epilogue
  // lane holds, for block (nb, mb) and item v: output column
  //   colbase(nb) + 8*(v/4) + 4*(lane/32) + v%4, row arow_l[mb].
  bool sat = false;
  // fp16 outputs go through LDS, free once every wave has left the K loop:
  // each wave puts its 4-column pieces there, then the workgroup copies
  // whole rows out in 16-byte pieces, eight to a 128-byte line.  Stored
  // directly, the MFMA layout puts 16 bytes into each of 32 rows per store
  // instruction.  fp32 rows (the stage API's) keep the direct stores.
  constexpr int kCols = MODE == kSwiGLU ? BN / 2 : BN;  // output columns of a tile
  constexpr int kStRow = kCols * 2 + 16;                 // staged row, padded
  constexpr bool kStageFits =
      TC::BM * kStRow <= TC::NSA * TC::kTileBytesA + TC::NSW * TC::kWBytes;
  if (kStageFits && (MODE != kDown || g.y16) && g.ldo % 8 == 0 && g.N % 8 == 0) {
    __syncthreads();  // the K loop's last LDS reads are done in every wave
#pragma unroll
    for (int mb = 0; mb < TC::MB; ++mb) {
      const int r = arow_l[mb];
      if (m0 + r >= cnt) continue;
      uint8_t* srow = smem + r * kStRow;
      const float rsc =
          MODE == kDown && g.row_scale != nullptr ? g.row_scale[row0 + m0 + r] : 1.f;
      if (MODE == kSwiGLU) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float h[4];
#pragma unroll
          for (int v = 0; v < 4; ++v)
            h[v] = silu(acc[0][mb][4 * q + v]) * acc[1][mb][4 * q + v];
          uint2 pk;
          pk.x = pack_h2(h[0], h[1], sat);
          pk.y = pack_h2(h[2], h[3], sat);
          *reinterpret_cast<uint2*>(srow + 2 * (wn * 32 + 8 * q + 4 * fh)) = pk;
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float h[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float z = acc[nb][mb][4 * q + v];
              h[v] = MODE == kDown ? (g.row_scale != nullptr ? z * rsc : z) : (z > 0.f ? z : 0.f);
            }
            uint2 pk;
            pk.x = pack_h2(h[0], h[1], sat);
            pk.y = pack_h2(h[2], h[3], sat);
            *reinterpret_cast<uint2*>(srow + 2 * (wn * 64 + nb * 32 + 8 * q + 4 * fh)) = pk;
          }
        }
      }
    }
    __syncthreads();
    const int rows = min(TC::BM, cnt - m0);
    const int col0 = MODE == kSwiGLU ? nt * (BN / 2) : nt * BN;
    const int ncol = min(kCols, g.N - col0);
    constexpr int kPieces = kCols / 8;  // 16-byte pieces of a staged row
    uint16_t* obase = static_cast<uint16_t*>(
        MODE == kDown && split ? static_cast<void*>(g.part) : g.out);
    for (int i = tid; i < rows * kPieces; i += kThreads) {
      const int r = i / kPieces, c = (i - r * kPieces) * 8;
      if (c >= ncol) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(smem + r * kStRow + 2 * c);
      *reinterpret_cast<uint4*>(obase + static_cast<int64_t>(row0 + m0 + r) * g.ldo + col0 + c) = v;
    }
  } else {
  #pragma unroll
    for (int mb = 0; mb < TC::MB; ++mb) {
      const int m = m0 + arow_l[mb];
      if (m >= cnt) continue;
      const int64_t orow_off = static_cast<int64_t>(row0 + m) * g.ldo;
      uint16_t* orow = static_cast<uint16_t*>(g.out) + orow_off;
      float* orow_f = (split ? g.part : static_cast<float*>(g.out)) + orow_off;
      // the routing weight of the row, when the caller asks for weighted rows
      // (each K split is scaled; the splits add up to the scaled row)
      const float rsc = MODE == kDown && g.row_scale != nullptr ? g.row_scale[row0 + m] : 1.f;
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
          pk.x = pack_h2(h[0], h[1], sat);
          pk.y = pack_h2(h[2], h[3], sat);
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
              float4 o = make_float4(acc[nb][mb][4 * q], acc[nb][mb][4 * q + 1],
                                     acc[nb][mb][4 * q + 2], acc[nb][mb][4 * q + 3]);
              if (g.row_scale != nullptr) {
                o.x *= rsc;
                o.y *= rsc;
                o.z *= rsc;
                o.w *= rsc;
              }
              if (g.y16) {  // fp16 rows inside the layer (saturating, reported)
                uint16_t* orow_h =
                    reinterpret_cast<uint16_t*>(split ? static_cast<void*>(g.part) : g.out) +
                    orow_off;
                uint2 pk;
                pk.x = pack_h2(o.x, o.y, sat);
                pk.y = pack_h2(o.z, o.w, sat);
                *reinterpret_cast<uint2*>(orow_h + col) = pk;
              } else {
                *reinterpret_cast<float4*>(orow_f + col) = o;
              }
            } else {
              float h[4];
  #pragma unroll
              for (int v = 0; v < 4; ++v) {
                const float z = acc[nb][mb][4 * q + v];
                h[v] = z > 0.f ? z : 0.f;
              }
              uint2 pk;
              pk.x = pack_h2(h[0], h[1], sat);
              pk.y = pack_h2(h[2], h[3], sat);
              *reinterpret_cast<uint2*>(orow + col) = pk;
            }
          }
        }
      }
    }
  }
  if (g.err != nullptr && __ballot(sat) != 0 && lane == 0)
    atomicOr(g.err, MODE == kDown ? MOE_FLAG_Y_SATURATED : MOE_FLAG_H_SATURATED);
}

// bf16 activations -> fp16 for the 4-bit products, 8 per thread: exact
// for every value of fp16's normal range; beyond +-65504 saturated (and
// reported), below it rounded to fp16's subnormal grid (2^-24 apart)
__global__ void __launch_bounds__(256)
to_f16_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int64_t n8,
              int32_t* __restrict__ err) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  bool sat = false;
  if (i < n8) {
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = __uint_as_float(w[j] << 16), b = __uint_as_float(w[j] & 0xffff0000u);
      sat |= !(fabsf(a) <= 65504.f) || !(fabsf(b) <= 65504.f);
      a = fminf(fmaxf(a, -65504.f), 65504.f);
      b = fminf(fmaxf(b, -65504.f), 65504.f);
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      const h2 p = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
      o[j] = __builtin_bit_cast(uint32_t, p);
    }
    reinterpret_cast<uint4*>(y)[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (err != nullptr && __ballot(sat) != 0 && (threadIdx.x & 63) == 0)
    atomicOr(err, MOE_FLAG_X_SATURATED);
}

int ntiles(int mode, int N) {
  const int cols = mode == kSwiGLU ? BN / 2 : BN;
  return (N + cols - 1) / cols;
}

template <int BMT>
hipError_t launch_bm(int mode, bool gather, bool u4, const GemmArgs& g, dim3 grid,
                     hipStream_t s) {
  const dim3 block(kThreads);
  if (u4) {
    // routed experts only: the gate/up product gathers, the down one does not
    if (g.ksplit != 1) return hipErrorInvalidValue;
    if (mode == kSwiGLU && gather)
      hipLaunchKernelGGL((grouped_gemm_kernel<kSwiGLU, true, true, BMT>), grid, block, 0, s, g);
    else if (mode == kReLU && gather)
      hipLaunchKernelGGL((grouped_gemm_kernel<kReLU, true, true, BMT>), grid, block, 0, s, g);
    else if (mode == kDown && !gather)
      hipLaunchKernelGGL((grouped_gemm_kernel<kDown, false, true, BMT>), grid, block, 0, s, g);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (mode == kSwiGLU && gather)
    hipLaunchKernelGGL((grouped_gemm_kernel<kSwiGLU, true, false, BMT>), grid, block, 0, s, g);
  else if (mode == kSwiGLU)
    hipLaunchKernelGGL((grouped_gemm_kernel<kSwiGLU, false, false, BMT>), grid, block, 0, s, g);
  else if (mode == kReLU && gather)
    hipLaunchKernelGGL((grouped_gemm_kernel<kReLU, true, false, BMT>), grid, block, 0, s, g);
  else if (mode == kReLU)
    hipLaunchKernelGGL((grouped_gemm_kernel<kReLU, false, false, BMT>), grid, block, 0, s, g);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<kDown, false, false, BMT>), grid, block, 0, s, g);
  return hipGetLastError();
}

// Workgroups of a routed (ragged) launch: rows_upper, an upper bound on the
// kept rows, fills rows_upper / bm M tiles plus at most one partial tile per
// expert; rounded to whole XCD rounds.  The XCD ranges written by the
// dispatch hold at most an eighth of these each.
int64_t routed_grid(int64_t rows_upper, int bm, int E, int NT, int ksplit) {
  const int64_t n = (rows_upper / bm + E) * NT * ksplit;
  return (n + kXcds - 1) / kXcds * kXcds;
}

// rows_upper: an upper bound on the group's rows (single group) or on the
// kept rows (grouped)
hipError_t launch_one(int mode, bool gather, const GemmArgs& g, int64_t rows_upper, int bm,
                      hipStream_t s, bool u4 = false) {
  int64_t n = g.tiles ? routed_grid(rows_upper, bm, g.E, g.NT, g.ksplit)
                      : ((rows_upper + bm - 1) / bm * g.NT * g.ksplit + 7) / 8 * 8;
  if (n <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(n));
  if (bm == 128) return launch_bm<128>(mode, gather, u4, g, grid, s);
  if (bm == 256) return launch_bm<256>(mode, gather, u4, g, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace

int routed_bm(const Dims& D) {
  if (!D.u4) return 256;
  const int64_t nmax = std::min<int64_t>(D.slots, D.cap * D.E);
  return nmax >= 64 * static_cast<int64_t>(D.E) ? 256 : 128;
}

// Tile costs for the XCD ranges, in units of one 32-row block's share of a
// K step, from per-workgroup timestamps of the Mixtral- and Qwen-shaped
// layers: a gate/up K step costs about 12-19 units plus one per 32-row block
// (Mixtral-shaped 1.03 us with one block, 1.45 us with eight), a down K step
// about 5-11 plus one per block; set-up, first loads and epilogue add a few
// microseconds per tile.  The spread between workloads (and between XCDs)
// is what the run-time claims of the ranges' last quarters even out.
constexpr int kStepCostUp = 13, kTileCostUp = 100;
constexpr int kStepCostDown = 7, kTileCostDown = 60;

XcdPlan xcd_plan(const Dims& D, bool down) {
  XcdPlan p;
  if (!D.bf16 || (D.u4 && !u4_tiled(D))) return p;  // no routed tiled GEMM
  const int64_t nmax = std::min<int64_t>(D.slots, D.cap * D.E);
  if (down) {
    p.nt = ntiles(kDown, D.d);
    p.ksplit = down_splits(D);
    p.kt = static_cast<int>(D.F / BK / p.ksplit);
    p.c = p.kt * kStepCostDown + kTileCostDown;
  } else {
    p.nt = ntiles(D.swiglu ? kSwiGLU : kReLU, D.F);
    p.kt = static_cast<int>(D.d / BK);
    p.c = p.kt * kStepCostUp + kTileCostUp;
  }
  p.cap = static_cast<int>(routed_grid(nmax, routed_bm(D), static_cast<int>(D.E), p.nt,
                                       p.ksplit) / kXcds);
  return p;
}

int down_splits(const Dims& D) {
  if (!D.bf16 || D.u4) return 1;
  const int KT = D.F / BK;
  if (KT % 2 != 0 || KT < 16) return 1;
  const int64_t nmax = std::min<int64_t>(D.slots, D.cap * D.E);
  const int64_t t = (nmax / routed_bm(D) + D.E) * ntiles(kDown, D.d);  // tile upper bound
  constexpr int64_t kCUs = 256;
  const int64_t half_rounds1 = (t + kCUs - 1) / kCUs * 2;
  const int64_t half_rounds2 = (2 * t + kCUs - 1) / kCUs;
  return half_rounds2 * 10 < half_rounds1 * 9 ? 2 : 1;
}

hipError_t launch_shared_bf16(const Dims& D, const void* x,
                              const moe_expert_weights& w, void* Hs, void* Ys,
                              int32_t* err, hipStream_t s) {
  const int up_mode = D.swiglu ? kSwiGLU : kReLU;
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
    g.err = err;
    hipError_t e = launch_one(up_mode, false, g, D.T, 256, s);
    if (e != hipSuccess) return e;
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
    e = launch_one(kDown, false, h, D.T, 256, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_ffn_bf16(const Dims& D, const int32_t* offsets,
                           const int32_t* tiles1, const int32_t* tiles2,
                           const int32_t* sorted_token, const void* x,
                           const moe_expert_weights& w, const float* row_scale, bool y16,
                           void* H, void* Hs, void* Y, float* Ypart, void* Ys, int32_t* err,
                           hipEvent_t mid, hipStream_t s) {
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
    g.err = err;
    hipError_t e = launch_one(up_mode, true, g, nmax, routed_bm(D), s);
    if (e != hipSuccess) return e;
    if (mid != nullptr && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
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
    g.row_scale = row_scale;
    g.y16 = y16;
    g.err = err;
    if (g.ksplit > 1 && Ypart == nullptr) return hipErrorInvalidValue;
    hipError_t e = launch_one(kDown, false, g, nmax, routed_bm(D), s);
    if (e != hipSuccess) return e;
  }
  if (D.S > 0) return launch_shared_bf16(D, x, w, Hs, Ys, err, s);
  return hipSuccess;
}

hipError_t launch_ffn_u4_tiled(const Dims& D, const int32_t* offsets, const int32_t* tiles1,
                               const int32_t* tiles2, const int32_t* sorted_token,
                               const void* x, void* X16, const moe_expert_weights& w,
                               const float* row_scale, bool y16, void* H, void* Y,
                               int32_t* err, hipEvent_t mid, hipStream_t s) {
  const int up_mode = D.swiglu ? kSwiGLU : kReLU;
  const int64_t nmax = std::min<int64_t>(D.slots, D.cap * D.E);
  // one (scale, bias) per 64 weights of a row, an even number per row
  if (D.d % 128 != 0 || D.F % 128 != 0) return hipErrorInvalidValue;
  {
    const int64_t n8 = D.T * D.d / 8;
    hipLaunchKernelGGL(to_f16_kernel, dim3(static_cast<unsigned>((n8 + 255) / 256)), dim3(256),
                       0, s, static_cast<const uint16_t*>(x), static_cast<uint16_t*>(X16), n8,
                       err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    GemmArgs g{};
    g.a = static_cast<const uint16_t*>(X16);
    g.a_bytes = static_cast<uint32_t>(D.T * D.d * 2);
    g.sorted_token = sorted_token;
    g.offsets = offsets;
    g.tiles = tiles1;
    g.E = D.E;
    g.q0 = static_cast<const uint8_t*>(w.gate);
    g.s0 = static_cast<const uint16_t*>(w.gate_scale);
    g.b0 = static_cast<const uint16_t*>(w.gate_bias);
    if (D.fused) {  // [E][2F] rows: each expert's gate rows, then its up rows
      g.q1 = g.q0 + static_cast<int64_t>(D.F) * (D.d / 2);
      g.s1 = g.s0 + static_cast<int64_t>(D.F) * (D.d / 64);
      g.b1 = g.b0 + static_cast<int64_t>(D.F) * (D.d / 64);
      g.qstride = 2 * static_cast<int64_t>(D.F);
    } else {
      g.q1 = static_cast<const uint8_t*>(w.up);
      g.s1 = static_cast<const uint16_t*>(w.up_scale);
      g.b1 = static_cast<const uint16_t*>(w.up_bias);
      g.qstride = D.F;
    }
    g.nibble_mask = 0x0F0F0F0Fu;
    g.N = D.F;
    g.K = D.d;
    g.out = H;
    g.ldo = D.F;
    g.NT = ntiles(up_mode, D.F);
    g.ksplit = 1;
    g.err = err;
    hipError_t e = launch_one(up_mode, true, g, nmax, routed_bm(D), s, true);
    if (e != hipSuccess) return e;
    if (mid != nullptr && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
  }
  GemmArgs g{};
  g.a = static_cast<const uint16_t*>(H);
  g.a_bytes = static_cast<uint32_t>(D.slots * D.F * 2);
  g.offsets = offsets;
  g.tiles = tiles2;
  g.E = D.E;
  g.q0 = g.q1 = static_cast<const uint8_t*>(w.down);
  g.s0 = g.s1 = static_cast<const uint16_t*>(w.down_scale);
  g.b0 = g.b1 = static_cast<const uint16_t*>(w.down_bias);
  g.qstride = D.d;
  g.nibble_mask = 0x0F0F0F0Fu;
  g.N = D.d;
  g.K = D.F;
  g.out = Y;
  g.row_scale = row_scale;
  g.y16 = y16;
  g.err = err;
  g.ldo = D.d;
  g.NT = ntiles(kDown, D.d);
  g.ksplit = 1;
  return launch_one(kDown, false, g, nmax, routed_bm(D), s, true);
}

}  // namespace moe
