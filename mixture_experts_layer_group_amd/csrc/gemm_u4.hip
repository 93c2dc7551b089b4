// Grouped expert FFN with 4-bit affine routed weights (Edge0 "MoE Spec and
// Routing" page, QuantSpec: bits 4, group 64, mode affine; w = scale*q +
// bias), bf16 activations, fp32 accumulation.
//
// Built for decode-shaped batches, where each touched expert sees a handful
// of rows and the layer is bound by streaming the packed weights from HBM:
// every weight byte is read once and serves up to 4 of the expert's rows.
// The affine dequantisation is factored per group so no dequantised weight
// is formed:
//   sum_j x_j (s q_j + b) = s * sum_j x_j q_j + b * sum_j x_j
// The codes enter the matrix cores as exact fp16 values (1024 + q for the
// even nibbles, 1024 + 16q for the odd ones, one AND-OR per pair of codes)
// and sum_j x_j q_j is formed by v_mfma_f32_4x4x4_16b_f16: 16 independent
// 4x4x4 products per instruction, each block taking 4 units of the weight
// matrix against up to 4 activation rows over its own slice of K.  The
// blocks of one unit group split K between them; their partial sums, scaled
// per group, are added across lanes once per item.
//
// One kernel serves both products:
//   up   : unit = hidden column f; the gate row f and the up row f, the
//          epilogue writes H = silu(gate) * up (fp16, as on the
//          matrix-core path)
//   down : unit = output column n of W_down, writes Y (fp32)
#include <algorithm>
#include <type_traits>

#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kMaxK = 2048;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// In-place sum of V per-lane values over the lanes that differ only in the
// bits D, D/2, ..., 4 (the K slices of a unit group).  Butterfly with
// halving: at distance D the lane with bit D set keeps the upper half of its
// values and sends the lower half; once one value is left the remaining
// distances add it whole.  On return a lane holds max(1, V >> halvings)
// totals, those of indices kred_index(lane, j).
template <int D, int CNT, int V>
__device__ __forceinline__ void kred(float (&v)[V], int lane) {
  if constexpr (D >= 4) {
    if constexpr (CNT > 1) {
      constexpr int kHalf = CNT / 2;
      const bool upper = (lane & D) != 0;
#pragma unroll
      for (int i = 0; i < kHalf; ++i) {
        const float send = upper ? v[i] : v[i + kHalf];
        const float keep = upper ? v[i + kHalf] : v[i];
        v[i] = keep + xor_move<D>(send, lane);
      }
      kred<D / 2, kHalf, V>(v, lane);
    } else {
      v[0] += xor_move<D>(v[0], lane);
      kred<D / 2, 1, V>(v, lane);
    }
  }
}

// index of v[j] after kred<DTOP, V, V> on this lane
template <int V, int DTOP>
__device__ __forceinline__ int kred_index(int lane, int j) {
  int idx = j, c = V;
#pragma unroll
  for (int d = DTOP; d >= 4 && c > 1; d >>= 1) {
    c /= 2;
    if (lane & d) idx += c;
  }
  return idx;
}

// lowest distance at which kred<DTOP, V, V> still halves (2 * DTOP when it
// never does); lanes that differ only in the bits from 4 up to below it
// hold the same totals
template <int V, int DTOP>
constexpr int kred_last() {
  int c = V, last = 2 * DTOP;
  for (int d = DTOP; d >= 4 && c > 1; d >>= 1) {
    c /= 2;
    last = d;
  }
  return last < 4 ? 4 : last;
}

// Work layout for a reduction length K (a power of two from 64 to 2048).
// Lane 4b+i of a wave is row i of MFMA block b (unit i of the block's group
// in the A operand, activation row i in the B operand); block
// b = ug * NKS + ks takes the 4 units of unit group ug over K slice ks (KB
// elements).  An item is UPI = 4 * NUG consecutive units of one expert:
// 32 * KB bytes of codes per matrix (4 KiB; 2 KiB for K = 64) and
// 2 * KB bytes each of scales and biases.
template <int K>
struct KCfg {
  static constexpr int KB = K < 128 ? K : 128;
  static constexpr int NKS = K / KB;         // K slices per unit group
  static constexpr int NUG = 16 / NKS;       // unit groups per item
  static constexpr int UPI = 4 * NUG;        // units per item
  static constexpr int WPL = KB / 8;         // packed words per lane and matrix
  static constexpr int GPL = KB / 64;        // quantisation groups per K slice
  static constexpr int G = K / 64;           // groups per unit row
  static constexpr int kCode = UPI * K / 2;  // code bytes per matrix
  static constexpr int kDma = kCode / 1024;  // wave-wide 16-byte loads per matrix
  static constexpr int kSB = UPI * G * 2;    // scale (or bias) bytes per matrix
  static constexpr int kSBLanes = kSB / 4;   // lanes of its 4-byte load
  // In LDS, 16-byte piece p of a kSeg-byte segment of unit u sits at slot
  // p ^ (u % kPieces): the 16 lanes that one LDS read serves together (4 K
  // slices x 4 units) then hit distinct banks for K >= 512.
  static constexpr int kSeg = K / 2 < 64 ? K / 2 : 64;
  static constexpr int kPieces = kSeg / 16;
  static_assert(NKS * NUG == 16 && GPL >= 1 && WPL % 4 == 0, "blocks");
  static_assert(kCode == 32 * KB && kCode % 1024 == 0 && kSB == 2 * KB, "item layout");
};

// ---------------------------------------------------------------- streaming
// The packed weights stream through LDS.  The active experts are listed on
// the device and their items numbered (expert, row chunk, unit block) with
// the unit block fastest; every wave of a persistent grid takes one
// contiguous range of items of equal cost, an item of r rows costing
// kItemCost + r, so a wave on a busy expert takes fewer items.  A chunk is up
// to 4 of the expert's rows (the 4 columns of every MFMA block), so an
// expert with more than 4 rows streams its weights once per chunk.  A wave
// is an independent pipeline over a private ring of NS stages in LDS: the
// direct-to-LDS loads of later items are issued before the current item is
// computed (NS-1 of them; NS on the gate/up product, which copies an item
// into registers as soon as it arrives and reloads its stage at once), and
// the only wait is the wave's own vmcnt.  Inside the loop no other vector
// load is waited for except when a new row chunk's activations are read.
// The buffer descriptors carry each expert matrix's size, so a load past
// the last unit fetches nothing.
constexpr int kItemCost = 12;    // cost of an item beyond its rows, in rows
constexpr int kMaxExperts = 1024;
constexpr int kMaxChunkRows = 4;

// Per product: one workgroup per CU of 8 (gate/up) or 16 (down) waves, two
// stages per wave: 144 KiB of ring for the decode shapes (K = 2048 and 512).
// Measured on the decode layer: the down kernel with 16 waves beats 8 waves
// with 3 or 4 stages (with or without the register copy) and 12 waves by
// 1-4%; fewer waves with deeper rings (4 x 4, 4 x 8) are slower by a
// quarter or more.
template <bool PAIR, int K>
struct SCfg {
  using KC = KCfg<K>;
  static constexpr int kWaves = PAIR ? 8 : 16;
  static constexpr int kRows = kMaxChunkRows;
  static constexpr int kStages = 2;
  // an item is read into registers as soon as it arrives (frees its stage
  // one item earlier; needs about 50 VGPRs that the 16-wave down kernel lacks)
  static constexpr bool kRegs = PAIR;
  static constexpr int M = PAIR ? 2 : 1;
  static constexpr int kBytes = M * KC::kCode + 2 * M * KC::kSB;  // one stage
  static constexpr int kLoads = M * KC::kDma + 2 * M;  // load instructions per item
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kPasses = (kMaxExperts + kThreads - 1) / kThreads;
  static constexpr int kLds =
      kWaves * kStages * kBytes + (3 * kMaxExperts + 2) * 4 + 3 * kPasses * kWaves * 4;
  static_assert(kLds <= 160 * 1024, "stream layout");
};

// The direct-to-LDS loads are written out here rather than through the
// compiler builtin: for the builtin the compiler waits for every pending
// LDS load before any LDS read (vmcnt(0)), which would drain the ring on
// every item.  Written out, the loads are ordered only by the explicit
// waits below (and by the memory clobbers); the compiler's own counter
// waits for its loads stay correct, only more conservative, because vector
// memory loads complete in issue order.
typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));

// buffer descriptor: base, stride 0, size in bytes (loads past it fetch
// nothing), the raw-buffer flags
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  rsrc_t r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xffffu);
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000u;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) void*)p));
}

// 64 lanes x 16 bytes from rsrc at voff into LDS [lds, lds + 1024).  The
// whole offset is in the VGPR: the range check covers only that part.
__device__ __forceinline__ void dma16(rsrc_t rs, uint32_t lds, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rs), "{m0}"(lds)
               : "memory");
}

// active lanes x 4 bytes into LDS [lds, lds + 4 * lanes)
__device__ __forceinline__ void dma4(rsrc_t rs, uint32_t lds, uint32_t voff) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rs), "{m0}"(lds)
               : "memory");
}

// wait until at most N vector-memory operations of this wave are pending.
// The counted waits of the ring rest on two facts: every load of an item is
// issued by the wave (the loads are asm statements, which the compiler can
// neither drop nor merge; the one lane-dependent condition, on the scale and
// bias loads when K = 64, holds for lanes 0-31 of every wave), and
// vector-memory operations retire in issue order.  Any other vector-memory operation the
// compiler places between an item's loads and its wait only makes the count
// more conservative: whether it is older or younger than the awaited item,
// "at most N pending" still implies that the item's loads have retired.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <int L, int NS>
__device__ __forceinline__ void wait_later(int later) {
  // `later` item groups of L loads each were issued after the awaited one
  if constexpr (NS > 3) {
    if (later >= 3) { wait_vm<3 * L>(); return; }
  }
  if constexpr (NS > 2) {
    if (later == 2) { wait_vm<2 * L>(); return; }
  }
  if (later == 1) { wait_vm<L>(); return; }
  wait_vm<0>();
}

// A VGPR holding c that the optimiser cannot fold back into a literal, so
// that (a & m) | c with m in it is one v_and_or_b32 (a VOP3 instruction
// takes no literal here).  The AND-OR itself stays ordinary code: the
// matrix cores read its results, and the compiler must see it as the VALU
// write it is to keep the required wait states in front of them.
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
  return r;
}

// The 8 codes of one packed word as four fp16 pairs:
//   c[0] = (q0, q4) + 1024,  c[1] = 16 * (q1, q5) + 1024,
//   c[2] = (q2, q6) + 1024,  c[3] = 16 * (q3, q7) + 1024
// (0x6400 is 1024.0; a code in mantissa bits 0-3 adds q, in bits 4-7 adds
// 16q, both exactly).  m_lo = 0x000F000F, m_hi = 0x00F000F0.
__device__ __forceinline__ void unpack8(uint32_t w, uint32_t m_lo, uint32_t m_hi,
                                        half2_t* c) {
  const uint32_t h = w >> 8;
  c[0] = __builtin_bit_cast(half2_t, (w & m_lo) | 0x64006400u);
  c[1] = __builtin_bit_cast(half2_t, (w & m_hi) | 0x64006400u);
  c[2] = __builtin_bit_cast(half2_t, (h & m_lo) | 0x64006400u);
  c[3] = __builtin_bit_cast(half2_t, (h & m_hi) | 0x64006400u);
}

// Eight activations of a row (bf16, or fp16 when !BF16) as the two MFMA B
// operands that match unpack8: xa = (x0, x4, x2, x6) against the codes
// that carry 1024 + q, xb = (x1, x5, x3, x7) against 1024 + 16q, with the
// fp32 sums of the fp16 values of each set.
template <bool BF16>
__device__ __forceinline__ void load_word(const uint16_t* p, half4_t& xa, half4_t& xb,
                                          float& sa, float& sb) {
  const uint4 t = *reinterpret_cast<const uint4*>(p);
  const uint32_t tw[4] = {t.x, t.y, t.z, t.w};
  _Float16 h[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (BF16) {
      h[2 * i] = static_cast<_Float16>(__uint_as_float(tw[i] << 16));
      h[2 * i + 1] = static_cast<_Float16>(__uint_as_float(tw[i] & 0xffff0000u));
    } else {
      h[2 * i] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(tw[i] & 0xffffu));
      h[2 * i + 1] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(tw[i] >> 16));
    }
  }
  xa = half4_t{h[0], h[4], h[2], h[6]};
  xb = half4_t{h[1], h[5], h[3], h[7]};
  sa += (static_cast<float>(h[0]) + static_cast<float>(h[4])) +
        (static_cast<float>(h[2]) + static_cast<float>(h[6]));
  sb += (static_cast<float>(h[1]) + static_cast<float>(h[5])) +
        (static_cast<float>(h[3]) + static_cast<float>(h[7]));
}

struct U4Args {
  const int32_t* offsets;       // [E+1]
  const int32_t* sorted_token;  // nullptr: activation row = kept row
  const uint16_t* a;            // bf16 x [T][K] or fp16 H [rows][K]
  const uint8_t* q[2];          // packed codes of expert 0 (gate, up | down)
  const uint8_t* s[2];          // bf16 scales of expert 0
  const uint8_t* b[2];          // bf16 biases of expert 0
  void* out;                    // fp16 H [rows][N] (pair) or fp32 Y [rows][N]
  int E;
  int N;                        // units (output columns) per expert
  int rstride;                  // rows from one expert's matrix to the next
  int32_t* err;                 // MOE_FLAG_H_SATURATED is OR-ed in (or nullptr)
  const float* row_scale;       // down: factor of each output row (nullptr: 1)
};

// exclusive prefix over the lanes of a wave, and the wave total: an
// inclusive scan inside each row of 16 lanes by DPP row shifts (a lane
// without a source lane reads 0), then the totals of the rows before this
// one from three lane reads
__device__ __forceinline__ int wave_prefix(int v, int lane, int& total) {
  int inc = v;
  inc += dpp_i<0x111>(inc);  // row_shr:1
  inc += dpp_i<0x112>(inc);  // row_shr:2
  inc += dpp_i<0x114>(inc);  // row_shr:4
  inc += dpp_i<0x118>(inc);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(inc, 15);
  const int r1 = __builtin_amdgcn_readlane(inc, 31);
  const int r2 = __builtin_amdgcn_readlane(inc, 47);
  const int r3 = __builtin_amdgcn_readlane(inc, 63);
  const int row = lane >> 4;
  inc += (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
  total = r0 + r1 + r2 + r3;
  return inc - v;
}

// WEIGHTED (down product only): each output row is multiplied by
// g.row_scale[row]
template <bool PAIR, int K, bool WEIGHTED>
__device__ __forceinline__ void u4_stream(const U4Args& g, uint8_t* smem) {
  using SL = SCfg<PAIR, K>;
  using KC = KCfg<K>;
  constexpr int kRows = SL::kRows;
  constexpr int kSWaves = SL::kWaves;
  constexpr int UPI = KC::UPI;
  constexpr int G = KC::G;
  constexpr int NS = SL::kStages;
  constexpr int M = SL::M;
  constexpr int L = SL::kLoads;
  constexpr int V = 4 * M;             // an item's per-lane values: 4 units x M matrices
  constexpr int DTOP = 2 * KC::NKS;    // largest lane distance between K slices

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int32_t* act_e = reinterpret_cast<int32_t*>(smem + kSWaves * NS * SL::kBytes);
  int32_t* act_p = act_e + kMaxExperts;     // [A+1] first chunk of each active expert
  int32_t* act_c = act_p + kMaxExperts + 1; // [A+1] cost before each active expert
  int32_t* wsum = act_c + kMaxExperts + 1;  // [3 * passes][kSWaves] per-wave totals

  // ---- the active experts in expert order, and their row chunks
  const int E = g.E;
  constexpr int kT = SL::kThreads;  // expert tid + kT * h
  constexpr int kH = SL::kPasses;
  int cnt[kH];
#pragma unroll
  for (int h = 0; h < kH; ++h) {
    const int e = tid + kT * h;
    cnt[h] = e < E ? g.offsets[e + 1] - g.offsets[e] : 0;
  }
  const int NBW = (g.N + UPI - 1) / UPI;
  int rank[kH], first[kH], cost[kH];
#pragma unroll
  for (int h = 0; h < kH; ++h) {
    int t0, t1, t2;
    const int ch = (cnt[h] + kRows - 1) / kRows;
    rank[h] = wave_prefix(cnt[h] > 0 ? 1 : 0, lane, t0);
    first[h] = wave_prefix(ch, lane, t1);
    // every chunk costs NBW items of kItemCost plus its rows
    cost[h] = wave_prefix(NBW * (ch * kItemCost + cnt[h]), lane, t2);
    if (lane == 0) {
      wsum[(3 * h) * kSWaves + wave] = t0;
      wsum[(3 * h + 1) * kSWaves + wave] = t1;
      wsum[(3 * h + 2) * kSWaves + wave] = t2;
    }
  }
  __syncthreads();
  int tot[kH][3], bef[kH][3];
#pragma unroll
  for (int h = 0; h < kH; ++h)
#pragma unroll
    for (int q = 0; q < 3; ++q) tot[h][q] = bef[h][q] = 0;
#pragma unroll
  for (int h = 0; h < kH; ++h)
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) {
        const int c = wsum[(3 * h + q) * kSWaves + w];
        bef[h][q] += w < wave ? c : 0;
        tot[h][q] += c;
      }
  int A = 0, C = 0, TC = 0;  // totals of the passes before h, then overall
#pragma unroll
  for (int h = 0; h < kH; ++h) {
    if (cnt[h] > 0) {
      const int r = A + bef[h][0] + rank[h];
      act_e[r] = tid + kT * h;
      act_p[r] = C + bef[h][1] + first[h];
      act_c[r] = TC + bef[h][2] + cost[h];
    }
    A += tot[h][0];
    C += tot[h][1];
    TC += tot[h][2];
  }
  A = __builtin_amdgcn_readfirstlane(A);
  C = __builtin_amdgcn_readfirstlane(C);
  TC = __builtin_amdgcn_readfirstlane(TC);
  if (tid == 0) {
    act_p[A] = C;
    act_c[A] = TC;
  }
  __syncthreads();

  // ---- this wave's items: (active expert a, chunk k, unit block b), item
  // i = (act_p[a] + k) * NBW + b.  The wave starts at the first item whose
  // cost prefix reaches gw * TC / W and ends where the next wave starts.
  // Item numbers and costs fit in 32 bits (checked on the host).
  const int64_t W = static_cast<int64_t>(gridDim.x) * kSWaves;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * kSWaves + wave;
  auto start_item = [&](int64_t wv) -> int {
    const int x = static_cast<int>(wv * TC / W);
    if (x >= TC) return C * NBW;
    int lo = 0, hi = A - 1;  // largest a with act_c[a] <= x
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (act_c[mid] <= x) lo = mid; else hi = mid - 1;
    }
    const int e = act_e[lo];
    const int cnt_e = g.offsets[e + 1] - g.offsets[e];
    const int ch = act_p[lo + 1] - act_p[lo];
    const int full = NBW * (kItemCost + kRows);  // cost of a chunk of kRows rows
    const int y = x - act_c[lo];
    int k = min(y / full, ch - 1);
    const int rows = min(kRows, cnt_e - k * kRows);
    const int rem = y - k * full;
    const int b = (rem + kItemCost + rows - 1) / (kItemCost + rows);  // may be NBW
    return (act_p[lo] + k) * NBW + b;
  };
  const int i0 = __builtin_amdgcn_readfirstlane(start_item(gw));
  const int n = __builtin_amdgcn_readfirstlane(start_item(gw + 1)) - i0;
  uint8_t* ring = smem + wave * NS * SL::kBytes;
  int a0 = 0, k0 = 0, b0 = 0;
  if (n > 0) {
    const int c0 = i0 / NBW;
    b0 = i0 - c0 * NBW;
    int lo = 0, hi = A - 1;  // largest a with act_p[a] <= c0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (act_p[mid] <= c0) lo = mid; else hi = mid - 1;
    }
    a0 = __builtin_amdgcn_readfirstlane(lo);
    k0 = c0 - act_p[a0];
  }
  // iterators of the next item to load (a, b) and to compute (a, k, b)
  int ia = a0, ik = k0, ib = b0;
  int ca = a0, ck = k0, cb = b0;
  auto advance = [&](int& a, int& k, int& b) {
    if (++b == NBW) {
      b = 0;
      if (++k == act_p[a + 1] - act_p[a]) {
        k = 0;
        ++a;
      }
    }
  };

  // ---- per-lane layout
  const int i4 = lane & 3;  // unit i4 of the block's group (A), activation row i4 (B)
  const int blk = lane >> 2;
  const int ug = blk / KC::NKS, ks = blk % KC::NKS;
  // load c of a matrix fills LDS bytes [1024c, 1024c + 1024) of the item's
  // code region; lane l writes bytes 1024c + 16l and fetches the piece that
  // the slot rotation puts there
  uint32_t dma_off[KC::kDma];
#pragma unroll
  for (int c = 0; c < KC::kDma; ++c) {
    const int q = c * 1024 + 16 * lane;
    const int u = q / (K / 2), o = q % (K / 2);
    const int slot = (o % KC::kSeg) / 16;
    dma_off[c] = static_cast<uint32_t>(u * (K / 2) + (o / KC::kSeg) * KC::kSeg +
                                       ((slot ^ (u % KC::kPieces)) * 16));
  }
  // read c of a lane: 16 bytes (4 packed words) of unit 4*ug + i4 at code
  // byte ks * KB/2 + 16c of its row
  uint32_t rd_off[KC::WPL / 4];
#pragma unroll
  for (int c = 0; c < KC::WPL / 4; ++c) {
    const int u = 4 * ug + i4;
    const int o = ks * (KC::KB / 2) + 16 * c;
    const int piece = (o % KC::kSeg) / 16;
    rd_off[c] = static_cast<uint32_t>(u * (K / 2) + (o / KC::kSeg) * KC::kSeg +
                                      ((piece ^ (u % KC::kPieces)) * 16));
  }

  auto issue = [&](int t) {
    const int a = ia;
    const int u0 = ib * UPI;
    advance(ia, ik, ib);
    const int e = __builtin_amdgcn_readfirstlane(act_e[a]);
    const uint32_t st = __builtin_amdgcn_readfirstlane(
        lds_addr(ring + (t % NS) * SL::kBytes));
    const int64_t erow = static_cast<int64_t>(e) * g.rstride;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const rsrc_t rq = make_rsrc(g.q[m] + erow * (K / 2), g.N * (K / 2));
      const uint32_t vq = static_cast<uint32_t>(u0 * (K / 2));
#pragma unroll
      for (int c = 0; c < KC::kDma; ++c)
        dma16(rq, st + m * KC::kCode + c * 1024, vq + dma_off[c]);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t vs = static_cast<uint32_t>(u0 * G * 2 + lane * 4);
      const rsrc_t rs = make_rsrc(g.s[m] + erow * (G * 2), g.N * G * 2);
      const rsrc_t rb = make_rsrc(g.b[m] + erow * (G * 2), g.N * G * 2);
      // the item's scales (biases) are kSB contiguous bytes
      if (KC::kSBLanes >= 64 || lane < KC::kSBLanes) {
        dma4(rs, st + M * KC::kCode + (2 * m) * KC::kSB, vs);
        dma4(rb, st + M * KC::kCode + (2 * m + 1) * KC::kSB, vs);
      }
    }
  };

  // the chunk's activation row i4 over K slice ks, as MFMA B operands
  const uint32_t m_lo = opaque_vgpr(0x000F000Fu), m_hi = opaque_vgpr(0x00F000F0u);
  half4_t xa[KC::WPL], xb[KC::WPL];
  float xs[KC::GPL], xc[KC::GPL];
  float row_f = 1.f;  // the factor of this lane's output row (down product)
  auto load_rows = [&](int row0, int rows) {
    // a lane past the chunk's rows reads the chunk's first row and keeps
    // zeros, so no branch divides the wave here
    const bool live = i4 < rows;
    const int32_t kr = row0 + (live ? i4 : 0);
    const int64_t src = g.sorted_token ? static_cast<int64_t>(g.sorted_token[kr])
                                       : static_cast<int64_t>(kr);
    const uint16_t* p = g.a + src * K + ks * KC::KB;
    if constexpr (WEIGHTED) row_f = g.row_scale[kr];
    const half4_t zero = half4_t{0, 0, 0, 0};
#pragma unroll
    for (int gg = 0; gg < KC::GPL; ++gg) {
      float sa = 0.f, sb = 0.f;
#pragma unroll
      for (int w = gg * 8; w < gg * 8 + 8; ++w) {
        load_word<PAIR>(p + 8 * w, xa[w], xb[w], sa, sb);
        xa[w] = live ? xa[w] : zero;
        xb[w] = live ? xb[w] : zero;
      }
      xs[gg] = live ? sa + sb : 0.f;
      // offsets carried by the codes: 1024 per element of xa, 64 (1024/16)
      // per element of xb
      xc[gg] = live ? fmaf(1024.f, sa, 64.f * sb) : 0.f;
    }
  };

  // kRegs: an item's codes and its group scales and biases, read out of its
  // stage into registers, so that the stage can take the next load before
  // the item is computed (otherwise they are read from the stage as it goes)
  uint4 rq[M][KC::WPL / 4];
  uint32_t rsc[M][4][KC::GPL], rbi[M][4][KC::GPL];
  auto fetch = [&](const uint8_t* st) {
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int c = 0; c < KC::WPL / 4; ++c)
        rq[m][c] = *reinterpret_cast<const uint4*>(st + m * KC::kCode + rd_off[c]);
    const uint16_t* sb = reinterpret_cast<const uint16_t*>(st + M * KC::kCode);
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int so = (4 * ug + v) * G + ks * KC::GPL;
#pragma unroll
        for (int gg = 0; gg < KC::GPL; ++gg) {
          rsc[m][v][gg] = sb[(2 * m) * (KC::kSB / 2) + so + gg];
          rbi[m][v][gg] = sb[(2 * m + 1) * (KC::kSB / 2) + so + gg];
        }
      }
  };

  // a hidden activation outside the fp16 range (or NaN); reported once,
  // after the item loop, so the flag adds no memory operation between the
  // ring's loads and their waits
  bool sat = false;
  // the item in stage st (fetched with kRegs): units u0.. of the expert,
  // chunk rows row0..
  auto compute = [&](const uint8_t* st, int row0, int rows, int u0) {
    float4_t acc[M][KC::GPL][2];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int gg = 0; gg < KC::GPL; ++gg)
        acc[m][gg][0] = acc[m][gg][1] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
      for (int c = 0; c < KC::WPL / 4; ++c) {
        uint4 q;
        if constexpr (SL::kRegs)
          q = rq[m][c];
        else
          q = *reinterpret_cast<const uint4*>(st + m * KC::kCode + rd_off[c]);
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int w = 4 * c + t;
          half2_t cc[4];
          unpack8(qw[t], m_lo, m_hi, cc);
          const half4_t aa = half4_t{cc[0][0], cc[0][1], cc[2][0], cc[2][1]};
          const half4_t ab = half4_t{cc[1][0], cc[1][1], cc[3][0], cc[3][1]};
          acc[m][w / 8][0] = __builtin_amdgcn_mfma_f32_4x4x4f16(aa, xa[w], acc[m][w / 8][0], 0, 0, 0);
          acc[m][w / 8][1] = __builtin_amdgcn_mfma_f32_4x4x4f16(ab, xb[w], acc[m][w / 8][1], 0, 0, 0);
        }
      }
    }
    // result register v of a lane: unit 4*ug + v against activation row i4,
    // over K slice ks; apply the slice's group scales and biases
    const uint16_t* sb = reinterpret_cast<const uint16_t*>(st + M * KC::kCode);
    float val[V];  // index v * M + m
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int so = (4 * ug + v) * G + ks * KC::GPL;
        float tot = 0.f;
#pragma unroll
        for (int gg = 0; gg < KC::GPL; ++gg) {
          const uint32_t sw = SL::kRegs ? rsc[m][v][gg] : sb[(2 * m) * (KC::kSB / 2) + so + gg];
          const uint32_t bw = SL::kRegs ? rbi[m][v][gg] : sb[(2 * m + 1) * (KC::kSB / 2) + so + gg];
          const float sc = __uint_as_float(sw << 16);
          const float bi = __uint_as_float(bw << 16);
          const float dm = fmaf(acc[m][gg][1][v], 0.0625f, acc[m][gg][0][v]) - xc[gg];
          tot = fmaf(sc, dm, fmaf(bi, xs[gg], tot));
        }
        val[v * M + m] = tot;
      }
    }
    kred<DTOP, V, V>(val, lane);
    constexpr int C = KC::NKS >= V ? 1 : V / KC::NKS;
    constexpr int kLast = kred_last<V, DTOP>();
    // lanes that differ only in the bits from 4 to below kLast hold the
    // same totals: the one with those bits clear writes
    const bool writer = (lane & (kLast - 1) & ~3) == 0;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float gv = val[j], upv = 0.f;
      const int idx = kred_index<V, DTOP>(lane, j);
      if (PAIR) {
        // gate and up of one (unit, row) sit side by side when a lane keeps
        // several totals, else in the lanes kLast apart
        if constexpr (C > 1) {
          if (j % 2 == 1) continue;
          upv = val[j + 1];
        } else {
          upv = xor_move<kLast>(val[0], lane);
          if (idx % 2 == 1) continue;
        }
      }
      const int u = u0 + 4 * ug + idx / M;
      if (!writer || i4 >= rows || u >= g.N) continue;
      const int64_t o = static_cast<int64_t>(row0 + i4) * g.N + u;
      if (PAIR) {  // hidden activation, fp16 (saturating)
        float h = gv / (1.f + __expf(-gv)) * upv;
        sat |= !(fabsf(h) <= 65504.f);
        h = fminf(fmaxf(h, -65504.f), 65504.f);
        static_cast<_Float16*>(g.out)[o] = static_cast<_Float16>(h);
      } else {  // expert output, fp32
        static_cast<float*>(g.out)[o] = WEIGHTED ? gv * row_f : gv;
      }
    }
  };

  int cache_e = -1, cache_k = -1;
  // With kRegs the item is read into registers as soon as it has arrived
  // and its stage takes the load of the item NS ahead at once, so NS items
  // are in flight while one is computed; without, the stage of item t-1
  // takes the item NS-1 ahead.
  constexpr int AHEAD = SL::kRegs ? NS : NS - 1;
  for (int t = 0; t < AHEAD && t < n; ++t) issue(t);
  for (int t = 0; t < n; ++t) {
    if constexpr (!SL::kRegs) {
      if (t + NS - 1 < n) issue(t + NS - 1);  // into the stage freed by item t-1
    }
    wait_later<L, NS>(min(NS - 1, n - 1 - t));
    if constexpr (SL::kRegs) {
      fetch(ring + (t % NS) * SL::kBytes);
      if (t + NS < n) {
        // the stage's reads must have returned before its next load lands
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(t + NS);
      }
    }
    const int a = ca, k = ck;
    const int u0 = cb * UPI;
    advance(ca, ck, cb);
    const int e = __builtin_amdgcn_readfirstlane(act_e[a]);
    // the offsets are read through the constant address space: a scalar
    // load, which leaves the direct loads in flight alone (a vector load here
    // would make the compiler wait for every pending load of the wave)
    const auto* offs = (const __attribute__((address_space(4))) int32_t*)(g.offsets);
    const int row0 = offs[e] + k * kRows;
    const int rows = min(kRows, offs[e + 1] - row0);
    if (cache_e != e || cache_k != k) {
      load_rows(row0, rows);
      cache_e = e;
      cache_k = k;
    }
    compute(ring + (t % NS) * SL::kBytes, row0, rows, u0);
  }
  if (PAIR && g.err != nullptr && __ballot(sat) != 0 && lane == 0)
    atomicOr(g.err, MOE_FLAG_H_SATURATED);
}

#define MOE_U4S_KERNEL(P, K)                                                    \
  __global__ void __launch_bounds__((SCfg<P, K>::kThreads))                   \
      u4s_kernel_##P##_##K(U4Args g) {                                        \
    __shared__ __attribute__((aligned(16))) uint8_t smem[SCfg<P, K>::kLds];   \
    u4_stream<P, K, false>(g, smem);                                          \
  }
// the down product with weighted rows
#define MOE_U4W_KERNEL(K)                                                       \
  __global__ void __launch_bounds__((SCfg<false, K>::kThreads))               \
      u4s_kernel_weighted_##K(U4Args g) {                                     \
    __shared__ __attribute__((aligned(16))) uint8_t smem[SCfg<false, K>::kLds]; \
    u4_stream<false, K, true>(g, smem);                                       \
  }
MOE_U4S_KERNEL(true, 2048)
MOE_U4S_KERNEL(true, 1024)
MOE_U4S_KERNEL(true, 512)
MOE_U4S_KERNEL(true, 256)
MOE_U4S_KERNEL(true, 128)
MOE_U4S_KERNEL(true, 64)
MOE_U4S_KERNEL(false, 2048)
MOE_U4S_KERNEL(false, 1024)
MOE_U4S_KERNEL(false, 512)
MOE_U4S_KERNEL(false, 256)
MOE_U4S_KERNEL(false, 128)
MOE_U4S_KERNEL(false, 64)
MOE_U4W_KERNEL(2048)
MOE_U4W_KERNEL(1024)
MOE_U4W_KERNEL(512)
MOE_U4W_KERNEL(256)
MOE_U4W_KERNEL(128)
MOE_U4W_KERNEL(64)
#undef MOE_U4W_KERNEL
#undef MOE_U4S_KERNEL

int stream_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  return cus;
}

// K is a power of two from 64 to 2048
bool supported_k(int K) { return K >= 64 && K <= kMaxK && (K & (K - 1)) == 0; }

template <bool PAIR>
hipError_t launch_stream(int K, const U4Args& g, hipStream_t s) {
  const dim3 grid(stream_grid()), block(SCfg<PAIR, 64>::kThreads);
#define MOE_U4S(KK)                                                                    \
  case KK:                                                                             \
    hipLaunchKernelGGL(PAIR ? u4s_kernel_true_##KK                                     \
                            : (g.row_scale ? u4s_kernel_weighted_##KK : u4s_kernel_false_##KK), \
                       grid, block, 0, s, g);                                          \
    break;
  switch (K) {
    MOE_U4S(2048)
    MOE_U4S(1024)
    MOE_U4S(512)
    MOE_U4S(256)
    MOE_U4S(128)
    MOE_U4S(64)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_U4S
  return hipGetLastError();
}

}  // namespace

// Average kept rows per expert from which the tiled matrix-core kernel
// (256-row tiles, weights read once per tile) takes over from the weight
// stream (weights read once per 4-row chunk).
constexpr int kTiledRowsPerExpert = 32;

bool u4_tiled(const Dims& D) {
  const bool stream_ok = D.swiglu && supported_k(D.d) && supported_k(D.F) && D.E <= kMaxExperts;
  const bool tiled_ok = D.d % 128 == 0 && D.F % 128 == 0;
  if (!stream_ok) return true;  // the spec check lets through only shapes one of them takes
  if (!tiled_ok) return false;
  const int64_t rows = std::min<int64_t>(D.slots, D.cap * D.E);
  return rows >= static_cast<int64_t>(kTiledRowsPerExpert) * D.E;
}

hipError_t launch_ffn_u4(const Dims& D, int group, const int32_t* offsets,
                         const int32_t* sorted_token, const void* x,
                         const moe_expert_weights& w, const float* row_scale, void* H,
                         void* Y, int32_t* err, hipEvent_t mid, hipStream_t s) {
  if (!supported_k(D.d) || !supported_k(D.F) || !D.swiglu || group != 64 ||
      D.E > kMaxExperts)
    return hipErrorInvalidValue;
  // item numbers and item costs are 32-bit: row chunks (at most T*k/4 + E)
  // times unit blocks per expert (at least 4 units each), times the cost of
  // an item
  const int64_t chunks = D.slots / kMaxChunkRows + D.E;
  const int64_t blocks = std::max(D.F, D.d) / 4 + 1;
  if (chunks * blocks * (kItemCost + kMaxChunkRows) > INT32_MAX) return hipErrorInvalidValue;
  const int64_t words_d = D.d / 8, groups_d = D.d / 64;
  U4Args g{};
  g.offsets = offsets;
  g.sorted_token = sorted_token;
  g.a = static_cast<const uint16_t*>(x);
  g.q[0] = static_cast<const uint8_t*>(w.gate);
  g.s[0] = static_cast<const uint8_t*>(w.gate_scale);
  g.b[0] = static_cast<const uint8_t*>(w.gate_bias);
  if (D.fused) {  // each expert's F gate rows, then its F up rows
    g.q[1] = g.q[0] + static_cast<int64_t>(D.F) * words_d * 4;
    g.s[1] = g.s[0] + static_cast<int64_t>(D.F) * groups_d * 2;
    g.b[1] = g.b[0] + static_cast<int64_t>(D.F) * groups_d * 2;
  } else {
    g.q[1] = static_cast<const uint8_t*>(w.up);
    g.s[1] = static_cast<const uint8_t*>(w.up_scale);
    g.b[1] = static_cast<const uint8_t*>(w.up_bias);
  }
  g.out = H;
  g.err = err;
  g.E = D.E;
  g.N = D.F;
  g.rstride = D.fused ? 2 * D.F : D.F;
  hipError_t e = launch_stream<true>(D.d, g, s);
  if (e != hipSuccess) return e;
  if (mid != nullptr && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
  U4Args h{};
  h.offsets = offsets;
  h.sorted_token = nullptr;
  h.a = static_cast<const uint16_t*>(H);
  h.q[0] = h.q[1] = static_cast<const uint8_t*>(w.down);
  h.s[0] = h.s[1] = static_cast<const uint8_t*>(w.down_scale);
  h.b[0] = h.b[1] = static_cast<const uint8_t*>(w.down_bias);
  h.out = Y;
  h.E = D.E;
  h.N = D.d;
  h.rstride = D.d;
  h.row_scale = row_scale;
  return launch_stream<false>(D.F, h, s);
}

}  // namespace moe
