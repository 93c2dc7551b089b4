// Grouped expert FFN with 4-bit affine routed weights (Edge0 "MoE Spec and
// Routing" page, QuantSpec: bits 4, group 64, mode affine; w = scale*q +
// bias), bf16 activations, fp32 accumulation.
//
// Built for decode-shaped batches, where each touched expert sees a handful
// of rows and the layer is bound by streaming the packed weights from HBM:
// every weight byte is read once and used for all of the expert's rows.
// The affine dequantisation is factored per group so no dequantised weight
// is formed:
//   sum_j x_j (s q_j + b) = s * sum_j x_j q_j + b * sum_j x_j
// over the 32-element run a lane owns (always inside one group of 64), and
// the codes enter v_dot2_f32_f16 as exact fp16 values (1024 + q or
// 1024 + 16q), two per instruction, against the lane's activations
// pre-packed as fp16 pairs.
//
// One kernel serves both products:
//   up   : unit = hidden column f; the gate row f and the up row f, the
//          epilogue writes H = silu(gate) * up (fp16, as on the
//          matrix-core path)
//   down : unit = output column n of W_down, writes Y (fp32)
// LPR = K/32 lanes share one unit; a wave-wide 16-byte load covers 64/LPR
// units, and the lane groups reduce their partial sums together.
#include <type_traits>

#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kMaxK = 2048;  // one pass of 64 lanes x 32 elements per row

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// The value of this lane's partner at distance D (a power of two up to 32):
// partners differ in bit D of the lane index and possibly in lower bits.
// D <= 8 are DPP moves inside rows of 16 lanes (the two xor pairings of a
// quad, then the mirrors of 8 and 16 lanes), 16 and 32 the gfx950 row
// swaps; none goes through LDS.
template <int D>
__device__ __forceinline__ float pair_move(float v, int lane) {
  if constexpr (D == 1) {
    return dpp_f<kDppXor1>(v);
  } else if constexpr (D == 2) {
    return dpp_f<kDppXor2>(v);
  } else if constexpr (D == 4) {
    return dpp_f<kDppHalfMirror>(v);
  } else if constexpr (D == 8) {
    return dpp_f<kDppMirror>(v);
  } else if constexpr (D == 16) {
    // odd rows of the first result hold the even rows, and the other way
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else {
    static_assert(D == 32, "distance");
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  }
}

// In-place reduction of V per-lane values over each group of LPR lanes
// (LPR and V powers of two).  Butterfly with halving: at distance D the
// lane with bit D set keeps the upper half of its values and sends the
// lower half, so each exchange carries half of the values and V values cost
// about V moves in all instead of V*log2(LPR).  Any partner that differs in
// bit D (and possibly lower bits) holds the same index subset at that step,
// so the pair_move pairings serve as well as xor.  On return a lane holds
// C = max(1, V/LPR) totals in v[0..C): those of indices
// reduce_index(lane, j), identical on lanes that differ only below the
// last halving distance.
template <int D, int CNT, int V>
__device__ __forceinline__ void reduce_step(float (&v)[V], int lane) {
  if constexpr (D >= 1) {
    if constexpr (CNT > 1) {
      constexpr int kHalf = CNT / 2;
      const bool upper = (lane & D) != 0;
#pragma unroll
      for (int i = 0; i < kHalf; ++i) {
        const float send = upper ? v[i] : v[i + kHalf];
        const float keep = upper ? v[i + kHalf] : v[i];
        v[i] = keep + pair_move<D>(send, lane);
      }
      reduce_step<D / 2, kHalf, V>(v, lane);
    } else {
      v[0] += pair_move<D>(v[0], lane);
      reduce_step<D / 2, 1, V>(v, lane);
    }
  }
}

template <int V, int LPR>
__device__ __forceinline__ void multi_reduce(float (&v)[V], int lane) {
  reduce_step<LPR / 2, V, V>(v, lane);
}

// index of v[j] after multi_reduce<V, LPR> on this lane
template <int V, int LPR>
__device__ __forceinline__ int reduce_index(int lane, int j) {
  int idx = j, c = V;
#pragma unroll
  for (int d = LPR / 2; d >= 1 && c > 1; d >>= 1) {
    c /= 2;
    if (lane & d) idx += c;
  }
  return idx;
}

// lowest lane distance at which multi_reduce<V, LPR> still halves
template <int V, int LPR>
constexpr int last_halving_distance() {
  int c = V, last = LPR;
  for (int d = LPR / 2; d >= 1 && c > 1; d >>= 1) {
    c /= 2;
    last = d;
  }
  return last;
}

// lanes per unit: each lane owns 32 elements of K, so LPR = K/32 (K is a
// power of two from 64 to 2048)
int pick_lpr(int K) {
  int l = 64;
  while (l > 1 && K % (32 * l) != 0) l >>= 1;
  return l;
}

// ---------------------------------------------------------------- streaming
// The packed weights stream through LDS.  Work is cut into items: one row
// chunk (up to kRows of the expert's rows) against kSub wave-wide 16-byte
// loads per matrix, i.e. kSub * (64/LPR) consecutive units of one expert
// (kSub KiB of codes per matrix) plus their scales and biases (64 kSub
// bytes each).  The active
// experts are listed on the device and their items numbered (expert, row
// chunk, unit block) with the unit block fastest; every wave of a persistent
// grid takes one contiguous range of items of equal cost, an item of r rows
// costing kItemCost + r (its loads and unpacking, then r rows of dot
// products), so a wave on a busy expert takes fewer items.  An expert with
// more than kRows rows streams its weights once per chunk.  A wave is an independent pipeline over a private ring of NS
// stages in LDS: the direct-to-LDS loads of the item NS-1 ahead are issued
// before the current item is computed, so NS-1 items per wave are always in
// flight, and the only wait is the wave's own vmcnt.  The buffer descriptors
// carry each expert matrix's size, so a load past the last unit fetches
// nothing.
constexpr int kItemCost = 2;     // cost of an item beyond its rows, in rows
constexpr int kMaxExperts = 1024;
constexpr int kMaxChunkRows = 4;

// Per product: waves per workgroup (one workgroup per CU), wave-wide 16-byte
// loads per matrix and item, rows per chunk (held in registers) and stages
// per wave.  Both keep 144 KiB of LDS in the ring.  Measured on the decode
// layer (256 experts, top-8, 32 tokens): 16 waves with 2-row chunks keep the
// registers under 128 (4 waves per SIMD) and beat 8 waves with 4-row
// chunks by a third; 1-row chunks lose what they save in registers to
// unpacking the codes once per row.
template <bool PAIR>
struct SCfg {
  static constexpr int kWaves = 16;
  static constexpr int kSub = 2;
  static constexpr int kRows = 2;
  static constexpr int kStages = PAIR ? 2 : 4;
  static constexpr int M = PAIR ? 2 : 1;
  static constexpr int kCode = kSub * 1024;  // codes of one matrix
  static constexpr int kSB = kSub * 64;      // scales (or biases) of one matrix
  static constexpr int kSBLanes = kSB / 4;   // lanes of its 4-byte load
  static constexpr int kBytes = M * kCode + 2 * M * kSB;  // one stage
  static constexpr int kLoads = M * kSub + 2 * M;  // load instructions per item
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kPasses = (kMaxExperts + kThreads - 1) / kThreads;
  static constexpr int kLds =
      kWaves * kStages * kBytes + (3 * kMaxExperts + 2) * 4 + 3 * kPasses * kWaves * 4;
  static_assert(kRows <= kMaxChunkRows && kLds <= 160 * 1024, "stream layout");
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

// wait until at most N vector-memory operations of this wave are pending
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

// (a & m) | c in one instruction (the masks would otherwise cost an AND and
// an OR each: a VOP3 instruction takes no literal here)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "s"(c));
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
  c[0] = __builtin_bit_cast(half2_t, and_or(w, m_lo, 0x64006400u));
  c[1] = __builtin_bit_cast(half2_t, and_or(w, m_hi, 0x64006400u));
  c[2] = __builtin_bit_cast(half2_t, and_or(h, m_lo, 0x64006400u));
  c[3] = __builtin_bit_cast(half2_t, and_or(h, m_hi, 0x64006400u));
}

// One lane's 32 activations of a row as fp16 pairs xp[4m + j] = (x_{8m+j},
// x_{8m+j+4}) matching unpack8, with the fp32 sums over all 32 (xs) and
// over the pairs j = 1, 3 (s13).
template <bool BF16>
__device__ __forceinline__ void load_row(const uint16_t* p, half2_t* xp, float& xs,
                                         float& s13) {
  xs = 0.f;
  s13 = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint4 t = *reinterpret_cast<const uint4*>(p + 8 * m);
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
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half2_t v;
      v[0] = h[j];
      v[1] = h[j + 4];
      xp[m * 4 + j] = v;
      const float pair = static_cast<float>(h[j]) + static_cast<float>(h[j + 4]);
      xs += pair;
      if (j & 1) s13 += pair;
    }
  }
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
};

// exclusive prefix over the lanes of a wave, and the wave total
__device__ __forceinline__ int wave_prefix(int v, int lane, int& total) {
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  total = __shfl(inc, 63, 64);
  return inc - v;
}

template <bool PAIR, int LPR>
__device__ __forceinline__ void u4_stream(const U4Args& g, uint8_t* smem) {
  using SL = SCfg<PAIR>;
  constexpr int kRows = SL::kRows;
  constexpr int kSWaves = SL::kWaves;
  constexpr int kSUB = SL::kSub;
  constexpr int K = 32 * LPR;
  constexpr int UPW = 64 / LPR;        // units per wave-wide load
  constexpr int UPI = kSUB * UPW;      // units per item
  constexpr int G = K / 64;            // quantisation groups per row
  constexpr int NS = SL::kStages;
  constexpr int M = SL::M;
  constexpr int L = SL::kLoads;

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
      const uint32_t vq = static_cast<uint32_t>(u0 * (K / 2) + lane * 16);
#pragma unroll
      for (int j = 0; j < kSUB; ++j) dma16(rq, st + m * SL::kCode + j * 1024, vq + j * 1024);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t vs = static_cast<uint32_t>(u0 * G * 2 + lane * 4);
      const rsrc_t rs = make_rsrc(g.s[m] + erow * (G * 2), g.N * G * 2);
      const rsrc_t rb = make_rsrc(g.b[m] + erow * (G * 2), g.N * G * 2);
      // the item's scales (biases) are kSB contiguous bytes
      if (SL::kSBLanes >= 64 || lane < SL::kSBLanes) {
        dma4(rs, st + M * SL::kCode + (2 * m) * SL::kSB, vs);
        dma4(rb, st + M * SL::kCode + (2 * m + 1) * SL::kSB, vs);
      }
    }
  };

  // the chunk's activation rows, held in registers
  const int kl = lane % LPR;
  const int sg = lane / LPR;
  const uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u;
  half2_t xp[kRows][16];
  float xs[kRows], xc[kRows];
  auto load_rows = [&](int row0, int rows) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      if (r < rows) {
        const int32_t kr = row0 + r;
        const int64_t src = g.sorted_token ? static_cast<int64_t>(g.sorted_token[kr])
                                           : static_cast<int64_t>(kr);
        float s13;
        load_row<PAIR>(g.a + src * K + 32 * kl, xp[r], xs[r], s13);
        // offsets carried by the codes: 1024 per element of the pairs
        // j = 0, 2 and 64 (1024/16) per element of the pairs j = 1, 3
        xc[r] = 1024.f * xs[r] - 960.f * s13;
      }
    }
  };

  // R rows (register slots 0..R-1, kept rows row0..) against the codes in
  // stage st
  auto rows_pass = [&](auto RC, const uint8_t* st, int row0, int u0) {
    constexpr int R = decltype(RC)::value;
    constexpr int V = kSUB * R * M;
    float v[V];
#pragma unroll
    for (int j = 0; j < kSUB; ++j) {
      const int ul = j * UPW + sg;  // unit inside the item
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint4 w = *reinterpret_cast<const uint4*>(st + m * SL::kCode + j * 1024 + lane * 16);
        const uint16_t* sb = reinterpret_cast<const uint16_t*>(st + M * SL::kCode);
        const float sc = bf16_to_f32(sb[(2 * m) * (SL::kSB / 2) + ul * G + kl / 2]);
        const float bi = bf16_to_f32(sb[(2 * m + 1) * (SL::kSB / 2) + ul * G + kl / 2]);
        half2_t c[4][4];
        unpack8(w.x, m_lo, m_hi, c[0]);
        unpack8(w.y, m_lo, m_hi, c[1]);
        unpack8(w.z, m_lo, m_hi, c[2]);
        unpack8(w.w, m_lo, m_hi, c[3]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float a0 = 0.f, a1 = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            a0 = __builtin_amdgcn_fdot2(c[q][0], xp[r][4 * q + 0], a0, false);
            a1 = __builtin_amdgcn_fdot2(c[q][1], xp[r][4 * q + 1], a1, false);
            a0 = __builtin_amdgcn_fdot2(c[q][2], xp[r][4 * q + 2], a0, false);
            a1 = __builtin_amdgcn_fdot2(c[q][3], xp[r][4 * q + 3], a1, false);
          }
          const float dm = fmaf(a1, 0.0625f, a0);  // sum x (offset + q)
          v[(j * R + r) * M + m] = fmaf(sc, dm - xc[r], bi * xs[r]);
        }
      }
    }
    multi_reduce<V, LPR>(v, lane);
    constexpr int CT = V / LPR > 1 ? V / LPR : 1;
    // gate and up of one (unit, row) sit side by side when a lane keeps
    // several totals, else in the lanes one last-halving distance apart
    constexpr int kPartner = last_halving_distance<V, LPR>();
    const bool writer = (lane & (kPartner - 1)) == 0;
#pragma unroll
    for (int j = 0; j < CT; ++j) {
      float gv = v[j], upv = 0.f;
      const int idx = reduce_index<V, LPR>(lane, j);
      if (PAIR) {
        if (CT > 1) {
          if (j % 2 == 1) continue;
          upv = v[j + 1];
        } else {
          upv = pair_move<kPartner>(v[0], lane);
          if (idx % 2 == 1) continue;
        }
      }
      const int jl = idx / (R * M);
      const int r = (idx / M) % R;
      const int u = u0 + jl * UPW + sg;
      if (!writer || u >= g.N) continue;
      const int64_t o = static_cast<int64_t>(row0 + r) * g.N + u;
      if (PAIR) {  // hidden activation, fp16 (saturating)
        float h = gv / (1.f + __expf(-gv)) * upv;
        h = fminf(fmaxf(h, -65504.f), 65504.f);
        static_cast<_Float16*>(g.out)[o] = static_cast<_Float16>(h);
      } else {  // expert output, fp32
        static_cast<float*>(g.out)[o] = gv;
      }
    }
  };

  int cache_e = -1, cache_k = -1;
  for (int t = 0; t < NS - 1 && t < n; ++t) issue(t);
  for (int t = 0; t < n; ++t) {
    if (t + NS - 1 < n) issue(t + NS - 1);  // into the stage freed by item t-1
    wait_later<L, NS>(min(NS - 1, n - 1 - t));
    const int a = ca, k = ck;
    const int u0 = cb * UPI;
    advance(ca, ck, cb);
    const int e = __builtin_amdgcn_readfirstlane(act_e[a]);
    const int row0 = __builtin_amdgcn_readfirstlane(g.offsets[e]) + k * kRows;
    const int rows = min(kRows, __builtin_amdgcn_readfirstlane(g.offsets[e + 1]) - row0);
    if (cache_e != e || cache_k != k) {
      load_rows(row0, rows);
      cache_e = e;
      cache_k = k;
    }
    const uint8_t* st = ring + (t % NS) * SL::kBytes;
    if (kRows == 4 && rows == 4) {
      rows_pass(std::integral_constant<int, kRows>(), st, row0, u0);
    } else if (kRows == 4 && rows == 3) {
      // rows 0-1 as a pair, then row 2 alone (moved to slot 0)
      rows_pass(std::integral_constant<int, 2>(), st, row0, u0);
#pragma unroll
      for (int q = 0; q < 16; ++q) xp[0][q] = xp[2][q];
      xs[0] = xs[2];
      xc[0] = xc[2];
      rows_pass(std::integral_constant<int, 1>(), st, row0 + 2, u0);
      cache_e = -1;  // slot 0 no longer holds the chunk's first row
    } else if (rows == 2) {
      rows_pass(std::integral_constant<int, 2>(), st, row0, u0);
    } else {
      rows_pass(std::integral_constant<int, 1>(), st, row0, u0);
    }
  }
}

#define MOE_U4S_KERNEL(P, LPR)                                                  \
  __global__ void __launch_bounds__(SCfg<P>::kThreads)                       \
      u4s_kernel_##P##_##LPR(U4Args g) {                                      \
    __shared__ __attribute__((aligned(16))) uint8_t smem[SCfg<P>::kLds];      \
    u4_stream<P, LPR>(g, smem);                                               \
  }
MOE_U4S_KERNEL(true, 64)
MOE_U4S_KERNEL(true, 32)
MOE_U4S_KERNEL(true, 16)
MOE_U4S_KERNEL(true, 8)
MOE_U4S_KERNEL(true, 4)
MOE_U4S_KERNEL(true, 2)
MOE_U4S_KERNEL(false, 64)
MOE_U4S_KERNEL(false, 32)
MOE_U4S_KERNEL(false, 16)
MOE_U4S_KERNEL(false, 8)
MOE_U4S_KERNEL(false, 4)
MOE_U4S_KERNEL(false, 2)
#undef MOE_U4S_KERNEL

int stream_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  return cus;
}

template <bool PAIR>
hipError_t launch_stream(int K, const U4Args& g, hipStream_t s) {
  const dim3 grid(stream_grid()), block(SCfg<PAIR>::kThreads);
#define MOE_U4S(L)                                                                   \
  case L:                                                                            \
    hipLaunchKernelGGL(PAIR ? u4s_kernel_true_##L : u4s_kernel_false_##L, grid, block, \
                       0, s, g);                                                     \
    break;
  switch (pick_lpr(K)) {
    MOE_U4S(64)
    MOE_U4S(32)
    MOE_U4S(16)
    MOE_U4S(8)
    MOE_U4S(4)
    MOE_U4S(2)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_U4S
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_u4(const Dims& D, int group, const int32_t* offsets,
                         const int32_t* sorted_token, const void* x,
                         const moe_expert_weights& w, void* H, void* Y,
                         hipStream_t s) {
  if (D.d > kMaxK || D.F > kMaxK || !D.swiglu || group != 64 || D.E > kMaxExperts ||
      D.d != 32 * pick_lpr(D.d) || D.F != 32 * pick_lpr(D.F))
    return hipErrorInvalidValue;
  // item numbers and item costs are 32-bit: row chunks (at most T*k/4 + E)
  // times unit blocks per expert, times the cost of an item
  const int64_t chunks = D.slots / std::min(SCfg<true>::kRows, SCfg<false>::kRows) + D.E;
  // unit blocks are >= kSub units
  const int64_t blocks =
      std::max(D.F, D.d) / std::min(SCfg<true>::kSub, SCfg<false>::kSub) + 1;
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
  g.E = D.E;
  g.N = D.F;
  g.rstride = D.fused ? 2 * D.F : D.F;
  hipError_t err = launch_stream<true>(D.d, g, s);
  if (err != hipSuccess) return err;
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
  return launch_stream<false>(D.F, h, s);
}

}  // namespace moe
