// Grouped expert FFN with 4-bit affine routed weights (Edge0 "MoE Spec and
// Routing" page, QuantSpec: bits 4, group 64, mode affine; w = scale*q +
// bias), bf16 activations, fp32 accumulation.
//
// Built for decode-shaped batches, where each touched expert sees a handful
// of rows and the layer is bound by streaming the packed weights from HBM:
// every weight byte is read once, 16 bytes per lane, and reused from
// registers for all of the expert's rows.  The affine
// dequantisation is factored per group so no dequantised weight is formed:
//   sum_j x_j (s q_j + b) = s * sum_j x_j q_j + b * sum_j x_j
// over the 32-element run a lane owns (always inside one group of 64), and
// the codes enter v_dot2_f32_f16 as the exact fp16 values 1024 + q, two per
// instruction, against the lane's activations pre-packed as fp16 pairs.
//
// One kernel serves both products:
//   up   : unit = hidden column f; the lane loads the gate row f and the up
//          row f, the epilogue writes H = silu(gate) * up (fp16, as on the
//          matrix-core path)
//   down : unit = output column n of W_down, writes Y (fp32)
// LPR lanes share one unit and each lane streams one 16-byte vector of it
// per pass; a wave works on 64/LPR units at once and reduces inside each
// lane group.
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kMaxK = 2048;  // one pass of 64 lanes x 32 elements per row

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Codes as fp16: OR-ing a code q (0..15) into the mantissa of 1024.0
// (0x6400) gives exactly 1024 + q, two codes per 32-bit word.  Word w holds
// elements 0..7 in nibbles 0..7, so (w >> 4j) & 0x000F000F carries elements
// j and j+4 into the two halves.
__device__ __forceinline__ half2_t code_pair(uint32_t w, int j) {
  return __builtin_bit_cast(half2_t, ((w >> (4 * j)) & 0x000F000Fu) | 0x64006400u);
}

// sum over one lane's 32 elements of x_i * (1024 + q_i), two products per
// v_dot2 (fp16 products are exact in fp32); xp[m*4 + j] = (x_{8m+j},
// x_{8m+j+4})
__device__ __forceinline__ float dot32(const uint4& w, const half2_t* xp) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_fdot2(code_pair(ws[m], j), xp[m * 4 + j], acc, false);
  return acc;
}

// sum over one lane's 32 elements of x_i * (1024 + q_i) for R rows at once,
// each code pair unpacked once: out[r * stride] for row r
template <int R>
__device__ __forceinline__ void dots(const uint4& w, const half2_t (*xp)[16], float* out,
                                     int stride) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half2_t cp = code_pair(ws[m], j);
#pragma unroll
      for (int r = 0; r < R; ++r)
        acc[r] = __builtin_amdgcn_fdot2(cp, xp[r][m * 4 + j], acc[r], false);
    }
#pragma unroll
  for (int r = 0; r < R; ++r) out[r * stride] = acc[r];
}

// a lane's 32 activation values of one row (bf16 tokens or fp16 hidden
// rows) as fp16 pairs matching code_pair, and their fp32 sum
template <bool BF16>
__device__ __forceinline__ float load_pairs(const uint16_t* p, half2_t* xp) {
  float sum = 0.f;
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
      sum += static_cast<float>(h[j]) + static_cast<float>(h[j + 4]);
    }
  }
  return sum;
}

// In-place reduction of V per-lane values over each group of LPR lanes
// (LPR and V powers of two).  Butterfly with halving: at distance D the
// lane with bit D set keeps the upper half of its values and sends the
// lower half, so each exchange carries half of the values and V values cost
// about V shuffles in all instead of V*log2(LPR).  On return a lane holds
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
        v[i] = keep + __shfl_xor(send, D, 64);
      }
      reduce_step<D / 2, kHalf, V>(v, lane);
    } else {
      v[0] += __shfl_xor(v[0], D, 64);
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

// Decode-shaped grouped expert FFN, one workgroup per (expert, block of
// units).  Each wave owns UB * (64/LPR) consecutive units; LPR lanes share a
// unit and each lane owns 32 consecutive K elements (inside one
// quantisation group).  All of a wave's packed weights (UB 16-byte loads
// per matrix) and their scales and biases are requested before any
// arithmetic, so a wave keeps 16 B x UB x (1 or 2) per lane in flight; the
// expert's rows are then taken one at a time (each lane reads its own 32
// elements of the row) against the weights held in registers, and the
// per-lane partial sums of every unit and matrix are reduced together by
// multi_reduce.
template <bool PAIR, int LPR, int UB>
__global__ void __launch_bounds__(256)
u4_kernel(const int32_t* __restrict__ offsets,
          const int32_t* __restrict__ sorted_token,  // nullptr: a rows direct
          const uint16_t* __restrict__ a,             // [.., K] bf16 x or fp16 H
          const uint32_t* __restrict__ q0,            // [E][N][K/8]
          const uint16_t* __restrict__ s0,            // [E][N][K/64]
          const uint16_t* __restrict__ b0,
          const uint32_t* __restrict__ q1,            // up (PAIR)
          const uint16_t* __restrict__ s1,
          const uint16_t* __restrict__ b1,
          void* __restrict__ out, int N, int rstride) {
  constexpr int K = 32 * LPR;
  constexpr int UPW = 64 / LPR;     // units per wave-wide load
  constexpr int UPWB = UB * UPW;    // units per wave
  constexpr int UPB = 4 * UPWB;     // units per workgroup
  constexpr int RP = 1;
  constexpr int M = PAIR ? 2 : 1;   // matrices
  constexpr int V = UB * RP * M;    // partial sums per lane and pass
  constexpr int C = V / LPR > 1 ? V / LPR : 1;
  const int e = blockIdx.x;
  const int32_t row0 = offsets[e];
  const int cnt = offsets[e + 1] - row0;
  if (cnt <= 0) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sg = lane / LPR, kl = lane % LPR;
  const int ubase = blockIdx.y * UPB + wave * UPWB;
  constexpr int words = K / 8, groups = K / 64;
  const int gi = kl / 2;  // this lane's quantisation group

  // ---- all weight requests of the wave first
  uint4 w0[UB], w1[UB];
  float sc0[UB], bi0[UB], sc1[UB], bi1[UB];
#pragma unroll
  for (int i = 0; i < UB; ++i) {
    const int u = min(ubase + i * UPW + sg, N - 1);
    // rstride: rows from one expert's matrix to the next (N; 2N when gate
    // and up are fused)
    const int64_t wrow = static_cast<int64_t>(e) * rstride + u;
    w0[i] = *reinterpret_cast<const uint4*>(q0 + wrow * words + 4 * kl);
    sc0[i] = bf16_to_f32(s0[wrow * groups + gi]);
    bi0[i] = bf16_to_f32(b0[wrow * groups + gi]);
    if (PAIR) {
      w1[i] = *reinterpret_cast<const uint4*>(q1 + wrow * words + 4 * kl);
      sc1[i] = bf16_to_f32(s1[wrow * groups + gi]);
      bi1[i] = bf16_to_f32(b1[wrow * groups + gi]);
    }
  }

  // the expert's rows, RP at a time: each lane reads its own 32 elements of
  // a row straight from memory (the row index is uniform, so it comes in
  // through the scalar cache)
  for (int rp = 0; rp < cnt; rp += RP) {
    {
      half2_t xp[RP][16];
      float xsum[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const int rr = min(rp + r, cnt - 1);
        const int64_t src = sorted_token ? sorted_token[row0 + rr]
                                         : static_cast<int64_t>(row0 + rr);
        xsum[r] = load_pairs<PAIR>(a + src * K + 32 * kl, xp[r]);
      }
      // v[(i*RP + r)*M + m]
      float v[V];
#pragma unroll
      for (int i = 0; i < UB; ++i) {
        // one unit at a time: its codes are unpacked once for all rows
        dots<RP>(w0[i], xp, &v[i * RP * M], M);
        if (PAIR) dots<RP>(w1[i], xp, &v[i * RP * M + 1], M);
#pragma unroll
        for (int r = 0; r < RP; ++r) {
          v[(i * RP + r) * M] = sc0[i] * (v[(i * RP + r) * M] - 1024.f * xsum[r]) +
                                bi0[i] * xsum[r];
          if (PAIR)
            v[(i * RP + r) * M + 1] =
                sc1[i] * (v[(i * RP + r) * M + 1] - 1024.f * xsum[r]) + bi1[i] * xsum[r];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      multi_reduce<V, LPR>(v, lane);
      // with several totals per lane, the gate and up of one (unit, row)
      // sit side by side; with one, in the lanes one last-halving distance
      // apart
      constexpr int kPartner = last_halving_distance<V, LPR>();
      // lanes below the last halving distance hold copies: the one with
      // those bits clear writes
      const bool writer = (lane & (kPartner - 1)) == 0;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        float g = v[j], upv = 0.f;
        int idx = reduce_index<V, LPR>(lane, j);
        if (PAIR) {
          if (C > 1) {
            if (j % 2 == 1) continue;
            upv = v[j + 1];
          } else {
            upv = __shfl_xor(v[0], kPartner, 64);
            if (idx % 2 == 1) continue;
          }
        }
        const int unit_i = idx / (RP * M);
        const int r = (idx / M) % RP;
        if (!writer || rp + r >= cnt) continue;
        const int u = ubase + unit_i * UPW + sg;
        if (u >= N) continue;
        const int64_t o = static_cast<int64_t>(row0 + rp + r) * N + u;
        if (PAIR) {  // hidden activation, fp16 (saturating)
          float h = g / (1.f + __expf(-g)) * upv;
          h = fminf(fmaxf(h, -65504.f), 65504.f);
          static_cast<_Float16*>(out)[o] = static_cast<_Float16>(h);
        } else {  // expert output, fp32
          static_cast<float*>(out)[o] = g;
        }
      }
    }
  }
}

// lanes per unit: each lane owns 32 elements of K, so LPR = K/32 (K is a
// power of two from 64 to 2048)
int pick_lpr(int K) {
  int l = 64;
  while (l > 1 && K % (32 * l) != 0) l >>= 1;
  return l;
}

constexpr int kUB = 4;  // wave-wide weight loads per matrix in flight

template <bool PAIR, int LPR>
int units_per_block() { return 4 * kUB * (64 / LPR); }

template <bool PAIR>
hipError_t launch_u4(int K, int E, int N, int rstride, hipStream_t s,
                     const int32_t* offsets,
                     const int32_t* st, const uint16_t* a, const uint32_t* q0,
                     const uint16_t* s0, const uint16_t* b0, const uint32_t* q1,
                     const uint16_t* s1, const uint16_t* b1, void* out) {
#define MOE_U4(L)                                                                  \
  {                                                                                \
    const int upb = 4 * kUB * (64 / L);                                            \
    const dim3 grid(E, (N + upb - 1) / upb);                                       \
    hipLaunchKernelGGL((u4_kernel<PAIR, L, kUB>), grid, dim3(256), 0, s, offsets,  \
                       st, a, q0, s0, b0, q1, s1, b1, out, N, rstride);            \
    break;                                                                         \
  }
  switch (pick_lpr(K)) {
    case 64: MOE_U4(64)
    case 32: MOE_U4(32)
    case 16: MOE_U4(16)
    case 8: MOE_U4(8)
    case 4: MOE_U4(4)
    default: MOE_U4(2)
  }
#undef MOE_U4
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_u4(const Dims& D, int group, const int32_t* offsets,
                         const int32_t* sorted_token, const void* x,
                         const moe_expert_weights& w, void* H, void* Y,
                         hipStream_t s) {
  if (D.d > kMaxK || D.F > kMaxK || !D.swiglu || group != 64 ||
      D.d != 32 * pick_lpr(D.d) || D.F != 32 * pick_lpr(D.F))
    return hipErrorInvalidValue;
  const uint32_t* qg = static_cast<const uint32_t*>(w.gate);
  const uint16_t* sg = static_cast<const uint16_t*>(w.gate_scale);
  const uint16_t* bg = static_cast<const uint16_t*>(w.gate_bias);
  const uint32_t* qu = static_cast<const uint32_t*>(w.up);
  const uint16_t* su = static_cast<const uint16_t*>(w.up_scale);
  const uint16_t* bu = static_cast<const uint16_t*>(w.up_bias);
  if (D.fused) {  // each expert's F gate rows, then its F up rows
    qu = qg + static_cast<int64_t>(D.F) * (D.d / 8);
    su = sg + static_cast<int64_t>(D.F) * (D.d / group);
    bu = bg + static_cast<int64_t>(D.F) * (D.d / group);
  }
  hipError_t err = launch_u4<true>(D.d, D.E, D.F, D.fused ? 2 * D.F : D.F, s, offsets,
                                   sorted_token, static_cast<const uint16_t*>(x), qg,
                                   sg, bg, qu, su, bu, H);
  if (err != hipSuccess) return err;
  return launch_u4<false>(
      D.F, D.E, D.d, D.d, s, offsets, nullptr, static_cast<const uint16_t*>(H),
      static_cast<const uint32_t*>(w.down), static_cast<const uint16_t*>(w.down_scale),
      static_cast<const uint16_t*>(w.down_bias), nullptr, nullptr, nullptr, Y);
}

}  // namespace moe
