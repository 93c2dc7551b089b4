// Grouped expert FFN with 4-bit affine routed weights (Edge0 "MoE Spec and
// Routing" page, QuantSpec: bits 4, group 64, mode affine; w = scale*q +
// bias), bf16 activations, fp32 accumulation.
//
// Built for decode-shaped batches, where each touched expert sees a handful
// of rows and the layer is bound by streaming the packed weights from HBM:
// every weight byte is read once, 16 bytes per lane, and reused from
// registers for all of the expert's rows, which sit in LDS.  The affine
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

constexpr int kRC = 8;            // expert rows staged in LDS per pass
constexpr int kUnitsPerBlock = 64;
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

// a lane's 32 activation values of one row (bf16 tokens or fp16 hidden
// rows, from LDS) as fp16 pairs matching code_pair, and their fp32 sum
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

constexpr int kRowsPerPass = 2;  // expert rows multiplied per weight pass

// One lane owns 32 consecutive K elements (inside one quantisation group);
// LPR = lanes per unit.  sum_i x_i (s q_i + b) = s (sum x_i (1024 + q_i)
// - 1024 sum x_i) + b sum x_i.
template <bool PAIR, int LPR>
__global__ void __launch_bounds__(256)
u4_kernel(const int32_t* __restrict__ offsets,
          const int32_t* __restrict__ sorted_token,  // nullptr: a rows direct
          const uint16_t* __restrict__ a,             // [.., K] bf16 x or fp16 H
          const uint32_t* __restrict__ q0,            // [E][N][K/8]
          const uint16_t* __restrict__ s0,            // [E][N][K/G]
          const uint16_t* __restrict__ b0,
          const uint32_t* __restrict__ q1,            // up (PAIR)
          const uint16_t* __restrict__ s1,
          const uint16_t* __restrict__ b1,
          void* __restrict__ out, int N, int K, int G) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [kRC][K]
  const int e = blockIdx.x;
  const int32_t row0 = offsets[e];
  const int cnt = offsets[e + 1] - row0;
  if (cnt <= 0) return;
  const int u_base = blockIdx.y * kUnitsPerBlock;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int UPW = 64 / LPR;  // units per wave pass
  const int sg = lane / LPR, kl = lane % LPR;
  const int words = K / 8, groups = K / G;

  for (int rc0 = 0; rc0 < cnt; rc0 += kRC) {
    const int nr = min(kRC, cnt - rc0);
    __syncthreads();
    // stage the rows [rc0, rc0+nr) in LDS, 16 bytes per thread
    const int vec_per_row = K / 8;
    for (int i = threadIdx.x; i < nr * vec_per_row; i += blockDim.x) {
      const int r = i / vec_per_row, c = i % vec_per_row;
      const int64_t src = sorted_token ? sorted_token[row0 + rc0 + r]
                                       : static_cast<int64_t>(row0 + rc0 + r);
      reinterpret_cast<uint4*>(xs)[static_cast<int64_t>(r) * vec_per_row + c] =
          reinterpret_cast<const uint4*>(a + src * K)[c];
    }
    __syncthreads();
    // K <= 32 * LPR (the launcher checks), so this runs once
#pragma unroll 1
    for (int kc = 0; kc < K; kc += 32 * LPR) {
      const int kb = kc + 32 * kl;  // first element owned by this lane
      const int gi = kb / G;
#pragma unroll 1
      for (int rp = 0; rp < nr; rp += kRowsPerPass) {
        half2_t xp[kRowsPerPass][16];
        float xsum[kRowsPerPass];
#pragma unroll
        for (int r = 0; r < kRowsPerPass; ++r)
          xsum[r] = (rp + r < nr)
                        ? load_pairs<PAIR>(xs + static_cast<int64_t>(rp + r) * K + kb, xp[r])
                        : 0.f;
#pragma unroll 4
        for (int ub = wave * UPW; ub < kUnitsPerBlock; ub += 4 * UPW) {
          const int u = u_base + ub + sg;
          const bool live = u < N;
          const int uu = live ? u : N - 1;
          const int64_t wrow = static_cast<int64_t>(e) * N + uu;
          const uint4 w0 = *reinterpret_cast<const uint4*>(q0 + wrow * words + kb / 8);
          uint4 w1 = make_uint4(0, 0, 0, 0);
          if (PAIR) w1 = *reinterpret_cast<const uint4*>(q1 + wrow * words + kb / 8);
          const float sc0 = bf16_to_f32(s0[wrow * groups + gi]);
          const float bi0 = bf16_to_f32(b0[wrow * groups + gi]);
          float sc1 = 0.f, bi1 = 0.f;
          if (PAIR) {
            sc1 = bf16_to_f32(s1[wrow * groups + gi]);
            bi1 = bf16_to_f32(b1[wrow * groups + gi]);
          }
          float acc0[kRowsPerPass], acc1[kRowsPerPass];
#pragma unroll
          for (int r = 0; r < kRowsPerPass; ++r) {
            const float d0 = dot32(w0, xp[r]) - 1024.f * xsum[r];
            acc0[r] = sc0 * d0 + bi0 * xsum[r];
            if (PAIR) {
              const float d1 = dot32(w1, xp[r]) - 1024.f * xsum[r];
              acc1[r] = sc1 * d1 + bi1 * xsum[r];
            }
#pragma unroll
            for (int o = LPR / 2; o > 0; o >>= 1) {
              acc0[r] += __shfl_xor(acc0[r], o, 64);
              if (PAIR) acc1[r] += __shfl_xor(acc1[r], o, 64);
            }
          }
          if (kl == 0 && live) {
#pragma unroll
            for (int r = 0; r < kRowsPerPass; ++r) {
              if (rp + r >= nr) break;
              const int64_t o = static_cast<int64_t>(row0 + rc0 + rp + r) * N + u;
              if (PAIR) {  // hidden activation, fp16 (saturating)
                float h = acc0[r] / (1.f + __expf(-acc0[r])) * acc1[r];
                h = fminf(fmaxf(h, -65504.f), 65504.f);
                static_cast<_Float16*>(out)[o] = static_cast<_Float16>(h);
              } else {  // expert output, fp32
                static_cast<float*>(out)[o] = acc0[r];
              }
            }
          }
        }
      }
    }
  }
}

// lanes per unit: each lane owns 32 elements of K, so LPR = K/32 (K is a
// multiple of 64 and at most 2048)
int pick_lpr(int K) {
  int l = 64;
  while (l > 1 && K % (32 * l) != 0) l >>= 1;
  return l;
}

template <bool PAIR>
hipError_t launch_u4(int K, dim3 grid, size_t lds, hipStream_t s,
                     const int32_t* offsets, const int32_t* st,
                     const uint16_t* a, const uint32_t* q0, const uint16_t* s0,
                     const uint16_t* b0, const uint32_t* q1, const uint16_t* s1,
                     const uint16_t* b1, void* out, int N, int G) {
#define MOE_U4(L)                                                              \
  hipLaunchKernelGGL((u4_kernel<PAIR, L>), grid, dim3(256), lds, s, offsets,   \
                     st, a, q0, s0, b0, q1, s1, b1, out, N, K, G)
  switch (pick_lpr(K)) {
    case 64: MOE_U4(64); break;
    case 32: MOE_U4(32); break;
    case 16: MOE_U4(16); break;
    case 8: MOE_U4(8); break;
    case 4: MOE_U4(4); break;
    default: MOE_U4(2); break;
  }
#undef MOE_U4
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_u4(const Dims& D, int group, const int32_t* offsets,
                         const int32_t* sorted_token, const void* x,
                         const moe_expert_weights& w, void* H, void* Y,
                         hipStream_t s) {
  if (D.d > kMaxK || D.F > kMaxK || !D.swiglu ||
      D.d != 32 * pick_lpr(D.d) || D.F != 32 * pick_lpr(D.F))
    return hipErrorInvalidValue;
  {
    const dim3 grid(D.E, (D.F + kUnitsPerBlock - 1) / kUnitsPerBlock);
    const size_t lds = static_cast<size_t>(kRC) * D.d * 2;
    hipError_t err = launch_u4<true>(
        D.d, grid, lds, s, offsets, sorted_token,
        static_cast<const uint16_t*>(x), static_cast<const uint32_t*>(w.gate),
        static_cast<const uint16_t*>(w.gate_scale),
        static_cast<const uint16_t*>(w.gate_bias),
        static_cast<const uint32_t*>(w.up), static_cast<const uint16_t*>(w.up_scale),
        static_cast<const uint16_t*>(w.up_bias), H, D.F,
        group);
    if (err != hipSuccess) return err;
  }
  {
    const dim3 grid(D.E, (D.d + kUnitsPerBlock - 1) / kUnitsPerBlock);
    const size_t lds = static_cast<size_t>(kRC) * D.F * 2;
    return launch_u4<false>(
        D.F, grid, lds, s, offsets, nullptr,
        static_cast<const uint16_t*>(H), static_cast<const uint32_t*>(w.down),
        static_cast<const uint16_t*>(w.down_scale),
        static_cast<const uint16_t*>(w.down_bias), nullptr, nullptr, nullptr,
        Y, D.d, group);
  }
}

}  // namespace moe
