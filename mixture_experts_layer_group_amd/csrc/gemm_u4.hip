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
// over each 32-element run a lane owns (always inside one group of 64).
//
// One kernel serves both products:
//   up   : unit = hidden column f; the lane loads the gate row f and the up
//          row f, the epilogue writes H = silu(gate) * up (fp16, as on the
//          matrix-core path)
//   down : unit = output column n of W_down, writes Y (fp32)
// LPR lanes share one unit and each lane streams VPL 16-byte vectors of it
// per pass; a wave works on 64/LPR units at once and reduces inside each
// lane group.
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kRC = 8;            // expert rows staged in LDS per pass
constexpr int kUnitsPerBlock = 64;
constexpr int kMaxK = 4096;  // kRC rows of K bf16 stay within 64 KiB of LDS

__device__ __forceinline__ void unpack8(uint32_t w, float* q) {
  const uint32_t lo = w & 0x0F0F0F0Fu;         // nibbles 0,2,4,6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // nibbles 1,3,5,7
  q[0] = static_cast<float>(lo & 0xFFu);
  q[1] = static_cast<float>(hi & 0xFFu);
  q[2] = static_cast<float>((lo >> 8) & 0xFFu);
  q[3] = static_cast<float>((hi >> 8) & 0xFFu);
  q[4] = static_cast<float>((lo >> 16) & 0xFFu);
  q[5] = static_cast<float>((hi >> 16) & 0xFFu);
  q[6] = static_cast<float>(lo >> 24);
  q[7] = static_cast<float>(hi >> 24);
}

template <bool PAIR, int LPR, int VPL>
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
  constexpr int UPW = 64 / LPR;   // units per wave pass
  constexpr int SPAN = 32 * VPL;  // elements per lane per K pass
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
    for (int ub = wave * UPW; ub < kUnitsPerBlock; ub += 4 * UPW) {
      const int u = u_base + ub + sg;
      const bool live = u < N;
      const int uu = live ? u : N - 1;
      const int64_t wrow = static_cast<int64_t>(e) * N + uu;
      float acc0[kRC], acc1[kRC];
#pragma unroll
      for (int r = 0; r < kRC; ++r) acc0[r] = acc1[r] = 0.f;
      for (int kc = 0; kc < K; kc += SPAN * LPR) {
        const int kb = kc + SPAN * kl;  // first element owned by this lane
        uint4 w0[VPL], w1[VPL];
        float sc0[VPL], bi0[VPL], sc1[VPL], bi1[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          w0[v] = *reinterpret_cast<const uint4*>(q0 + wrow * words + kb / 8 + 4 * v);
          if (PAIR) w1[v] = *reinterpret_cast<const uint4*>(q1 + wrow * words + kb / 8 + 4 * v);
        }
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          const int gi = (kb + 32 * v) / G;
          sc0[v] = bf16_to_f32(s0[wrow * groups + gi]);
          bi0[v] = bf16_to_f32(b0[wrow * groups + gi]);
          if (PAIR) {
            sc1[v] = bf16_to_f32(s1[wrow * groups + gi]);
            bi1[v] = bf16_to_f32(b1[wrow * groups + gi]);
          }
        }
#pragma unroll
        for (int r = 0; r < kRC; ++r) {
          if (r >= nr) break;
          const uint4* xv = reinterpret_cast<const uint4*>(xs + static_cast<int64_t>(r) * K + kb);
#pragma unroll
          for (int v = 0; v < VPL; ++v) {
            float qa[32], qb[32], xf[32];
            unpack8(w0[v].x, qa); unpack8(w0[v].y, qa + 8);
            unpack8(w0[v].z, qa + 16); unpack8(w0[v].w, qa + 24);
            if (PAIR) {
              unpack8(w1[v].x, qb); unpack8(w1[v].y, qb + 8);
              unpack8(w1[v].z, qb + 16); unpack8(w1[v].w, qb + 24);
            }
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const uint4 t = xv[4 * v + h];
              const uint32_t tw[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
              for (int m = 0; m < 4; ++m) {
                if (PAIR) {  // bf16 tokens
                  xf[8 * h + 2 * m] = __uint_as_float(tw[m] << 16);
                  xf[8 * h + 2 * m + 1] = __uint_as_float(tw[m] & 0xffff0000u);
                } else {     // fp16 hidden rows
                  xf[8 * h + 2 * m] = static_cast<float>(
                      __builtin_bit_cast(_Float16, static_cast<uint16_t>(tw[m] & 0xffffu)));
                  xf[8 * h + 2 * m + 1] = static_cast<float>(
                      __builtin_bit_cast(_Float16, static_cast<uint16_t>(tw[m] >> 16)));
                }
              }
            }
            float xsum = 0.f, pa = 0.f, pb = 0.f;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
              xsum += xf[j];
              pa = fmaf(xf[j], qa[j], pa);
              if (PAIR) pb = fmaf(xf[j], qb[j], pb);
            }
            acc0[r] += sc0[v] * pa + bi0[v] * xsum;
            if (PAIR) acc1[r] += sc1[v] * pb + bi1[v] * xsum;
          }
        }
      }
      // reduce inside the LPR-lane group
#pragma unroll
      for (int r = 0; r < kRC; ++r) {
#pragma unroll
        for (int o = LPR / 2; o > 0; o >>= 1) {
          acc0[r] += __shfl_xor(acc0[r], o, 64);
          if (PAIR) acc1[r] += __shfl_xor(acc1[r], o, 64);
        }
      }
      if (kl == 0 && live) {
#pragma unroll
        for (int r = 0; r < kRC; ++r) {
          if (r >= nr) break;
          const int64_t o = static_cast<int64_t>(row0 + rc0 + r) * N + u;
          if (PAIR) {  // hidden activation, fp16 (saturating)
            float h = acc0[r] / (1.f + __expf(-acc0[r])) * acc1[r];
            h = fminf(fmaxf(h, -65504.f), 65504.f);
            static_cast<_Float16*>(out)[o] = static_cast<_Float16>(h);
          }
          else  // expert output, fp32
            static_cast<float*>(out)[o] = acc0[r];
        }
      }
    }
  }
}

// lanes per unit and 16-byte vectors per lane for reduction length K
// (K is a multiple of 64): VPL = 4 when K % 128 == 0, else 2; LPR the largest
// power of two <= 64 with 32*VPL*LPR dividing K.
void pick_shape(int K, int* lpr, int* vpl) {
  *vpl = (K % 128 == 0) ? 4 : 2;
  int l = 64;
  while (l > 1 && K % (32 * *vpl * l) != 0) l >>= 1;
  *lpr = l;
}

template <bool PAIR>
hipError_t launch_u4(int K, dim3 grid, size_t lds, hipStream_t s,
                     const int32_t* offsets, const int32_t* st,
                     const uint16_t* a, const uint32_t* q0, const uint16_t* s0,
                     const uint16_t* b0, const uint32_t* q1, const uint16_t* s1,
                     const uint16_t* b1, void* out, int N, int G) {
  int lpr, vpl;
  pick_shape(K, &lpr, &vpl);
#define MOE_U4(L, V)                                                          \
  hipLaunchKernelGGL((u4_kernel<PAIR, L, V>), grid, dim3(256), lds, s,        \
                     offsets, st, a, q0, s0, b0, q1, s1, b1, out, N, K, G)
#define MOE_U4V(L) if (vpl == 4) MOE_U4(L, 4); else MOE_U4(L, 2)
  switch (lpr) {
    case 64: MOE_U4V(64); break;
    case 32: MOE_U4V(32); break;
    case 16: MOE_U4V(16); break;
    case 8: MOE_U4V(8); break;
    case 4: MOE_U4V(4); break;
    case 2: MOE_U4V(2); break;
    default: MOE_U4V(1); break;
  }
#undef MOE_U4V
#undef MOE_U4
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_u4(const Dims& D, int group, const int32_t* offsets,
                         const int32_t* sorted_token, const void* x,
                         const moe_expert_weights& w, void* H, void* Y,
                         hipStream_t s) {
  if (D.d > kMaxK || D.F > kMaxK || !D.swiglu) return hipErrorInvalidValue;
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
