// Routing health and the aux-loss-free bias update, from a layer call's
// dispatch counts: one workgroup of 1024 threads (E <= 1024), block-wide
// reductions in a fixed order.
//   health: "Mixture of Experts" blog page, second program (RoutingHealth,
//     MoELayer._health) and third program (routing_health,
//     load_balancing_loss);
//   bias:   dockyard "Mixture-of-Experts" page, "Aux-loss-free load
//     balancing": each step an expert's selection bias moves up by the step
//     size when its load is below the mean load and down when above.
#include <math.h>

#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kHealthThreads = 1024;
constexpr float kCollapseRatio = 0.5f;

// block-wide fp32 sum over the 16 waves, fixed order
__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < kHealthThreads / kWave; ++i) s += red[i];
  return s;
}
// block-wide int sum / max over the 16 waves (exact in any order: the
// totals fit int32 because T*k <= 2^31 - 1)
__device__ int wave_isum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ int wave_imax(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ int block_isum(int v, int* red) {
  v = wave_isum(v);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  int s = 0;
  for (int i = 0; i < kHealthThreads / kWave; ++i) s += red[i];
  return s;
}
__device__ int block_imax(int v, int* red) {
  v = wave_imax(v);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  int s = red[0];
  for (int i = 1; i < kHealthThreads / kWave; ++i) s = max(s, red[i]);
  return s;
}

__global__ void __launch_bounds__(kHealthThreads)
health_kernel(const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
              const int32_t* __restrict__ dropped, const float* __restrict__ prob_sum,
              float* __restrict__ bias, float step, moe_health* __restrict__ h,
              int64_t T, int k, int E) {
  __shared__ float red[kHealthThreads / kWave];
  __shared__ int ired[kHealthThreads / kWave];
  const int e = threadIdx.x;
  const bool on = e < E;
  const int kept = on ? offsets[e + 1] - offsets[e] : 0;
  const int cnt = on ? counts[e] : 0;
  // integer totals and maxima, exact: kept and pre-drop slots
  const int kept_i = block_isum(kept, ired);
  const int cnt_i = block_isum(cnt, ired);
  const float kept_total = static_cast<float>(kept_i);
  const float cnt_total = static_cast<float>(cnt_i);
  const float cnt_max = static_cast<float>(block_imax(cnt, ired));
  const float kmax = static_cast<float>(block_imax(kept, ired));
  // entropy of the normalised kept shares
  const float q = (on && kept_total > 0.f) ? static_cast<float>(kept) / kept_total : 0.f;
  const float ent = block_sum(q > 0.f ? -q * logf(q) : 0.f, red);
  const float Tf = static_cast<float>(T);
  float aux = 0.f;
  if (prob_sum) {
    const float P = on ? prob_sum[e] / Tf : 0.f;
    aux = block_sum(on ? (static_cast<float>(kept) / (Tf * k)) * P : 0.f, red);
    aux *= static_cast<float>(E);
  }
  if (bias && on && step != 0.f) {
    // load below the mean <=> E*count < total (exact in integers)
    const int64_t total = cnt_i;
    const int64_t lhs = static_cast<int64_t>(E) * cnt;
    const float s = lhs < total ? 1.f : (lhs > total ? -1.f : 0.f);
    bias[e] = bias[e] + step * s;
  }
  if (threadIdx.x == 0) {
    const float maxent = logf(static_cast<float>(E));
    const float ratio = kept_total > 0.f ? ent / maxent : 0.f;
    moe_health r;
    r.aux = aux;
    r.aux3 = aux * static_cast<float>(k);
    r.entropy = kept_total > 0.f ? ent : 0.f;
    r.max_entropy = maxent;
    r.entropy_ratio = ratio;
    r.max_share = kept_total > 0.f ? kmax / kept_total : 0.f;
    r.dropped_fraction = static_cast<float>(dropped[0]) / (Tf * k);
    r.load_peak_over_mean = cnt_total > 0.f ? cnt_max / (cnt_total / static_cast<float>(E)) : 0.f;
    r.collapsed = ratio < kCollapseRatio ? 1 : 0;
    r.kept_total = kept_i;
    *h = r;
  }
}

}  // namespace

hipError_t launch_routing_health(const Dims& D, const int32_t* counts,
                                 const int32_t* offsets, const int32_t* dropped,
                                 const float* prob_sum, float* bias, float step,
                                 moe_health* h, hipStream_t s) {
  if (D.E > kHealthThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(health_kernel, dim3(1), dim3(kHealthThreads), 0, s, counts, offsets,
                     dropped, prob_sum, bias, step, h, D.T, D.k, D.E);
  return hipGetLastError();
}

}  // namespace moe
