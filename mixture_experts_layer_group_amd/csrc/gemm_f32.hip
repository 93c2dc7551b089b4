// fp32 grouped expert FFN on the vector ALUs (fp32 activations and
// weights).  Same computation as the bf16 MFMA path -- for each expert e,
// rows [offsets[e], offsets[e+1]) gathered through sorted_token, then
// ReLU ("Mixture of Experts" blog page, expert_forward) or SwiGLU (Edge0
// "MoE Spec and Routing" page, _swiglu) and the output projection -- with
// fp32 accumulation and an fp32 hidden activation.  Meant for small
// layers; one thread per output element, K-loop over contiguous rows.
#include "moe_internal.hpp"

namespace moe {
namespace {

__device__ __forceinline__ int find_group(const int32_t* __restrict__ off,
                                          int E, int32_t row) {
  int lo = 0, hi = E - 1;  // largest e with off[e] <= row
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float dot(const float* __restrict__ a,
                                     const float* __restrict__ b, int n) {
  float s = 0.f;
  for (int i = 0; i < n; ++i) s = fmaf(a[i], b[i], s);
  return s;
}

// H[r, n] = act(x[tok(r)] . Wa[e][n] (, x . Wb[e][n]))
// identity: rows are tokens 0..T-1 of one (shared) expert
__global__ void __launch_bounds__(256)
f32_up_kernel(const int32_t* __restrict__ offsets, int E,
              const int32_t* __restrict__ sorted_token,
              const float* __restrict__ x, const float* __restrict__ wa,
              const float* __restrict__ wb, int64_t wstride,
              float* __restrict__ H, int64_t rows_max, int d, int F, int swiglu,
              int identity) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = identity ? rows_max : offsets[E];
  if (idx >= total * F) return;
  const int64_t r = idx / F;
  const int n = static_cast<int>(idx % F);
  const int e = identity ? 0 : find_group(offsets, E, static_cast<int32_t>(r));
  const int64_t tok = identity ? r : sorted_token[r];
  const float* xr = x + tok * d;
  // wstride: elements from one expert's matrix to the next
  const int64_t wrow = static_cast<int64_t>(e) * wstride + static_cast<int64_t>(n) * d;
  const float a = dot(xr, wa + wrow, d);
  float h;
  if (swiglu) {
    const float b = dot(xr, wb + wrow, d);
    h = a / (1.f + expf(-a)) * b;
  } else {
    h = a > 0.f ? a : 0.f;
  }
  H[r * F + n] = h;
}

// Y[r, m] = H[r] . Wd[e][m]  (times row_scale[r] when it is given)
__global__ void __launch_bounds__(256)
f32_down_kernel(const int32_t* __restrict__ offsets, int E,
                const float* __restrict__ H, const float* __restrict__ wd,
                const float* __restrict__ row_scale, float* __restrict__ Y,
                int64_t rows_max, int d, int F, int identity) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = identity ? rows_max : offsets[E];
  if (idx >= total * d) return;
  const int64_t r = idx / d;
  const int m = static_cast<int>(idx % d);
  const int e = identity ? 0 : find_group(offsets, E, static_cast<int32_t>(r));
  const float y = dot(H + r * F, wd + (static_cast<int64_t>(e) * d + m) * F, F);
  Y[r * d + m] = row_scale != nullptr ? y * row_scale[r] : y;
}

}  // namespace

hipError_t launch_ffn_f32(const Dims& D, const int32_t* offsets,
                          const int32_t* sorted_token, const void* x,
                          const moe_expert_weights& w, const float* row_scale, void* H,
                          void* Hs, void* Y, void* Ys, hipEvent_t mid, hipStream_t s) {
  const float* xf = static_cast<const float*>(x);
  // FUSED_GATE_UP: each expert's [F][d] gate rows, then its up rows
  const int64_t mat = static_cast<int64_t>(D.F) * D.d;
  const float* wg = static_cast<const float*>(w.gate);
  const float* wu = D.fused ? wg + mat : static_cast<const float*>(w.up);
  {
    const int64_t n = D.slots * D.F;
    hipLaunchKernelGGL(f32_up_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, s, offsets, D.E, sorted_token, xf, wg, wu,
                       D.fused ? 2 * mat : mat, static_cast<float*>(H),
                       D.slots, D.d, D.F, D.swiglu ? 1 : 0, 0);
    if (mid != nullptr) {
      const hipError_t e = hipEventRecord(mid, s);
      if (e != hipSuccess) return e;
    }
    const int64_t m = D.slots * D.d;
    hipLaunchKernelGGL(f32_down_kernel, dim3(static_cast<unsigned>((m + 255) / 256)),
                       dim3(256), 0, s, offsets, D.E, static_cast<const float*>(H),
                       static_cast<const float*>(w.down), row_scale, static_cast<float*>(Y),
                       D.slots, D.d, D.F, 0);
  }
  for (int sh = 0; sh < D.S; ++sh) {
    const int64_t n = D.T * D.Fs;
    const int64_t smat = static_cast<int64_t>(D.Fs) * D.d;
    const int64_t so = static_cast<int64_t>(sh) * smat;
    const float* sg = static_cast<const float*>(w.shared_gate) + (D.fused ? 2 * so : so);
    const float* su = D.fused ? sg + smat
                              : (D.swiglu ? static_cast<const float*>(w.shared_up) + so
                                          : nullptr);
    hipLaunchKernelGGL(f32_up_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, s, offsets, 1, sorted_token, xf, sg, su,
                       int64_t{0}, static_cast<float*>(Hs), D.T, D.d, D.Fs,
                       D.swiglu ? 1 : 0, 1);
    const int64_t m = D.T * D.d;
    hipLaunchKernelGGL(f32_down_kernel, dim3(static_cast<unsigned>((m + 255) / 256)),
                       dim3(256), 0, s, offsets, 1, static_cast<const float*>(Hs),
                       static_cast<const float*>(w.shared_down) + so, nullptr,
                       static_cast<float*>(Ys) + static_cast<int64_t>(sh) * D.T * D.d,
                       D.T, D.d, D.Fs, 1);
  }
  return hipGetLastError();
}

}  // namespace moe
