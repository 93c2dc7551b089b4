// Combine: the routed expert outputs go back to token order, each scaled by
// its routing weight (unless the expert rows already carry it), summed with
// the always-on shared experts (dockyard_rl
// "Mixture-of-Experts" page, "The pipeline", combine; "Mixture of Experts"
// blog page, the third program's scatter-add, where a token routed to k
// experts collects k contributions; "Mixture-of-Experts Documentation",
// shared expert).  Written as a gather -- each token reads its own kept rows
// through slot_row -- so the sum has a fixed order (slot 0..k-1, then the
// shared experts) and needs no atomics.  Dropped slots (row -1) add nothing.
#include <algorithm>

#include "moe_internal.hpp"

namespace moe {
namespace {

__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
// 8 fp16 values (one 16-byte load), exactly widened to fp32
__device__ __forceinline__ void load8(const _Float16* p, float* v) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const h8 a = *reinterpret_cast<const h8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = static_cast<float>(a[j]);
}
__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
  uint4 a;
  a.x = pack_bf16x2(v[0], v[1]);
  a.y = pack_bf16x2(v[2], v[3]);
  a.z = pack_bf16x2(v[4], v[5]);
  a.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = a;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

constexpr int kMaxSlots = 64;

// One block per token of d/8 threads (up to 1024, whole waves): each thread
// owns 8 consecutive columns, so a row is one pass; the token's kept rows
// are loaded in groups of 4 before they are added (in slot order).  Expert
// rows are fp32 or fp16 (YT), the sum is fp32, the result is written in the
// output type.
template <typename OutT, typename YT>
__global__ void __launch_bounds__(1024)
combine_kernel(const YT* __restrict__ y, const YT* __restrict__ ypart,
               const int32_t* __restrict__ slot_row,
               const float* __restrict__ topk_w, const float* __restrict__ ysh,
               OutT* __restrict__ out, int64_t Tn, int k, int S, int d) {
  __shared__ int32_t rows[kMaxSlots];
  __shared__ float wts[kMaxSlots];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = slot_row[t * k + threadIdx.x];
    // no weights: the rows already carry them (moe_grouped_ffn with sorted_w)
    wts[threadIdx.x] = topk_w != nullptr ? topk_w[t * k + threadIdx.x] : 1.f;
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < k; i0 += 4) {
      float v[4][8], u[4][8];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int i = i0 + jj;
        const int32_t r = i < k ? rows[i] : -1;
        if (r < 0) continue;
        load8(y + static_cast<int64_t>(r) * d + c, v[jj]);
        if (ypart) load8(ypart + static_cast<int64_t>(r) * d + c, u[jj]);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int i = i0 + jj;
        if (i >= k || rows[i] < 0) continue;
        if (ypart) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[jj][j] += u[jj][j];
        }
        const float wi = wts[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(wi, v[jj][j], acc[j]);
      }
    }
    for (int s = 0; s < S; ++s) {
      float v[8];
      load8(ysh + (static_cast<int64_t>(s) * Tn + t) * d + c, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += v[j];
    }
    store8(out + t * d + c, acc);
  }
}

// one block per row band; rows at or past the kept count are skipped
__global__ void __launch_bounds__(256)
fold_split_kernel(const int32_t* __restrict__ offsets, int E, float* __restrict__ y,
                  const float* __restrict__ ypart, int d) {
  const int64_t r = blockIdx.x;
  if (r >= offsets[E]) return;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    float v[8], u[8];
    load8(y + r * d + c, v);
    load8(ypart + r * d + c, u);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] += u[j];
    store8(y + r * d + c, v);
  }
}

}  // namespace

hipError_t launch_fold_split(const Dims& D, const int32_t* offsets, float* Y,
                             const float* Ypart, hipStream_t s) {
  const int64_t rows = std::min<int64_t>(D.slots, D.cap * D.E);
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(fold_split_kernel, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s,
                     offsets, D.E, Y, Ypart, D.d);
  return hipGetLastError();
}

hipError_t launch_combine(const Dims& D, const void* y_rows, const void* y_part, bool y16,
                          const int32_t* slot_row, const float* topk_w,
                          const void* y_shared, void* out, hipStream_t s) {
  if (D.k > kMaxSlots) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(D.T));
  const int threads = std::min(1024, (D.d / 8 + 63) / 64 * 64);  // >= 64 >= k
  const int S = y_shared ? D.S : 0;
  const float* ys = static_cast<const float*>(y_shared);
  if (y16) {
    const _Float16* y = static_cast<const _Float16*>(y_rows);
    const _Float16* yp = static_cast<const _Float16*>(y_part);
    if (D.out_bf16)
      hipLaunchKernelGGL((combine_kernel<uint16_t, _Float16>), grid, dim3(threads), 0, s, y, yp,
                         slot_row, topk_w, ys, static_cast<uint16_t*>(out), D.T, D.k, S, D.d);
    else
      hipLaunchKernelGGL((combine_kernel<float, _Float16>), grid, dim3(threads), 0, s, y, yp,
                         slot_row, topk_w, ys, static_cast<float*>(out), D.T, D.k, S, D.d);
  } else {
    const float* y = static_cast<const float*>(y_rows);
    const float* yp = static_cast<const float*>(y_part);
    if (D.out_bf16)
      hipLaunchKernelGGL((combine_kernel<uint16_t, float>), grid, dim3(threads), 0, s, y, yp,
                         slot_row, topk_w, ys, static_cast<uint16_t*>(out), D.T, D.k, S, D.d);
    else
      hipLaunchKernelGGL((combine_kernel<float, float>), grid, dim3(threads), 0, s, y, yp,
                         slot_row, topk_w, ys, static_cast<float*>(out), D.T, D.k, S, D.d);
  }
  return hipGetLastError();
}

}  // namespace moe
