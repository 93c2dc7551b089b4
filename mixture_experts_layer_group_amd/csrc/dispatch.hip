// Dispatch: a stable counting sort of the T*k routing slots by expert with
// per-expert capacity ("Mixture of Experts" blog page: the first program's
// moe_layer keeps each expert's first `capacity` slots in arrival order;
// the third program's route_and_sort does the same with a stable sort,
// a bincount and expert offsets).  Integer-only and deterministic:
//   1. count   -- each block histograms a chunk of slots in LDS;
//   2. scan    -- one block turns the [blocks x E] histogram into each
//                 block's per-expert base rank (exclusive over blocks),
//                 applies the capacity, and writes counts, offsets, the
//                 drop count and the per-expert M-tile prefix of the GEMMs;
//   3. scatter -- each block walks its chunk in slot order, 256 slots per
//                 round; inside a wave, lanes holding the same expert are
//                 found by matching expert-id bits with ballots, so every
//                 slot gets its exact rank in token order without atomics.
#include "moe_internal.hpp"

namespace moe {
namespace {

__global__ void __launch_bounds__(256)
count_kernel(const int32_t* __restrict__ ids, int64_t S, int E,
             int32_t* __restrict__ hist) {
  extern __shared__ int32_t h[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
  __syncthreads();
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kDispatchChunk;
  const int64_t s1 = min(S, s0 + kDispatchChunk);
  for (int64_t s = s0 + threadIdx.x; s < s1; s += blockDim.x) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    hist[static_cast<int64_t>(blockIdx.x) * E + e] = h[e];
}

// One block of 1024 threads.  hist[b][e] becomes the exclusive base of
// expert e at block b.
__global__ void __launch_bounds__(1024)
scan_kernel(int32_t* __restrict__ hist, int nb, int E, int64_t S, int64_t cap,
            int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
            int32_t* __restrict__ dropped, int32_t* __restrict__ tiles1,
            int bm1, int32_t* __restrict__ tiles2, int bm2) {
  extern __shared__ int32_t sm[];
  int32_t* kept = sm;           // [E]
  int32_t* t1 = sm + E;         // [E]
  int32_t* t2 = sm + 2 * E;     // [E]
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int32_t run = 0;
    for (int b = 0; b < nb; ++b) {
      const int64_t i = static_cast<int64_t>(b) * E + e;
      const int32_t c = hist[i];
      hist[i] = run;
      run += c;
    }
    counts[e] = run;
    const int32_t kp = static_cast<int64_t>(run) < cap ? run : static_cast<int32_t>(cap);
    kept[e] = kp;
    t1[e] = (kp + bm1 - 1) / bm1;
    t2[e] = (kp + bm2 - 1) / bm2;
  }
  __syncthreads();
  // exclusive prefix over experts (E is at most a few thousand: thread 0
  // walks it; this kernel is launch-bound anyway)
  if (threadIdx.x == 0) {
    int32_t a = 0, b1 = 0, b2 = 0;
    for (int e = 0; e < E; ++e) {
      offsets[e] = a;
      if (tiles1) tiles1[e] = b1;
      if (tiles2) tiles2[e] = b2;
      a += kept[e];
      b1 += t1[e];
      b2 += t2[e];
    }
    offsets[E] = a;
    if (tiles1) tiles1[E] = b1;
    if (tiles2) tiles2[E] = b2;
    dropped[0] = static_cast<int32_t>(S - a);
  }
}

__global__ void __launch_bounds__(256)
scatter_kernel(const int32_t* __restrict__ ids, const float* __restrict__ w,
               int64_t S, int k, int E, int64_t cap, int nbits,
               const int32_t* __restrict__ base,
               const int32_t* __restrict__ offsets,
               int32_t* __restrict__ sorted_token, float* __restrict__ sorted_w,
               int32_t* __restrict__ slot_row) {
  extern __shared__ int32_t sm[];
  int32_t* run = sm;            // [E] running rank per expert
  int32_t* wcnt = sm + E;       // [4][E] per-wave counts of this round
  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    run[e] = base[static_cast<int64_t>(blockIdx.x) * E + e];
#pragma unroll
    for (int q = 0; q < 4; ++q) wcnt[q * E + e] = 0;
  }
  __syncthreads();
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kDispatchChunk;
  const int64_t s1 = min(S, s0 + kDispatchChunk);
  for (int64_t r0 = s0; r0 < s1; r0 += blockDim.x) {
    const int64_t s = r0 + threadIdx.x;
    int e = -1;
    if (s < s1) {
      const int v = ids[s];
      if (v >= 0 && v < E) e = v;
    }
    const bool valid = e >= 0;
    uint64_t mask = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t bal = __ballot(bit);
      mask &= bit ? bal : ~bal;
    }
    const int within = __popcll(mask & lt_mask);
    if (valid && within == 0) wcnt[wv * E + e] = __popcll(mask);
    __syncthreads();
    int32_t rank = 0;
    if (valid) {
      rank = run[e] + within;
      for (int q = 0; q < wv; ++q) rank += wcnt[q * E + e];
    }
    __syncthreads();
    for (int x = threadIdx.x; x < E; x += blockDim.x) {
      int32_t add = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        add += wcnt[q * E + x];
        wcnt[q * E + x] = 0;
      }
      run[x] += add;
    }
    if (s < s1) {
      int32_t row = -1;
      if (valid && static_cast<int64_t>(rank) < cap) {
        row = offsets[e] + rank;
        sorted_token[row] = static_cast<int32_t>(s / k);
        sorted_w[row] = w[s];
      }
      slot_row[s] = row;
    }
    __syncthreads();
  }
}

__global__ void tile_prefix_kernel(const int32_t* __restrict__ offsets, int E,
                                   int32_t* __restrict__ tiles1, int bm1,
                                   int32_t* __restrict__ tiles2, int bm2) {
  if (threadIdx.x != 0) return;
  int32_t b1 = 0, b2 = 0;
  for (int e = 0; e < E; ++e) {
    const int32_t n = offsets[e + 1] - offsets[e];
    tiles1[e] = b1;
    tiles2[e] = b2;
    b1 += (n + bm1 - 1) / bm1;
    b2 += (n + bm2 - 1) / bm2;
  }
  tiles1[E] = b1;
  tiles2[E] = b2;
}

template <typename T>
__global__ void __launch_bounds__(256)
gather_kernel(const int32_t* __restrict__ offsets, int E,
              const int32_t* __restrict__ sorted_token, const T* __restrict__ x,
              T* __restrict__ xp, int d) {
  const int64_t r = blockIdx.x;
  if (r >= offsets[E]) return;
  const int64_t t = sorted_token[r];
  // 16-byte vectors; d is a multiple of 8 elements
  const int nvec = d * static_cast<int>(sizeof(T)) / 16;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * d);
  uint4* dst = reinterpret_cast<uint4*>(xp + r * d);
  for (int i = threadIdx.x; i < nvec; i += blockDim.x) dst[i] = src[i];
}

}  // namespace

hipError_t launch_dispatch(const Dims& D, const int32_t* ids, const float* w,
                           int32_t* hist, int nblocks, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_token,
                           float* sorted_w, int32_t* slot_row, int32_t* dropped,
                           int32_t* tiles1, int32_t* tiles2, hipStream_t s) {
  const size_t hsz = static_cast<size_t>(D.E) * sizeof(int32_t);
  hipLaunchKernelGGL(count_kernel, dim3(nblocks), dim3(256), hsz, s, ids,
                     D.slots, D.E, hist);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 3 * hsz, s, hist,
                     nblocks, D.E, D.slots, D.cap, counts, offsets, dropped,
                     tiles1, kGemm1BM, tiles2, kGemm2BM);
  int nbits = 0;
  while ((1 << nbits) < D.E) ++nbits;
  hipLaunchKernelGGL(scatter_kernel, dim3(nblocks), dim3(256), 5 * hsz, s, ids,
                     w, D.slots, D.k, D.E, D.cap, nbits, hist, offsets,
                     sorted_token, sorted_w, slot_row);
  return hipGetLastError();
}

hipError_t launch_tile_prefix(const Dims& D, const int32_t* offsets,
                              int32_t* tiles1, int32_t* tiles2, hipStream_t s) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(64), 0, s, offsets, D.E,
                     tiles1, kGemm1BM, tiles2, kGemm2BM);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const Dims& D, const int32_t* offsets,
                              const int32_t* sorted_token, const void* x,
                              void* x_perm, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(D.slots));
  if (D.bf16)
    hipLaunchKernelGGL(gather_kernel<uint16_t>, grid, dim3(256), 0, s, offsets,
                       D.E, sorted_token, static_cast<const uint16_t*>(x),
                       static_cast<uint16_t*>(x_perm), D.d);
  else
    hipLaunchKernelGGL(gather_kernel<float>, grid, dim3(256), 0, s, offsets,
                       D.E, sorted_token, static_cast<const float*>(x),
                       static_cast<float*>(x_perm), D.d);
  return hipGetLastError();
}

}  // namespace moe
