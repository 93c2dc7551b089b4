// Dispatch: a stable counting sort of the T*k routing slots by expert with
// per-expert capacity ("Mixture of Experts" blog page: the first program's
// moe_layer keeps each expert's first `capacity` slots in arrival order;
// the third program's route_and_sort does the same with a stable sort,
// a bincount and expert offsets).  Integer-only and deterministic:
//   1. count   -- each block histograms a chunk of slots in LDS;
//   2. scan    -- one block turns the [blocks x E] histogram into each
//                 block's per-expert base rank (exclusive over blocks),
//                 applies the capacity, and writes counts, offsets, the
//                 drop count and the per-expert M-tile prefix of the GEMMs
//                 (block-wide prefix sums over experts);
//   3. scatter -- each block walks its chunk in slot order, 256 slots per
//                 round; inside a wave, lanes holding the same expert are
//                 found by matching expert-id bits with ballots, so every
//                 slot gets its exact rank in token order without atomics.
// When all slots fit one chunk (decode-sized batches) a single block does
// the three steps in one launch.
#include "moe_internal.hpp"

namespace moe {
namespace {

__global__ void __launch_bounds__(256)
count_kernel(const int32_t* __restrict__ ids, int64_t S, int E,
             int32_t* __restrict__ hist, int32_t* __restrict__ err) {
  extern __shared__ int32_t h[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
  __syncthreads();
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kDispatchChunk;
  const int64_t s1 = min(S, s0 + kDispatchChunk);
  bool bad = false;  // an id outside [0,E): its slot is dropped
  // the chunk's ids are all loaded before they are counted
  constexpr int kRounds = kDispatchChunk / 256;
  int idv[kRounds];
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    const int64_t s = s0 + q * 256 + threadIdx.x;
    idv[q] = s < s1 ? ids[s] : 0;
  }
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    if (s0 + q * 256 + threadIdx.x >= s1) break;
    const int e = idv[q];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    else bad = true;
  }
  if (err != nullptr && __ballot(bad) != 0 && (threadIdx.x & 63) == 0)
    atomicOr(err, MOE_FLAG_BAD_EXPERT_ID);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    hist[static_cast<int64_t>(blockIdx.x) * E + e] = h[e];
}

// Exclusive prefix sum of one value per thread over the block (blockDim a
// multiple of 64, at most 1024).  `wsum` is LDS scratch of 16 values.
// Returns the exclusive prefix; *total receives the block sum.
template <typename V>
__device__ __forceinline__ V block_exclusive_scan(V v, V* wsum, V* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  V x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const V y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  V base = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const V s = wsum[w];
    if (w < wv) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// The XCD ranges of one routed GEMM (XcdPlan): thread e holds expert e's
// kept rows `kp`, its first M tile `mt_off` and the M-tile total.  An
// expert's N-tile columns are contiguous in the tile list (each holds the
// expert's M tiles) and cost the same, w per column, so the tile where the
// running cost reaches x/8 of the total is found by the thread of the expert
// it falls in, rounded to the nearest column.  Thread 0 then clamps each
// boundary so that no range exceeds cap tiles and the later XCDs can still
// hold the rest, and writes the kXcds + 1 boundaries (the last one is the
// tile count); threads 0-7 zero the claim counters.
__device__ void xcd_bounds(int E, int32_t kp, int bm, int mt_off, int mt_total,
                           const XcdPlan& p, int32_t* __restrict__ bounds,
                           long long* wsum64, int* sh) {
  // the run-time claim counters of the ranges' last quarters start at zero
  if (threadIdx.x < kXcds)
    *reinterpret_cast<unsigned long long*>(bounds - (E + 1) + tile_claims_at(E) +
                                           kClaimStride * threadIdx.x) = 0;
  const int mte = threadIdx.x < E ? (kp + bm - 1) / bm : 0;
  long long w = 0;
  if (mte > 0) {
    const int last = kp - (mte - 1) * bm;
    const long long blocks = static_cast<long long>(mte - 1) * (bm / 32) + (last + 31) / 32;
    w = p.kt * blocks + static_cast<long long>(p.c) * mte;
  }
  long long wt;
  const long long P = block_exclusive_scan<long long>(w, wsum64, &wt);
  const long long split_cost = wt * p.nt;
  const long long total = split_cost * p.ksplit;
  const long long split_tiles = static_cast<long long>(mt_total) * p.nt;
  const long long all_tiles = split_tiles * p.ksplit;
  if (w > 0) {
    const long long lo = P * p.nt, hi = (P + w) * p.nt;
    for (int x = 1; x < kXcds; ++x) {
      const long long target = total * x / kXcds;
      const long long sp = target / split_cost;
      const long long r = target - sp * split_cost;
      if (r >= lo && r < hi) {
        const long long col = (r - lo + w / 2) / w;
        sh[x] = static_cast<int>(sp * split_tiles + static_cast<long long>(mt_off) * p.nt +
                                 col * mte);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long prev = 0;
    bounds[0] = 0;
    for (int x = 1; x < kXcds; ++x) {
      long long v = total > 0 ? sh[x] : 0;
      const long long lo = max(prev, all_tiles - static_cast<long long>(kXcds - x) * p.cap);
      v = min(max(v, lo), prev + p.cap);
      bounds[x] = static_cast<int32_t>(v);
      prev = v;
    }
    bounds[kXcds] = static_cast<int32_t>(all_tiles);
  }
  __syncthreads();
}

// Kept count, per-expert capacity and M-tile counts of one expert, written
// as exclusive prefixes over experts (thread e handles expert e; E <= 1024),
// then each routed GEMM's XCD ranges after its M-tile prefix.
__device__ __forceinline__ int expert_prefixes(int e, int E, int32_t cnt, int64_t S,
                                                int64_t cap, int32_t* __restrict__ counts,
                                                int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ dropped,
                                                int32_t* __restrict__ tiles1, int bm1,
                                                int32_t* __restrict__ tiles2, int bm2,
                                                const XcdPlan& p1, const XcdPlan& p2,
                                                int* wsum) {
  __shared__ long long wsum64[16];
  __shared__ int sh[kXcds];
  const bool on = e < E;
  const int32_t kp = on ? (static_cast<int64_t>(cnt) < cap ? cnt : static_cast<int32_t>(cap)) : 0;
  int tot;
  const int off = block_exclusive_scan(kp, wsum, &tot);
  if (on) {
    counts[e] = cnt;
    offsets[e] = off;
  }
  if (threadIdx.x == 0) {
    offsets[E] = tot;
    dropped[0] = static_cast<int32_t>(S - tot);
  }
  if (tiles1) {
    int t;
    const int o1 = block_exclusive_scan(on ? (kp + bm1 - 1) / bm1 : 0, wsum, &t);
    if (on) tiles1[e] = o1;
    if (threadIdx.x == 0) tiles1[E] = t;
    if (p1.nt > 0) xcd_bounds(E, kp, bm1, o1, t, p1, tiles1 + E + 1, wsum64, sh);
  }
  if (tiles2) {
    int t;
    const int o2 = block_exclusive_scan(on ? (kp + bm2 - 1) / bm2 : 0, wsum, &t);
    if (on) tiles2[e] = o2;
    if (threadIdx.x == 0) tiles2[E] = t;
    if (p2.nt > 0) xcd_bounds(E, kp, bm2, o2, t, p2, tiles2 + E + 1, wsum64, sh);
  }
  return off;
}

// One block of 1024 threads (thread e = expert e).  hist[b][e] becomes the
// exclusive base of expert e at block b.
__global__ void __launch_bounds__(1024)
scan_kernel(int32_t* __restrict__ hist, int nb, int E, int64_t S, int64_t cap,
            int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
            int32_t* __restrict__ dropped, int32_t* __restrict__ tiles1,
            int bm1, int32_t* __restrict__ tiles2, int bm2, XcdPlan p1, XcdPlan p2) {
  __shared__ int wsum[16];
  const int e = threadIdx.x;
  int32_t run = 0;
  if (e < E) {
    // blocks in groups of kG: the group's counts are all loaded before any
    // is replaced by its base (one memory round trip per group, not per block)
    constexpr int kG = 32;
    for (int b0 = 0; b0 < nb; b0 += kG) {
      int32_t c[kG];
#pragma unroll
      for (int j = 0; j < kG; ++j)
        c[j] = b0 + j < nb ? hist[static_cast<int64_t>(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kG; ++j) {
        if (b0 + j < nb) hist[static_cast<int64_t>(b0 + j) * E + e] = run;
        run += c[j];
      }
    }
  }
  expert_prefixes(e, E, run, S, cap, counts, offsets, dropped, tiles1, bm1,
                  tiles2, bm2, p1, p2, wsum);
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
  int32_t* offs = sm + 5 * E;   // [E] the experts' first rows
  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kDispatchChunk;
  const int64_t s1 = min(S, s0 + kDispatchChunk);
  // every round's ids and weights are loaded up front (one memory round
  // trip for the chunk instead of one per round)
  constexpr int kRounds = kDispatchChunk / 256;
  int idv[kRounds];
  float wvv[kRounds];
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    const int64_t s = s0 + q * 256 + threadIdx.x;
    idv[q] = s < s1 ? ids[s] : -1;
    wvv[q] = s < s1 ? w[s] : 0.f;
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    run[e] = base[static_cast<int64_t>(blockIdx.x) * E + e];
    offs[e] = offsets[e];
#pragma unroll
    for (int q = 0; q < 4; ++q) wcnt[q * E + e] = 0;
  }
  __syncthreads();
  const uint64_t lt_mask = (1ull << lane) - 1ull;
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    const int64_t r0 = s0 + q * 256;
    if (r0 >= s1) break;
    const int64_t s = r0 + threadIdx.x;
    int e = -1;
    if (s < s1) {
      const int v = idv[q];
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
        row = offs[e] + rank;
        sorted_token[row] = static_cast<int32_t>(s / k);
        sorted_w[row] = wvv[q];
      }
      slot_row[s] = row;
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(1024)
tile_prefix_kernel(const int32_t* __restrict__ offsets, int E,
                   int32_t* __restrict__ tiles1, int bm1,
                   int32_t* __restrict__ tiles2, int bm2, XcdPlan p1, XcdPlan p2) {
  __shared__ int wsum[16];
  __shared__ long long wsum64[16];
  __shared__ int sh[kXcds];
  const int e = threadIdx.x;
  const int32_t n = e < E ? offsets[e + 1] - offsets[e] : 0;
  int t;
  const int o1 = block_exclusive_scan(e < E ? (n + bm1 - 1) / bm1 : 0, wsum, &t);
  if (e < E) tiles1[e] = o1;
  if (e == 0) tiles1[E] = t;
  if (p1.nt > 0) xcd_bounds(E, n, bm1, o1, t, p1, tiles1 + E + 1, wsum64, sh);
  const int o2 = block_exclusive_scan(e < E ? (n + bm2 - 1) / bm2 : 0, wsum, &t);
  if (e < E) tiles2[e] = o2;
  if (e == 0) tiles2[E] = t;
  if (p2.nt > 0) xcd_bounds(E, n, bm2, o2, t, p2, tiles2 + E + 1, wsum64, sh);
}

// All of the dispatch in one block when the slots fit one chunk (decode-
// sized batches): LDS histogram, prefixes, then the stable rank/scatter of
// scatter_kernel with block base 0.
__global__ void __launch_bounds__(1024)
dispatch_small_kernel(const int32_t* __restrict__ ids, const float* __restrict__ w,
                      int64_t S, int k, int E, int64_t cap, int nbits,
                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                      int32_t* __restrict__ dropped, int32_t* __restrict__ tiles1,
                      int bm1, int32_t* __restrict__ tiles2, int bm2, XcdPlan p1, XcdPlan p2,
                      int32_t* __restrict__ sorted_token, float* __restrict__ sorted_w,
                      int32_t* __restrict__ slot_row, int32_t* __restrict__ err) {
  __shared__ int wsum[16];
  __shared__ int32_t h[1024];
  __shared__ int32_t run[1024];
  __shared__ int32_t offs[1024];
  __shared__ int32_t wcnt[16][1024];  // per-wave counts of one round
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) h[e] = 0;
  __syncthreads();
  bool bad = false;  // an id outside [0,E): its slot is dropped
  for (int64_t s = tid; s < S; s += blockDim.x) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    else bad = true;
  }
  if (err != nullptr && __ballot(bad) != 0 && (tid & 63) == 0)
    atomicOr(err, MOE_FLAG_BAD_EXPERT_ID);
  __syncthreads();
  const int32_t cnt = tid < E ? h[tid] : 0;
  const int off = expert_prefixes(tid, E, cnt, S, cap, counts, offsets, dropped,
                                  tiles1, bm1, tiles2, bm2, p1, p2, wsum);
  if (tid < E) offs[tid] = off;
  __syncthreads();
  // ranks: slots in flat order; inside a wave, lanes with the same expert
  // are matched on the expert-id bits; across waves, earlier waves' counts
  // are added through a per-wave table of all experts in LDS
  const int lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int e = tid; e < E; e += blockDim.x) run[e] = 0;
  __syncthreads();
  for (int64_t r0 = 0; r0 < S; r0 += blockDim.x) {
    const int64_t s = r0 + tid;
    int e = -1;
    if (s < S) {
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
    const int mine = __popcll(mask);
    int32_t rank = 0;
    for (int q = 0; q < nw; ++q)
      for (int x = tid; x < E; x += blockDim.x) wcnt[q][x] = 0;
    __syncthreads();
    if (valid && within == 0) wcnt[wv][e] = mine;
    __syncthreads();
    if (valid) {
      rank = run[e] + within;
      for (int q = 0; q < wv; ++q) rank += wcnt[q][e];
    }
    __syncthreads();
    for (int x = tid; x < E; x += blockDim.x) {
      int32_t add = 0;
      for (int q = 0; q < nw; ++q) add += wcnt[q][x];
      run[x] += add;
    }
    __syncthreads();
    if (s < S) {
      int32_t row = -1;
      if (valid && static_cast<int64_t>(rank) < cap) {
        row = offs[e] + rank;
        sorted_token[row] = static_cast<int32_t>(s / k);
        sorted_w[row] = w[s];
      }
      slot_row[s] = row;
    }
  }
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
                           int32_t* tiles1, int32_t* tiles2, int32_t* err,
                           hipStream_t s) {
  const size_t hsz = static_cast<size_t>(D.E) * sizeof(int32_t);
  int nbits = 0;
  while ((1 << nbits) < D.E) ++nbits;
  if (D.slots <= kDispatchChunk) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(1024), 0, s, ids, w,
                       D.slots, D.k, D.E, D.cap, nbits, counts, offsets, dropped,
                       tiles1, routed_bm(D), tiles2, routed_bm(D), xcd_plan(D, false),
                       xcd_plan(D, true), sorted_token, sorted_w, slot_row, err);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(count_kernel, dim3(nblocks), dim3(256), hsz, s, ids,
                     D.slots, D.E, hist, err);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, hist,
                     nblocks, D.E, D.slots, D.cap, counts, offsets, dropped,
                     tiles1, routed_bm(D), tiles2, routed_bm(D), xcd_plan(D, false),
                     xcd_plan(D, true));
  hipLaunchKernelGGL(scatter_kernel, dim3(nblocks), dim3(256), 6 * hsz, s, ids,
                     w, D.slots, D.k, D.E, D.cap, nbits, hist, offsets,
                     sorted_token, sorted_w, slot_row);
  return hipGetLastError();
}

hipError_t launch_tile_prefix(const Dims& D, const int32_t* offsets,
                              int32_t* tiles1, int32_t* tiles2, hipStream_t s) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, s, offsets, D.E,
                     tiles1, routed_bm(D), tiles2, routed_bm(D), xcd_plan(D, false),
                     xcd_plan(D, true));
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
