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

// The XCD ranges of the two routed GEMMs (XcdPlan; nt == 0 or tiles null:
// none), by the whole block (thread e holds expert e's kept rows kp and
// first M tile mt_off; E <= 1024).  An expert's N-tile columns are
// contiguous in the tile list (each holds its M tiles) and cost the same,
// w = kt x (its 32-row blocks) + c x (its M tiles), so in units of one
// column of every expert the list's cost is the prefix of w: expert e spans
// [pre[e], pre[e + 1]) (both read from LDS, so the spans tile the line
// exactly), its columns w / nt each.  The thread of the expert where the
// running cost reaches x/8 of the total (over the K splits) writes that
// boundary, rounded to the nearest column.  fp32 costs are plenty for
// balancing; a boundary no thread writes stays at -1, which the clamps
// lift.  Threads 0 and 64 then clamp each GEMM's boundaries so that no
// range exceeds cap tiles and the later XCDs can still hold the rest, and
// write the kXcds + 1 of them (the last is the tile count); threads 0-7 zero
// the claim counters.
struct XcdScratch {
  float wsum[2][16];
  float pre[2][1025];
  int sh[2][kXcds];
};

__device__ __forceinline__ float gemm_cost(int kp, int mte, const XcdPlan& p) {
  return mte > 0 ? static_cast<float>(p.kt) * static_cast<float>((kp + 31) >> 5) +
                       static_cast<float>(p.c) * static_cast<float>(mte)
                 : 0.f;
}

__device__ void xcd_bounds(int E, int32_t kp, int mte, int mt_off, int mt_total,
                           const XcdPlan& p1, int32_t* __restrict__ tiles1,
                           const XcdPlan& p2, int32_t* __restrict__ tiles2, XcdScratch& x_) {
  const int e = threadIdx.x, lane = e & (kWave - 1), wv = e / kWave, nw = blockDim.x / kWave;
  const bool on1 = tiles1 != nullptr && p1.nt > 0, on2 = tiles2 != nullptr && p2.nt > 0;
  if (e < kXcds) {
    if (on1)
      *reinterpret_cast<unsigned long long*>(tiles1 + tile_claims_at(E) + kClaimStride * e) = 0;
    if (on2)
      *reinterpret_cast<unsigned long long*>(tiles2 + tile_claims_at(E) + kClaimStride * e) = 0;
    x_.sh[0][e] = -1;
    x_.sh[1][e] = -1;
  }
  const float w[2] = {on1 ? gemm_cost(kp, mte, p1) : 0.f, on2 ? gemm_cost(kp, mte, p2) : 0.f};
  // exclusive prefix of both costs over the block (one pass, two barriers)
  float inc[2] = {w[0], w[1]};
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float y = __shfl_up(inc[g], o, kWave);
      if (lane >= o) inc[g] += y;
    }
  }
  if (lane == kWave - 1) {
    x_.wsum[0][wv] = inc[0];
    x_.wsum[1][wv] = inc[1];
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float base = 0.f;
    for (int v = 0; v < wv; ++v) base += x_.wsum[g][v];
    const float P = base + inc[g] - w[g];
    if (e < E) x_.pre[g][e] = P;
    if (e == E - 1) x_.pre[g][E] = P + w[g];
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const XcdPlan& p = g == 0 ? p1 : p2;
    const float total = x_.pre[g][E];
    if (w[g] > 0.f && total > 0.f) {
      const float lo = x_.pre[g][e], hi = x_.pre[g][e + 1];
      for (int x = 1; x < kXcds; ++x) {
        float r = total * static_cast<float>(p.ksplit * x) * (1.f / kXcds);
        int sp = 0;
        while (sp + 1 < p.ksplit && r >= total) {
          r -= total;
          ++sp;
        }
        if (r >= lo && r < hi) {
          int col = static_cast<int>((r - lo) * static_cast<float>(p.nt) / w[g] + 0.5f);
          col = col < 0 ? 0 : (col > p.nt ? p.nt : col);
          x_.sh[g][x] = sp * mt_total * p.nt + mt_off * p.nt + col * mte;
        }
      }
    }
  }
  __syncthreads();
  const int g = e == 0 ? 0 : (e == kWave && nw > 1 ? 1 : -1);
  if (g >= 0 && (g == 0 ? on1 : on2)) {
    const XcdPlan& p = g == 0 ? p1 : p2;
    int32_t* bounds = (g == 0 ? tiles1 : tiles2) + E + 1;
    const int all_tiles = mt_total * p.nt * p.ksplit;
    int prev = 0;
    bounds[0] = 0;
    for (int x = 1; x < kXcds; ++x) {
      int v = x_.sh[g][x];
      const int lo = max(prev, all_tiles - (kXcds - x) * p.cap);
      v = min(max(v, lo), prev + p.cap);
      bounds[x] = v;
      prev = v;
    }
    bounds[kXcds] = all_tiles;
  }
}

// Kept count, per-expert capacity and M-tile counts of one expert, written
// as exclusive prefixes over experts (thread e handles expert e; E <= 1024),
// then each routed GEMM's XCD ranges after its M-tile prefix.
__device__ __forceinline__ int expert_prefixes(int e, int E, int32_t cnt, int64_t S,
                                                int64_t cap, int32_t* __restrict__ counts,
                                                int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ dropped,
                                                int32_t* __restrict__ tiles1,
                                                int32_t* __restrict__ tiles2, int bm,
                                                const XcdPlan& p1, const XcdPlan& p2,
                                                int* wsum) {
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
  if (tiles1 || tiles2) {
    // both GEMMs use bm-row tiles: one M-tile prefix serves both
    int t;
    const int mte = on ? (kp + bm - 1) / bm : 0;
    const int o = block_exclusive_scan(mte, wsum, &t);
    if (on && tiles1) tiles1[e] = o;
    if (on && tiles2) tiles2[e] = o;
    if (threadIdx.x == 0) {
      if (tiles1) tiles1[E] = t;
      if (tiles2) tiles2[E] = t;
    }
    __shared__ XcdScratch xs;
    if ((tiles1 && p1.nt > 0) || (tiles2 && p2.nt > 0))
      xcd_bounds(E, kp, mte, o, t, p1, tiles1, p2, tiles2, xs);
  }
  return off;
}

// One block of 1024 threads (thread e = expert e).  hist[b][e] becomes the
// exclusive base of expert e at block b.
__global__ void __launch_bounds__(1024)
scan_kernel(int32_t* __restrict__ hist, int nb, int E, int64_t S, int64_t cap,
            int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
            int32_t* __restrict__ dropped, int32_t* __restrict__ tiles1,
            int32_t* __restrict__ tiles2, int bm, XcdPlan p1, XcdPlan p2) {
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
  expert_prefixes(e, E, run, S, cap, counts, offsets, dropped, tiles1, tiles2, bm, p1,
                  p2, wsum);
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
tile_prefix_kernel(const int32_t* __restrict__ offsets, int E, int32_t* __restrict__ tiles1,
                   int32_t* __restrict__ tiles2, int bm, XcdPlan p1, XcdPlan p2) {
  __shared__ int wsum[16];
  __shared__ XcdScratch xs;
  const int e = threadIdx.x;
  const int32_t n = e < E ? offsets[e + 1] - offsets[e] : 0;
  const int mte = (n + bm - 1) / bm;
  int t;
  const int o = block_exclusive_scan(mte, wsum, &t);
  if (e < E) {
    tiles1[e] = o;
    tiles2[e] = o;
  }
  if (e == 0) {
    tiles1[E] = t;
    tiles2[E] = t;
  }
  if (p1.nt > 0 || p2.nt > 0) xcd_bounds(E, n, mte, o, t, p1, tiles1, p2, tiles2, xs);
}

// All of the dispatch in one block when the slots fit one chunk (decode-
// sized batches): LDS histogram, prefixes, then the stable rank/scatter of
// scatter_kernel with block base 0.
__global__ void __launch_bounds__(1024)
dispatch_small_kernel(const int32_t* __restrict__ ids, const float* __restrict__ w,
                      int64_t S, int k, int E, int64_t cap, int nbits,
                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                      int32_t* __restrict__ dropped, int32_t* __restrict__ tiles1,
                      int32_t* __restrict__ tiles2, int bm, XcdPlan p1, XcdPlan p2,
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
                                  tiles1, tiles2, bm, p1, p2, wsum);
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
                       tiles1, tiles2, routed_bm(D), xcd_plan(D, false),
                       xcd_plan(D, true), sorted_token, sorted_w, slot_row, err);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(count_kernel, dim3(nblocks), dim3(256), hsz, s, ids,
                     D.slots, D.E, hist, err);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, hist,
                     nblocks, D.E, D.slots, D.cap, counts, offsets, dropped,
                     tiles1, tiles2, routed_bm(D), xcd_plan(D, false),
                     xcd_plan(D, true));
  hipLaunchKernelGGL(scatter_kernel, dim3(nblocks), dim3(256), 6 * hsz, s, ids,
                     w, D.slots, D.k, D.E, D.cap, nbits, hist, offsets,
                     sorted_token, sorted_w, slot_row);
  return hipGetLastError();
}

hipError_t launch_tile_prefix(const Dims& D, const int32_t* offsets,
                              int32_t* tiles1, int32_t* tiles2, hipStream_t s) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, s, offsets, D.E,
                     tiles1, tiles2, routed_bm(D), xcd_plan(D, false),
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
