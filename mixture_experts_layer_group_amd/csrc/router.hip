// Router: logits L = x @ Wr^T (fp32 accumulation on the vector ALUs -- the
// router is the smallest weight of the layer and is kept out of the matrix
// cores), then the top-k selection of either routing kind:
//   SOFTMAX_TOPK  -- Edge0 "MoE Spec and Routing" page, select_from_logits;
//                    "Mixture of Experts" blog page, route (softmax, keep
//                    the k most probable, renormalise over them);
//   SIGMOID_GROUP -- Edge0 page, group_select_from_logits (sigmoid scores,
//                    a selection-only bias, group-limited top-k, routed
//                    scaling).
// Ranking is decided on fp32 values with ties to the lower index, so it is
// reproducible bit for bit; softmax is monotone, so ranking the logits is
// ranking the probabilities.
#include "moe_internal.hpp"

#include <math.h>

#include <algorithm>

namespace moe {
namespace {

template <typename T>
__device__ __forceinline__ float ld1(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld1<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// 8 consecutive elements as fp32 (p + i must be 16-byte aligned for bf16,
// 32-byte for fp32)
__device__ __forceinline__ void ld8(const float* p, int64_t i, float* v) {
  const float4* q = reinterpret_cast<const float4*>(p + i);
  float4 a = q[0], b = q[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void ld8(const uint16_t* p, int64_t i, float* v) {
  uint4 a = *reinterpret_cast<const uint4*>(p + i);
  uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}

// ------------------------------------------------------------------ logits
// Many tokens and many experts: a 128 x 128 (token x expert) tile per
// 256-thread block, 8 x 8 outputs per thread, K staged through LDS in
// chunks of 32, double-buffered (the next chunk is loaded into registers
// while the current one is multiplied).  The reduction over d may be split
// over blockIdx.z: split q writes its partial logits to plane q
// ([S][T][E]) and the selection adds the planes in plane order, so the
// result does not depend on timing.  Every split is at most kper long and
// starts at a multiple of 32; d is a multiple of 8.
//
// Every term is one fp32 FMA (one rounding per product added), so the
// logits meet the forward error bound of a d-term fp32 dot product in any
// order.  bf16 x bf16 is not sent through v_dot2_f32_bf16: measured on
// gfx950 its result can differ from the exact a0*b0 + a1*b1 + c by up to
// 2.5 units of fp32 rounding of |a0 b0| + |a1 b1| + |c|, which over d/2
// steps exceeds that bound.
constexpr int RT = 128, RE = 128, RK = 32;

template <typename XT, typename WT>
__global__ void __launch_bounds__(256)
logits_tile_fma_kernel(const XT* __restrict__ x, const WT* __restrict__ wr,
                       float* __restrict__ L, int64_t T, int E, int d, int kper) {
  __shared__ __attribute__((aligned(16))) float xs[2][RK][RT + 4];
  __shared__ __attribute__((aligned(16))) float ws[2][RK][RE + 4];
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT;
  const int e0 = blockIdx.y * RE;
  const int kbeg = blockIdx.z * kper;
  const int kend = min(d, kbeg + kper);
  const int ty = tid / 16, tx = tid % 16;
  // loader: tile row lr, 16 consecutive K elements from lk
  const int lr = tid >> 1, lk = (tid & 1) * 16;
  const int64_t xt = t0 + lr;
  const int we = e0 + lr;
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  float xv[16], wv[16];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + lk + 8 * h;
      if (xt < T && k < kend) {
        ld8(x, xt * d + k, xv + 8 * h);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[8 * h + j] = 0.f;
      }
      if (we < E && k < kend) {
        ld8(wr, static_cast<int64_t>(we) * d + k, wv + 8 * h);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[8 * h + j] = 0.f;
      }
    }
  };
  auto lstore = [&](int b) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      xs[b][lk + j][lr] = xv[j];
      ws[b][lk + j][lr] = wv[j];
    }
  };
  const int nk = kend > kbeg ? (kend - kbeg + RK - 1) / RK : 0;
  if (nk > 0) {
    gload(kbeg);
    lstore(0);
    __syncthreads();
  }
  for (int c = 0; c < nk; ++c) {
    const int b = c & 1;
    if (c + 1 < nk) gload(kbeg + (c + 1) * RK);
#pragma unroll 4
    for (int kk = 0; kk < RK; ++kk) {
      const float4 a0 = *reinterpret_cast<const float4*>(&xs[b][kk][ty * 8]);
      const float4 a1 = *reinterpret_cast<const float4*>(&xs[b][kk][ty * 8 + 4]);
      const float4 b0 = *reinterpret_cast<const float4*>(&ws[b][kk][tx * 8]);
      const float4 b1 = *reinterpret_cast<const float4*>(&ws[b][kk][tx * 8 + 4]);
      const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float w[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    // buffer b^1 was last read before the previous barrier
    if (c + 1 < nk) lstore(b ^ 1);
    __syncthreads();
  }
  float* P = L + static_cast<int64_t>(blockIdx.z) * T * E;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = t0 + ty * 8 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = e0 + tx * 8 + j;
      if (e < E) P[t * E + e] = acc[i][j];
    }
  }
}

// Few experts (E <= 16): a wave takes TPW = 64/EB tokens and one slice of
// the reduction (blockIdx.y, kper long); lane l handles K elements l*8..+7
// of every 512 of the slice, so the loads of a token row and of a router
// row are contiguous across the wave.  Each lane keeps TPW x EB partial
// dot products (64 of them); a halving butterfly across the lanes then
// leaves lane l with the whole slice's sum for token l/EB, expert l%EB,
// which it writes to the slice's plane of partial logits ([S][T][E]).
template <int D, int CNT>
__device__ __forceinline__ void halve(float (&v)[64], int lane) {
  if constexpr (D >= 1) {
    constexpr int kHalf = CNT / 2;
    const bool upper = (lane & D) != 0;
#pragma unroll
    for (int i = 0; i < kHalf; ++i) {
      const float send = upper ? v[i] : v[i + kHalf];
      const float keep = upper ? v[i + kHalf] : v[i];
      v[i] = keep + xor_move<D>(send, lane);
    }
    halve<D / 2, kHalf>(v, lane);
  }
}

template <typename XT, typename WT, int EB>
__global__ void __launch_bounds__(256)
logits_few_e_kernel(const XT* __restrict__ x, const WT* __restrict__ wr,
                    float* __restrict__ L, int64_t T, int E, int d, int kper) {
  constexpr int TPW = kWave / EB;  // tokens per wave
  const int lane = threadIdx.x % kWave;
  const int64_t t0 = (static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave) * TPW;
  const int kbeg = blockIdx.y * kper;
  const int kend = min(d, kbeg + kper);
  float acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0.f;
  for (int k = kbeg + lane * 8; k < kend; k += kWave * 8) {
    float wv[EB][8];
#pragma unroll
    for (int e = 0; e < EB; ++e) {
      if (e < E) {
        ld8(wr, static_cast<int64_t>(e) * d + k, wv[e]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[e][j] = 0.f;
      }
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      float xv[8];
      if (t0 + t < T) {
        ld8(x, (t0 + t) * d + k, xv);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < EB; ++e)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[t * EB + e] = fmaf(xv[j], wv[e][j], acc[t * EB + e]);
    }
  }
  // lane l ends with the sum of value l (token l / EB, expert l % EB)
  halve<32, 64>(acc, lane);
  const int64_t t = t0 + lane / EB;
  const int e = lane % EB;
  if (t < T && e < E) L[(static_cast<int64_t>(blockIdx.y) * T + t) * E + e] = acc[0];
}

// Few tokens (decode): one wave per (expert row, 4 tokens), lanes split K.
// The loads of up to 4 K steps of 512 (the expert's router row and the 4
// token rows) are all issued before any product, so a row of up to 2048
// elements costs one memory round trip.
template <typename XT, typename WT>
__global__ void __launch_bounds__(256)
logits_rowdot_kernel(const XT* __restrict__ x, const WT* __restrict__ wr,
                     float* __restrict__ L, int64_t T, int E, int d) {
  constexpr int KC = 4;
  const int lane = threadIdx.x % kWave;
  const int e = blockIdx.x * 4 + threadIdx.x / kWave;
  if (e >= E) return;
  const WT* wrow = wr + static_cast<int64_t>(e) * d;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = lane * 8; k0 < d; k0 += kWave * 8 * KC) {
    float wv[KC][8];
    float xv[KC][4][8];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int k = k0 + c * kWave * 8;
      if (k < d) {
        ld8(wrow, k, wv[c]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + i < T) ld8(x, (t0 + i) * d + k, xv[c][i]);
      }
    }
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (k0 + c * kWave * 8 < d) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + i < T) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i] = fmaf(xv[c][i][j], wv[c][j], acc[i]);
          }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s = wave_sum(acc[i]);
    if (lane == 0 && t0 + i < T) L[(t0 + i) * E + e] = s;
  }
}

// ------------------------------------------------------------------ select
// (value, index) order used for every top-k: larger value first, equal
// values ordered by the lower index.
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// the better of two candidates, without branches; a lane with no candidate
// holds (-inf, INT_MAX), which every candidate beats (scores are finite)
__device__ __forceinline__ void take_better(float& v, int& i, float v2, int i2) {
  const bool take = (v2 > v) | ((v2 == v) & (i2 < i));
  v = take ? v2 : v;
  i = take ? i2 : i;
}

template <int CTRL>
__device__ __forceinline__ void best_step(float& v, int& i) {
  take_better(v, i, dpp_f<CTRL>(v), dpp_i<CTRL>(i));
}

// Wave-wide best (value, index) among candidates, the same in every lane;
// lanes without one pass (-inf, INT_MAX).  Rows of 16 lanes first (DPP), then
// the four row winners.
__device__ __forceinline__ void wave_best(float& v, int& i) {
  best_step<kDppXor1>(v, i);
  best_step<kDppXor2>(v, i);
  best_step<kDppHalfMirror>(v, i);
  best_step<kDppMirror>(v, i);
  float bv = lane_f(v, 0);
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r)
    take_better(bv, bi, lane_f(v, 16 * r), __builtin_amdgcn_readlane(i, 16 * r));
  v = bv;
  i = bi;
}

// One wave per token; EPL = experts per lane (expert lane + 64*j).
// The selection of every token t = blockIdx.x * NW + wave, + gridDim.x * NW
// ...: one wave per token.  The routing kind and
// the forced-id replay are template parameters, so each kernel carries only
// its own path.
template <int EPL, int NW, int ROUTER, bool FORCED>
__device__ __forceinline__ void
select_body(const float* __restrict__ L, int S, float* __restrict__ Lout,
            const float* __restrict__ bias, const int32_t* __restrict__ forced,
            int32_t* __restrict__ rejected,
            int32_t* __restrict__ ids, float* __restrict__ wout,
            float* __restrict__ probpart, int32_t* __restrict__ err, int64_t T,
            int E, int k, int norm, float scaling, int n_group, int topk_group) {
  constexpr int router = ROUTER;
  bool nonfinite = false;  // a logit that is NaN or infinite
  __shared__ float sel_lds[NW][EPL * kWave];
  __shared__ float pacc[NW][EPL * kWave];
  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  float pa[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) pa[j] = 0.f;
  const bool want_p = probpart != nullptr;
  const int G = router == MOE_ROUTER_SIGMOID_GROUP ? E / n_group : 0;

  for (int64_t t = static_cast<int64_t>(blockIdx.x) * NW + wv; t < T;
       t += static_cast<int64_t>(gridDim.x) * NW) {
    float v[EPL];
    float sc[EPL];  // sigmoid scores (SIGMOID_GROUP)
    uint32_t cand = 0;  // bit j: expert lane+64j may still be chosen
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + kWave * j;
      float lv = 0.f;
      if (e < E) {
        // partial logit planes added in plane order
        // all planes are loaded before the (in-order) additions
        if (S == 1) {
          lv = L[t * E + e];
        } else {
          float pv[kMaxLogitPlanes];
#pragma unroll
          for (int q = 0; q < kMaxLogitPlanes; ++q)
            pv[q] = q < S ? L[(q * T + t) * E + e] : 0.f;
          lv = pv[0];
#pragma unroll
          for (int q = 1; q < kMaxLogitPlanes; ++q)
            if (q < S) lv += pv[q];
        }
        if (Lout) Lout[t * E + e] = lv;
        nonfinite |= !(fabsf(lv) <= 3.402823466e38f);
      }
      v[j] = lv;
      sc[j] = 0.f;
      if (e < E) cand |= 1u << j;
    }
    if constexpr (ROUTER == MOE_ROUTER_SIGMOID_GROUP) {
      // s = sigmoid(L) held in fp32 (evaluated in fp64, rounded once);
      // selection score s + bias, also fp32
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = lane + kWave * j;
        sc[j] = static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(v[j]))));
        v[j] = sc[j] + ((bias != nullptr && e < E) ? bias[e] : 0.f);
        if (e < E) sel_lds[wv][e] = v[j];
      }
      if (topk_group < n_group && !FORCED) {
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // group score: sum of the two largest selection scores
        float gs = -INFINITY;
        int gi = INT_MAX;
        if (lane < n_group) {
          float a = -INFINITY, b = -INFINITY;
          for (int q = 0; q < G; ++q) {
            const float y = sel_lds[wv][lane * G + q];
            if (y > a) {
              b = a;
              a = y;
            } else if (y > b) {
              b = y;
            }
          }
          gs = a + b;
          gi = lane;
        }
        // keep the best topk_group groups (ties to the lower group)
        uint64_t kept = 0;
        for (int r = 0; r < topk_group; ++r) {
          const bool out = (kept >> lane) & 1ull;
          float bv = out ? -INFINITY : gs;
          int bi = out ? INT_MAX : gi;
          wave_best(bv, bi);
          kept |= 1ull << bi;
        }
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
          const int e = lane + kWave * j;
          if (e < E && !((kept >> (e / G)) & 1ull)) cand &= ~(1u << j);
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    // top-k by repeated wave argmax; lane r keeps the r-th winner
    int my_id = 0;
    float my_val = 0.f;
    bool reject = false;
    if constexpr (FORCED) {
      // router replay: lane r takes the r-th given id; a row that is not k
      // distinct experts in [0, E) is rejected (identity route, weight 0)
      const int fid = lane < k ? forced[t * k + lane] : 0;
      bool bad = lane < k && (fid < 0 || fid >= E);
      for (int j = 0; j < k; ++j) {
        const int o = __builtin_amdgcn_readlane(fid, j);
        if (lane < k && j < lane && o == fid) bad = true;
      }
      reject = __ballot(bad) != 0;
      my_id = reject ? lane : fid;
      if (lane >= k) my_id = 0;
      // the given expert's logit, fetched from the lane that holds it
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const float y = __shfl(v[j], my_id % kWave, kWave);
        if (my_id / kWave == j) my_val = y;
      }
      if (reject && lane == 0) atomicAdd(rejected, 1);
    }
    for (int r = 0; r < k && !FORCED; ++r) {
      float bv = -INFINITY;
      int bi = INT_MAX;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const bool c = (cand >> j) & 1u;
        take_better(bv, bi, c ? v[j] : -INFINITY, c ? lane + kWave * j : INT_MAX);
      }
      wave_best(bv, bi);
      if (lane == r) {
        my_id = bi;
        my_val = bv;
      }
      if ((bi % kWave) == lane) cand &= ~(1u << (bi / kWave));
    }
    float wk;
    if constexpr (ROUTER == MOE_ROUTER_SOFTMAX_TOPK) {
      // the largest logit: the first choice, or for given ids the maximum
      // over all experts (the same value whenever the first choice is given)
      float m = lane_f(my_val, 0);
      if constexpr (FORCED) {
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          if (lane + kWave * j < E) mx = fmaxf(mx, v[j]);
        m = wave_max(mx);
      }
      float S = 0.f;
      if (want_p || !norm) {
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          if (lane + kWave * j < E) part += expf(v[j] - m);
        S = wave_sum(part);
      }
      if (want_p) {
        const float inv = 1.f / S;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          if (lane + kWave * j < E) pa[j] += expf(v[j] - m) * inv;
      }
      const float ex = lane < k ? expf(my_val - m) : 0.f;
      const float den = norm ? wave_sum(ex) : S;
      wk = ex / den;
    } else {
      // raw sigmoid of the chosen expert (bias excluded), fetched from the
      // lane that holds it
      float s_e = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const float y = __shfl(sc[j], my_id % kWave, kWave);
        if (my_id / kWave == j) s_e = y;
      }
      if (lane >= k) s_e = 0.f;
      const float den = wave_sum(s_e) + 1e-20f;
      wk = (norm ? s_e / den : s_e) * scaling;
    }
    if (lane < k) {
      ids[t * k + lane] = my_id;
      wout[t * k + lane] = reject ? 0.f : wk;
    }
  }
  if (err != nullptr && __ballot(nonfinite) != 0 && lane == 0)
    atomicOr(err, MOE_FLAG_NONFINITE_LOGIT);
  if (want_p) {
#pragma unroll
    for (int j = 0; j < EPL; ++j) pacc[wv][lane + kWave * j] = pa[j];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      float s = 0.f;
      for (int q = 0; q < NW; ++q) s += pacc[q][e];
      probpart[static_cast<int64_t>(blockIdx.x) * E + e] = s;
    }
  }
}

template <int EPL, int ROUTER, bool FORCED>
__global__ void __launch_bounds__(256)
select_kernel(const float* __restrict__ L, int S, float* __restrict__ Lout,
              const float* __restrict__ bias, const int32_t* __restrict__ forced,
              int32_t* __restrict__ rejected,
              int32_t* __restrict__ ids, float* __restrict__ wout,
              float* __restrict__ probpart, int32_t* __restrict__ err, int64_t T,
              int E, int k, int norm, float scaling, int n_group, int topk_group) {
  select_body<EPL, kSelectWaves, ROUTER, FORCED>(L, S, Lout, bias, forced, rejected, ids,
                                                 wout, probpart, err, T, E, k, norm,
                                                 scaling, n_group, topk_group);
}


__global__ void prob_finalize_kernel(const float* __restrict__ part, int nb,
                                     int E, float* __restrict__ out) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  // rows added in row order; each group of 16 loaded before it is added
  float s = 0.f;
  for (int b0 = 0; b0 < nb; b0 += 16) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      v[j] = b0 + j < nb ? part[static_cast<int64_t>(b0 + j) * E + e] : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (b0 + j < nb) s += v[j];
  }
  out[e] = s;
}

// one counter cleared by a kernel (safe inside a captured graph)
__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

template <typename XT, typename WT>
hipError_t logits_dispatch(const Dims& D, const RouterPlan& p, const void* x,
                           const void* wr, float* L, hipStream_t s) {
  const XT* xp = static_cast<const XT*>(x);
  const WT* wp = static_cast<const WT*>(wr);
  if (p.kind == kRouterRowdot) {
    dim3 grid((D.E + 3) / 4, static_cast<unsigned>((D.T + 3) / 4));
    hipLaunchKernelGGL((logits_rowdot_kernel<XT, WT>), grid, dim3(256), 0, s,
                       xp, wp, L, D.T, D.E, D.d);
  } else if (p.kind == kRouterSmallE) {
    const int tpw = D.E <= 8 ? 8 : 4;  // 64 / EB tokens per wave
    dim3 grid(static_cast<unsigned>((D.T + 4 * tpw - 1) / (4 * tpw)), p.S);
    if (D.E <= 8)
      hipLaunchKernelGGL((logits_few_e_kernel<XT, WT, 8>), grid, dim3(256), 0,
                         s, xp, wp, L, D.T, D.E, D.d, p.kper);
    else
      hipLaunchKernelGGL((logits_few_e_kernel<XT, WT, 16>), grid, dim3(256), 0,
                         s, xp, wp, L, D.T, D.E, D.d, p.kper);
  } else {
    dim3 grid(static_cast<unsigned>((D.T + RT - 1) / RT), (D.E + RE - 1) / RE, p.S);
    hipLaunchKernelGGL((logits_tile_fma_kernel<XT, WT>), grid, dim3(256), 0, s,
                       xp, wp, L, D.T, D.E, D.d, p.kper);
  }
  return hipGetLastError();
}

}  // namespace

RouterPlan router_plan(const Dims& D) {
  RouterPlan p{};
  p.S = 1;
  p.kper = D.d;
  if (D.T <= 64) {
    p.kind = kRouterRowdot;
  } else if (D.E <= 16) {
    p.kind = kRouterSmallE;
    // about 8 waves per CU of a 256-CU part; slices of whole 512-element
    // steps of a wave
    const int64_t waves = (D.T + (D.E <= 8 ? 8 : 4) - 1) / (D.E <= 8 ? 8 : 4);
    const int steps = (D.d + 511) / 512;
    int S = static_cast<int>(std::min<int64_t>(kMaxLogitPlanes, (2048 + waves - 1) / waves));
    S = std::max(1, std::min(S, steps));
    p.kper = (steps + S - 1) / S * 512;
    p.S = (D.d + p.kper - 1) / p.kper;
  } else {
    p.kind = kRouterTiled;
    // about two blocks per CU of a 256-CU part, each split at least 256 long
    const int64_t tiles = ((D.T + RT - 1) / RT) * ((D.E + RE - 1) / RE);
    int S = static_cast<int>(std::min<int64_t>(kMaxLogitPlanes, (512 + tiles - 1) / tiles));
    S = std::max(1, std::min(S, D.d / 256));
    p.kper = ((D.d + S - 1) / S + RK - 1) / RK * RK;
    p.S = (D.d + p.kper - 1) / p.kper;
  }
  return p;
}

hipError_t launch_router_logits(const Dims& D, const RouterPlan& p, int act_dtype,
                                int router_dtype, const void* x, const void* wr,
                                float* logits, hipStream_t s) {
  const bool xb = act_dtype == MOE_DTYPE_BF16;
  const bool wb = router_dtype == MOE_DTYPE_BF16;
  if (xb && wb) return logits_dispatch<uint16_t, uint16_t>(D, p, x, wr, logits, s);
  if (xb) return logits_dispatch<uint16_t, float>(D, p, x, wr, logits, s);
  if (wb) return logits_dispatch<float, uint16_t>(D, p, x, wr, logits, s);
  return logits_dispatch<float, float>(D, p, x, wr, logits, s);
}

hipError_t launch_zero_i32(int32_t* p, hipStream_t s) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_router_select(const Dims& D, const moe_spec& sp,
                                const float* logits, int S, float* logits_out,
                                const float* bias, const int32_t* forced,
                                int32_t* rejected, int32_t* ids, float* w,
                                float* probpart, int32_t* err, int nblocks,
                                hipStream_t s) {
  const int epl = (D.E + kWave - 1) / kWave;
  const float scaling =
      sp.router == MOE_ROUTER_SIGMOID_GROUP ? sp.routed_scaling : 1.0f;
#define MOE_SELECT3(N, R, F)                                                   \
  hipLaunchKernelGGL((select_kernel<N, R, F>), dim3(nblocks), dim3(256), 0, s,  \
                     logits, S, logits_out, bias, forced, rejected, ids, w,     \
                     probpart, err, D.T, D.E, D.k, sp.norm_topk_prob, scaling,  \
                     sp.n_group, sp.topk_group)
#define MOE_SELECT(N)                                                           \
  {                                                                             \
    const bool f = forced != nullptr;                                           \
    if (sp.router == MOE_ROUTER_SOFTMAX_TOPK) {                                 \
      if (f) MOE_SELECT3(N, MOE_ROUTER_SOFTMAX_TOPK, true);                     \
      else MOE_SELECT3(N, MOE_ROUTER_SOFTMAX_TOPK, false);                      \
    } else {                                                                    \
      if (f) MOE_SELECT3(N, MOE_ROUTER_SIGMOID_GROUP, true);                    \
      else MOE_SELECT3(N, MOE_ROUTER_SIGMOID_GROUP, false);                     \
    }                                                                           \
  }
  if (epl <= 1) MOE_SELECT(1)
  else if (epl <= 2) MOE_SELECT(2)
  else if (epl <= 4) MOE_SELECT(4)
  else if (epl <= 8) MOE_SELECT(8)
  else MOE_SELECT(16)
#undef MOE_SELECT
#undef MOE_SELECT3
  return hipGetLastError();
}

hipError_t launch_prob_finalize(const Dims& D, const float* probpart,
                                int nblocks, float* prob_sum, hipStream_t s) {
  hipLaunchKernelGGL(prob_finalize_kernel, dim3((D.E + 255) / 256), dim3(256),
                     0, s, probpart, nblocks, D.E, prob_sum);
  return hipGetLastError();
}

}  // namespace moe
