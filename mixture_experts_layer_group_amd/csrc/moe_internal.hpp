// Internal declarations shared by the HIP translation units of the MoE
// library.  Not part of the C ABI (that is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) |
         (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ---------------------------------------------------------------- waves
constexpr int kWave = 64;

// Cross-lane moves inside each row of 16 lanes (DPP): every pairing below
// joins the two halves of a group, so after the four of them each row holds
// its reduction in all of its lanes.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sum over the wave: butterflies inside each row of 16 lanes, then the four
// row sums added in a fixed order ((r0 + r1) + (r2 + r3)).  Every lane
// returns the same bits.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// ---------------------------------------------------------------- sizes
// Per-call problem sizes derived from a validated spec.
struct Dims {
  int64_t T;
  int E, k, d, F, S, Fs;
  int64_t slots;      // T * k
  int64_t cap;        // INT64_MAX when unlimited
  bool bf16;          // bf16 activations
  bool u4;            // 4-bit routed weights
  bool swiglu;
  bool fused;         // FUSED_GATE_UP: gate holds [E][2F][d], gate rows first
  bool out_bf16;      // layer output in bf16 (else fp32)
  int router_dtype;   // MOE_DTYPE_* of the router weights
};

// Router logits plan for bf16 activations (matrix cores, router_mfma.hip):
// tiles of 128 tokens x BN experts, the reduction over d split over S
// workgroups whose partial logits the selection adds in order; npass = 3
// when fp32 router weights are split into three bf16 parts.
struct RouterPlan {
  bool mfma;       // false: fp32 activations, vector-ALU kernels, S = 1
  int npass, BN, mtiles, ntiles, kt_total, kt_split, S;
};
RouterPlan router_plan(const Dims& D, int router_dtype);
constexpr int kMaxLogitPlanes = 16;  // largest S

// Workspace carve-up (byte offsets, each 256-aligned).
struct WsLayout {
  size_t logits, w3, probpart, hist, tiles1, tiles2;  // logits: [S][T][E] partials
  size_t topk_ids, topk_w, counts, offsets, sorted_token, sorted_w, slot_row,
      dropped;
  size_t H, Hs, Y, Ypart, Ys;
  size_t total;
  int route_blocks;     // selection kernel grid (prob partial rows)
  int dispatch_blocks;  // count / scatter grid (histogram rows)
};

constexpr int kDispatchChunk = 2048;  // slots per dispatch block
constexpr int kSelectWaves = 4;       // tokens in flight per select block

// GEMM tile rows (M) of the bf16 grouped kernels; the dispatch scan writes
// the per-expert M-tile prefix for them.
constexpr int kGemm1BM = 256;
constexpr int kGemm2BM = 256;

// K splits of the grouped down projection (1 or 2).  Too few output tiles
// for the chip leave its last round of workgroups mostly idle; splitting
// the reduction in two halves the tile length and doubles the tile count.
// Split 1 writes its fp32 partial to a workspace buffer, which the combine
// adds to split 0's rows (in that order) before weighting.  The choice
// depends only on the shapes (sized for a 256-CU part), so the workspace
// layout does not depend on the device.
int down_splits(const Dims& D);

// ---------------------------------------------------------------- launchers
// router.hip
hipError_t launch_router_logits(const Dims& D, int act_dtype, int router_dtype,
                                const void* x, const void* wr, float* logits,
                                hipStream_t s);
// logits: S planes of partial logits [S][T][E], added in plane order;
// logits_out (may be null) receives the summed logits
hipError_t launch_router_select(const Dims& D, const moe_spec& sp,
                                const float* logits, int S, float* logits_out,
                                const float* bias, const int32_t* forced,
                                int32_t* rejected, int32_t* ids, float* w,
                                float* probpart, int nblocks, hipStream_t s);
// *p = 0 by a one-thread kernel
hipError_t launch_zero_i32(int32_t* p, hipStream_t s);
// router_mfma.hip: partial logits of plan p into part ([p.S][T][E]); w3
// holds 3*E*d bf16 when p.npass == 3
hipError_t launch_router_mfma(const Dims& D, const RouterPlan& p, const void* x,
                              const void* wr, uint16_t* w3, float* part,
                              hipStream_t s);
hipError_t launch_prob_finalize(const Dims& D, const float* probpart,
                                int nblocks, float* prob_sum, hipStream_t s);

// dispatch.hip
hipError_t launch_dispatch(const Dims& D, const int32_t* ids, const float* w,
                           int32_t* hist, int nblocks, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_token,
                           float* sorted_w, int32_t* slot_row, int32_t* dropped,
                           int32_t* tiles1, int32_t* tiles2, hipStream_t s);
hipError_t launch_gather_rows(const Dims& D, const int32_t* offsets,
                              const int32_t* sorted_token, const void* x,
                              void* x_perm, hipStream_t s);
hipError_t launch_tile_prefix(const Dims& D, const int32_t* offsets,
                              int32_t* tiles1, int32_t* tiles2, hipStream_t s);

// gemm_bf16.hip (bf16 activations, bf16 weights, MFMA)
hipError_t launch_ffn_bf16(const Dims& D, const int32_t* offsets,
                           const int32_t* tiles1, const int32_t* tiles2,
                           const int32_t* sorted_token, const void* x,
                           const moe_expert_weights& w, void* H, void* Hs,
                           void* Y, float* Ypart, void* Ys, hipStream_t s);
// Y[r] += Ypart[r] for the kept rows (r < offsets[E]): folds the second K
// split into the expert outputs with the combine's own fp32 addition
hipError_t launch_fold_split(const Dims& D, const int32_t* offsets, float* Y,
                             const float* Ypart, hipStream_t s);
// gemm_f32.hip (fp32 activations and weights, VALU)
hipError_t launch_ffn_f32(const Dims& D, const int32_t* offsets,
                          const int32_t* sorted_token, const void* x,
                          const moe_expert_weights& w, void* H, void* Hs,
                          void* Y, void* Ys, hipStream_t s);
// gemm_u4.hip (bf16 activations, 4-bit affine routed weights, VALU)
hipError_t launch_ffn_u4(const Dims& D, int group, const int32_t* offsets,
                         const int32_t* sorted_token, const void* x,
                         const moe_expert_weights& w, void* H, void* Y,
                         hipStream_t s);
// shared experts with bf16 weights on the MFMA kernel (used by the u4 path)
hipError_t launch_shared_bf16(const Dims& D, const void* x,
                              const moe_expert_weights& w, void* Hs, void* Ys,
                              hipStream_t s);

// stats.hip: routing health and the aux-loss-free bias update
hipError_t launch_routing_health(const Dims& D, const int32_t* counts,
                                 const int32_t* offsets, const int32_t* dropped,
                                 const float* prob_sum, float* bias, float step,
                                 moe_health* h, hipStream_t s);

// combine.hip (expert outputs are fp32)
// y_part (may be null): second K split of the expert rows, added to y_rows
hipError_t launch_combine(const Dims& D, const void* y_rows, const float* y_part,
                          const int32_t* slot_row, const float* topk_w,
                          const void* y_shared, void* out, hipStream_t s);

}  // namespace moe
