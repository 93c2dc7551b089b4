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

// The value held by lane (this lane xor D), D in {1, 2, 4, 8, 16, 32}: DPP
// quad permutations for 1 and 2, the row shifts by 4 (each direction serves
// the lanes whose partner stays inside their row of 16), the row rotation by
// 8, and the gfx950 row swaps for 16 and 32.  None goes through LDS.
template <int D>
__device__ __forceinline__ float xor_move(float v, int lane) {
  if constexpr (D == 1) {
    return dpp_f<kDppXor1>(v);
  } else if constexpr (D == 2) {
    return dpp_f<kDppXor2>(v);
  } else if constexpr (D == 4) {
    const float dn = dpp_f<0x114>(v);  // row_shr:4, from lane l-4
    const float up = dpp_f<0x104>(v);  // row_shl:4, from lane l+4
    return (lane & 4) ? dn : up;
  } else if constexpr (D == 8) {
    return dpp_f<0x128>(v);  // row_ror:8, xor 8 inside a row of 16
  } else if constexpr (D == 16) {
    // odd rows of the first result hold the even rows, and the other way
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else {
    static_assert(D == 32, "distance");
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  }
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

// Router logits plan (router.hip), all on the vector ALUs with fp32
// accumulation: a row-dot kernel for decode-sized batches, a kernel for
// few experts (a wave per 64/EB tokens, partial sums reduced across lanes)
// and 128 x 128 tiles for many; the last two may split the reduction over d
// over S blocks, each writing a plane of partial logits ([S][T][E]) that
// the selection adds in plane order.
enum { kRouterRowdot = 0, kRouterSmallE = 1, kRouterTiled = 2 };
struct RouterPlan {
  int kind;  // kRouter*
  int S;     // partial-logit planes (1 unless tiled)
  int kper;  // reduction length of one split
};
RouterPlan router_plan(const Dims& D);
constexpr int kMaxLogitPlanes = 16;  // largest S

// Workspace carve-up (byte offsets, each 256-aligned).
struct WsLayout {
  size_t logits, probpart, hist, tiles1, tiles2;  // logits: [S][T][E] partials
  size_t topk_ids, topk_w, counts, offsets, sorted_token, sorted_w, slot_row,
      dropped;
  size_t H, Hs, Y, Ypart, Ys, X16;
  size_t total;
  int route_blocks;     // selection kernel grid (prob partial rows)
  int dispatch_blocks;  // count / scatter grid (histogram rows)
};

constexpr int kDispatchChunk = 2048;  // slots per dispatch block
constexpr int kSelectWaves = 4;       // tokens in flight per select block

// Tile rows (M) of the routed grouped GEMMs (gemm_bf16.hip), 128 or 256,
// from the shapes only.  bf16 weights: 256 (measured: 128-row tiles with
// three LDS stages stream each weight panel for twice as many row blocks and
// were 15% slower on the DeepSeek-style down projection, no faster
// elsewhere).  4-bit weights: 128-row tiles below 64 kept rows per expert on
// average (less padding; 20% faster at 8-32 rows per expert), 256 above.
// The dispatch scan writes the per-expert M-tile prefix for this size.
int routed_bm(const Dims& D);

// How the routed grouped GEMM's tiles are shared out over the chip's 8 XCDs
// (hardware dispatch sends workgroup i to XCD i mod 8).  Each XCD takes a
// contiguous range of the tile list (so tiles sharing weights and rows meet
// in its L2), the ranges cut at equal estimated cost rather than equal
// count: a tile of b 32-row blocks costs kt*b + c (kt K steps; c the part of
// a K step that does not shrink with the rows, times kt, plus the tile's
// set-up and epilogue, in the same units), so XCDs given many short tiles
// (skewed routing, ragged tails) take more of them.  No range holds more
// than `cap` tiles, the workgroups one XCD receives.  The dispatch (or the
// tile-prefix kernel) writes the kXcds + 1 boundaries after the E + 1
// M-tile prefixes; nt == 0: no routed tiled GEMM runs.  The first three
// quarters of a range go to the XCD's workgroups by their order; the last
// quarter is claimed at run time through one 64-bit counter per XCD (low
// half: the XCD's own claims from the front, high half: other XCDs' claims
// from the back, the claim valid while the two sum to less than the
// quarter), so XCDs that finish early take over tiles of slower ones.  The
// producer of the boundaries zeroes the counters.
constexpr int kXcds = 8;  // (dispatch.hip divides by it with a shift)
struct XcdPlan {
  int nt = 0;      // N tiles
  int ksplit = 1;  // K splits (the tile list repeats once per split)
  int kt = 0;      // K steps per tile
  int c = 0;       // cost of a tile beyond kt per 32-row block
  int cap = 0;     // workgroups per XCD in the launch
};
XcdPlan xcd_plan(const Dims& D, bool down);
// Workgroups per XCD that may take tiles of other XCDs' last quarters (the
// grid's other surplus workgroups exit without touching memory).
constexpr int kStealers = 64;
// A tile-prefix buffer (int32 entries, 128-byte aligned): E + 1 prefixes,
// kXcds + 1 boundaries, then kXcds 64-bit claim counters, one per 128-byte
// line (kClaimStride entries apart).
constexpr int kClaimStride = 32;
__host__ __device__ inline int64_t tile_claims_at(int64_t E) {
  return (E + 1 + kXcds + 1 + kClaimStride - 1) / kClaimStride * kClaimStride;
}
__host__ __device__ inline int64_t tile_plan_entries(int64_t E) {
  return tile_claims_at(E) + kClaimStride * kXcds;
}

// K splits of the grouped down projection (1 or 2).  Too few output tiles
// for the chip leave its last round of workgroups mostly idle; splitting
// the reduction in two halves the tile length and doubles the tile count.
// Split 1 writes its fp32 partial to a workspace buffer, which the combine
// adds to split 0's rows (in that order) before weighting.  The choice
// depends only on the shapes (sized for a 256-CU part), so the workspace
// layout does not depend on the device.
int down_splits(const Dims& D);

// ---------------------------------------------------------------- launchers
// Every FFN launcher records `mid` (when not null) on the stream between its
// gate/up kernel and its down kernel, for profiling.
// router.hip
hipError_t launch_router_logits(const Dims& D, const RouterPlan& p, int act_dtype,
                                int router_dtype, const void* x, const void* wr,
                                float* logits, hipStream_t s);
// logits: S planes of partial logits [S][T][E], added in plane order;
// logits_out (may be null) receives the summed logits
hipError_t launch_router_select(const Dims& D, const moe_spec& sp,
                                const float* logits, int S, float* logits_out,
                                const float* bias, const int32_t* forced,
                                int32_t* rejected, int32_t* ids, float* w,
                                float* probpart, int32_t* err, int nblocks,
                                hipStream_t s);
// *p = 0 by a one-thread kernel
hipError_t launch_zero_i32(int32_t* p, hipStream_t s);
hipError_t launch_prob_finalize(const Dims& D, const float* probpart,
                                int nblocks, float* prob_sum, hipStream_t s);

// dispatch.hip
hipError_t launch_dispatch(const Dims& D, const int32_t* ids, const float* w,
                           int32_t* hist, int nblocks, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_token,
                           float* sorted_w, int32_t* slot_row, int32_t* dropped,
                           int32_t* tiles1, int32_t* tiles2, int32_t* err,
                           hipStream_t s);
hipError_t launch_gather_rows(const Dims& D, const int32_t* offsets,
                              const int32_t* sorted_token, const void* x,
                              void* x_perm, hipStream_t s);
hipError_t launch_tile_prefix(const Dims& D, const int32_t* offsets,
                              int32_t* tiles1, int32_t* tiles2, hipStream_t s);

// Expert FFN launchers.  row_scale (device [T*k] fp32, or nullptr): each
// routed expert row r of Y is multiplied by row_scale[r] (its routing
// weight) as it is written; shared-expert rows never are.  y16: the routed
// rows (and the down projection's second K split) are written as fp16
// (saturating at +-65504, MOE_FLAG_Y_SATURATED), for the layer's combine.
// gemm_bf16.hip (bf16 activations, bf16 weights, MFMA)
hipError_t launch_ffn_bf16(const Dims& D, const int32_t* offsets,
                           const int32_t* tiles1, const int32_t* tiles2,
                           const int32_t* sorted_token, const void* x,
                           const moe_expert_weights& w, const float* row_scale, bool y16,
                           void* H, void* Hs, void* Y, float* Ypart, void* Ys, int32_t* err,
                           hipEvent_t mid, hipStream_t s);
// Y[r] += Ypart[r] for the kept rows (r < offsets[E]): folds the second K
// split into the expert outputs with the combine's own fp32 addition
hipError_t launch_fold_split(const Dims& D, const int32_t* offsets, float* Y,
                             const float* Ypart, hipStream_t s);
// gemm_f32.hip (fp32 activations and weights, VALU)
hipError_t launch_ffn_f32(const Dims& D, const int32_t* offsets,
                          const int32_t* sorted_token, const void* x,
                          const moe_expert_weights& w, const float* row_scale, void* H,
                          void* Hs, void* Y, void* Ys, hipEvent_t mid, hipStream_t s);
// gemm_u4.hip (bf16 activations, 4-bit affine routed weights, VALU)
hipError_t launch_ffn_u4(const Dims& D, int group, const int32_t* offsets,
                         const int32_t* sorted_token, const void* x,
                         const moe_expert_weights& w, const float* row_scale, void* H,
                         void* Y, int32_t* err, hipEvent_t mid, hipStream_t s);
// gemm_bf16.hip: 4-bit routed weights on the tiled matrix-core kernel
// (dequantised in the K loop), for groups of many rows; d and F multiples of
// 128; tiles1 / tiles2 as for launch_ffn_bf16; X16: workspace [T][d] for
// the fp16 copy of x both products are formed from
hipError_t launch_ffn_u4_tiled(const Dims& D, const int32_t* offsets, const int32_t* tiles1,
                               const int32_t* tiles2, const int32_t* sorted_token,
                               const void* x, void* X16, const moe_expert_weights& w,
                               const float* row_scale, bool y16, void* H, void* Y,
                               int32_t* err, hipEvent_t mid, hipStream_t s);
// whether a 4-bit layer runs the tiled kernels (true) or the weight-stream
// kernels of gemm_u4.hip (false); depends on the shapes only
bool u4_tiled(const Dims& D);
// shared experts with bf16 weights on the MFMA kernel (used by the u4 path)
hipError_t launch_shared_bf16(const Dims& D, const void* x,
                              const moe_expert_weights& w, void* Hs, void* Ys,
                              int32_t* err, hipStream_t s);

// stats.hip: routing health and the aux-loss-free bias update
hipError_t launch_routing_health(const Dims& D, const int32_t* counts,
                                 const int32_t* offsets, const int32_t* dropped,
                                 const float* prob_sum, float* bias, float step,
                                 moe_health* h, hipStream_t s);

// combine.hip (expert outputs are fp32)
// y_part (may be null): second K split of the expert rows, added to y_rows
// y16: y_rows and y_part hold fp16 rows
hipError_t launch_combine(const Dims& D, const void* y_rows, const void* y_part, bool y16,
                          const int32_t* slot_row, const float* topk_w,
                          const void* y_shared, void* out, hipStream_t s);

}  // namespace moe
