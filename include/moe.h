/*
 * moe.h -- C ABI of the sparse Mixture-of-Experts layer forward on MI355X
 * (gfx950): route -> dispatch -> grouped expert FFN -> combine.
 *
 * The pipeline and its four stages follow the dockyard_rl design doc
 * "Mixture-of-Experts", section "The pipeline".  Every entry point below
 * names the passage that defines its operation.
 *
 * Conventions shared by every call
 *   - All tensors are row-major and contiguous.  Pointers marked "device"
 *     point to GPU memory; "host" pointers are ordinary host memory.
 *   - The caller owns every buffer.  The library allocates nothing and
 *     keeps no state between calls, so calls are reentrant; calls that
 *     share a workspace must not overlap.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t, NULL =
 *     the null stream).  Outputs are valid once the stream reaches the
 *     call.  No call synchronises the host or copies device data to it.
 *   - Arguments are validated on the host before anything is launched; on
 *     any error status nothing is launched and nothing is written.
 *   - T = 0 is a valid no-op.
 *   - bf16 tensors hold IEEE bfloat16 bit patterns (uint16 storage).
 *   - Non-finite inputs are outside the contract.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,        /* inconsistent spec field (see moe_spec_validate) */
  MOE_ERR_INVALID_TOPK = 2,       /* top_k outside [1, num_experts] */
  MOE_ERR_CAPACITY_TOO_TIGHT = 3, /* 0 < capacity_factor < 1 */
  MOE_ERR_SHAPE = 4,              /* null / misaligned required pointer, bad T */
  MOE_ERR_WORKSPACE = 5,          /* workspace missing or too small */
  MOE_ERR_HIP = 6,                /* a HIP launch failed */
  MOE_ERR_UNSUPPORTED = 7         /* valid spec this build has no kernel for */
} moe_status;

/* Routing kinds, Edge0 "MoE Spec and Routing" page, RouterKind. */
enum { MOE_ROUTER_SOFTMAX_TOPK = 0, MOE_ROUTER_SIGMOID_GROUP = 1 };
/* Expert activations: SwiGLU silu(gate)*up (Edge0 page, _swiglu), and the
 * ReLU two-layer MLP of the "Mixture of Experts" blog page (expert_forward). */
enum { MOE_ACT_SWIGLU = 0, MOE_ACT_RELU = 1 };
/* Storage types.  U4_AFFINE: Edge0 page, QuantSpec (bits 4, group 64,
 * mode affine). */
enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1, MOE_DTYPE_U4_AFFINE = 2 };
/* Expert weight layouts, Edge0 page, WeightLayout: SEPARATE stacks gate,
 * up and down one tensor each; FUSED_GATE_UP stacks each expert's gate
 * rows directly above its up rows in one tensor (twice the out rows, the
 * two slices interleaved expert by expert), down separate. */
enum { MOE_LAYOUT_SEPARATE = 0, MOE_LAYOUT_FUSED_GATE_UP = 1 };

/* Data-dependent conditions found on the device.  Calls that take an
 * `errors` word (device int32, or NULL when not wanted) OR these bits into
 * it and never clear it, so one word can collect a whole sequence of calls:
 * zero it before the first call whose conditions you want to see.  None of
 * them stops the computation.  The dockyard_rl "Mixture-of-Experts" page
 * ("Router replay (R3)") asks that a bad route be reported rather than
 * silently mis-handled; these bits are how the device reports one.
 *   MOE_FLAG_BAD_EXPERT_ID   moe_dispatch met an expert id outside [0,E);
 *                            that slot is treated as dropped (slot_row -1)
 *   MOE_FLAG_H_SATURATED     a hidden activation (silu(gate)*up, or the
 *                            ReLU output) of the bf16 / 4-bit path was
 *                            outside the fp16 range (or NaN) and was stored
 *                            as +-65504
 *   MOE_FLAG_NONFINITE_LOGIT a router logit was NaN or infinite (an input
 *                            outside the contract; the routing of that
 *                            token is then undefined)
 *   MOE_FLAG_X_SATURATED     a 4-bit layer on the tiled kernels met an
 *                            activation outside the fp16 range (or NaN);
 *                            its fp16 copy was stored as +-65504
 *   MOE_FLAG_Y_SATURATED     moe_layer_forward on the matrix-core kernels
 *                            (bf16 layers, 4-bit layers on the tiled
 *                            kernels) keeps the expert rows in fp16: an
 *                            expert output outside the fp16 range (or NaN)
 *                            was stored as +-65504 */
enum {
  MOE_FLAG_BAD_EXPERT_ID = 1,
  MOE_FLAG_H_SATURATED = 2,
  MOE_FLAG_NONFINITE_LOGIT = 4,
  MOE_FLAG_X_SATURATED = 8,
  MOE_FLAG_Y_SATURATED = 16
};

/* Everything the math depends on; the subset of the Edge0 page's MoESpec
 * (and the blog page's MoEConfig) that changes results. */
typedef struct moe_spec {
  int32_t num_experts;     /* E routed experts, >= 2 */
  int32_t top_k;           /* k experts per token, 1 <= k <= E */
  int32_t hidden;          /* d, token width */
  int32_t ffn;             /* F, routed expert FFN width */
  int32_t router;          /* MOE_ROUTER_* */
  int32_t norm_topk_prob;  /* 1: renormalise the kept weights */
  float routed_scaling;    /* SIGMOID_GROUP weight multiplier (1.0 if unused) */
  int32_t n_group;         /* SIGMOID_GROUP: groups of E/n_group contiguous experts */
  int32_t topk_group;      /* SIGMOID_GROUP: surviving groups */
  double capacity_factor;  /* 0 = unlimited; otherwise >= 1 */
  int32_t shared_experts;  /* always-on experts, added unweighted */
  int32_t shared_ffn;      /* their FFN width */
  int32_t act;             /* MOE_ACT_* */
  int32_t act_dtype;       /* F32 or BF16: x, hidden H, expert outputs, out,
                              shared-expert weights */
  int32_t weight_dtype;    /* routed expert weights: F32, BF16 or U4_AFFINE */
  int32_t router_dtype;    /* router weight Wr: F32 or BF16 */
  int32_t quant_group;     /* U4_AFFINE group size along K (64) */
  int32_t out_dtype;       /* F32 or BF16: the layer output (the combine
                              accumulates in fp32 either way) */
  int32_t layout;          /* MOE_LAYOUT_*: how gate and up are stored */
} moe_spec;

/* Expert weights, device pointers.  SEPARATE layout (Edge0 page,
 * WeightLayout): one stacked tensor per projection with the expert on axis
 * 0, each matrix [out, in] row-major (K contiguous), applied as x @ W^T.
 *   gate : [E, F, d]  (SwiGLU gate; the ReLU expert's input matrix)
 *   up   : [E, F, d]  (SwiGLU only; NULL for ReLU)
 *   down : [E, d, F]  (the output matrix for both activations)
 * For U4_AFFINE the three pointers hold packed codes as uint32 words
 * [E, N, K/8] (element 8j+i of a row in nibble i of word j, low nibble
 * first) and *_scale / *_bias hold bf16 [E, N, K/quant_group]; the weight
 * is scale*q + bias.
 * Shared experts (act dtype, never quantised): shared_gate [S, Fs, d],
 * shared_up [S, Fs, d] (SwiGLU), shared_down [S, d, Fs].
 * FUSED_GATE_UP layout (SwiGLU only): gate points to the fused tensor
 * [E, 2F, d] whose expert e holds its F gate rows followed by its F up rows
 * (for U4_AFFINE: codes [E, 2F, d/8], gate_scale / gate_bias
 * [E, 2F, d/quant_group]), shared_gate to [S, 2Fs, d] likewise; up,
 * up_scale, up_bias and shared_up must be NULL (MOE_ERR_INVALID_ARG
 * otherwise).  The kernels read the fused tensor in place. */
typedef struct moe_expert_weights {
  const void* gate;
  const void* up;
  const void* down;
  const void* gate_scale;
  const void* gate_bias;
  const void* up_scale;
  const void* up_bias;
  const void* down_scale;
  const void* down_bias;
  const void* shared_gate;
  const void* shared_up;
  const void* shared_down;
} moe_expert_weights;

/* Optional device outputs of moe_layer_forward; any member may be NULL.
 *   topk_ids [T,k] int32, topk_w [T,k] fp32, logits [T,E] fp32,
 *   counts_pre [E] int32 (slots per expert before capacity),
 *   offsets [E+1] int32 (kept rows per expert, exclusive prefix),
 *   dropped [1] int32, prob_sum [E] fp32 (sum over tokens of the softmax
 *   probabilities; SOFTMAX_TOPK only),
 *   slot_row [T,k] int32, sorted_token [T*k] int32,
 *   errors [1] int32: MOE_FLAG_* bits of this call are OR-ed in (the word
 *     is not cleared by the call).
 * ffn_events: host pointer to three hipEvent_t (or NULL), recorded on the
 *   stream right before the first expert-FFN kernel, between the routed
 *   gate/up kernel and the routed down kernel, and right after the last
 *   expert-FFN kernel (shared experts included) -- the expert GEMMs exactly
 *   as this call issues them, for profiling. */
typedef struct moe_layer_stats {
  int32_t* topk_ids;
  float* topk_w;
  float* logits;
  int32_t* counts_pre;
  int32_t* offsets;
  int32_t* dropped;
  float* prob_sum;
  int32_t* slot_row;
  int32_t* sorted_token;
  int32_t* errors;
  void* const* ffn_events;
} moe_layer_stats;

/* hipStream_t, passed as an opaque pointer. */
typedef void* moe_stream_t;

/* Host-only check of a spec for T tokens (no GPU work).  Errors, after the
 * validation of the blog page's MoEConfig / Router / MoELayer:
 *   MOE_ERR_INVALID_TOPK        k outside [1, E]
 *   MOE_ERR_CAPACITY_TOO_TIGHT  0 < capacity_factor < 1
 *   MOE_ERR_INVALID_ARG         E < 2; d, F < 1; unknown enum (out_dtype
 *     must be F32 or BF16); negative
 *     capacity factor; SIGMOID_GROUP with n_group < 1, E % n_group != 0,
 *     E/n_group < 2 (a group's top-two is undefined), topk_group outside
 *     [1, n_group], or k > topk_group*E/n_group; shared experts with
 *     shared_ffn < 1; U4_AFFINE with quant_group != 64 or d, F not
 *     multiples of it; BF16 activations with F32 routed weights;
 *     layout not a MOE_LAYOUT_* value; FUSED_GATE_UP with ReLU
 *   MOE_ERR_SHAPE               T < 0 or T*max(k,1) above 2^31 - 1
 *   MOE_ERR_UNSUPPORTED         F32 activations with non-F32 weights;
 *     d not a multiple of 8; BF16 activations whose d, F or shared_ffn is
 *     not a multiple of 64; E > 1024; k > 64; n_group > 64; U4_AFFINE
 *     whose d and F are neither powers of two up to 2048 with SwiGLU (the
 *     weight-stream kernels) nor multiples of 128 (the tiled kernels);
 *     bf16 tensors (x, the hidden rows, one expert matrix) of 4 GiB or more */
moe_status moe_spec_validate(const moe_spec* spec, int64_t T);

/* Per-expert capacity, "Mixture of Experts" blog page, first program's
 * moe_layer and second program's MoEConfig.capacity_for:
 * max(1, int(T*k/E*capacity_factor)) in double precision, left to right,
 * truncated; INT64_MAX when capacity_factor is 0 (unlimited).
 * cap_out: host.  Errors as moe_spec_validate. */
moe_status moe_capacity(const moe_spec* spec, int64_t T, int64_t* cap_out);

/* Bytes of device workspace that moe_layer_forward needs for T tokens; the
 * same size is enough for every stage call below.  bytes: host. */
moe_status moe_workspace_size(const moe_spec* spec, int64_t T, size_t* bytes);

/* Router: logits L = x @ Wr^T accumulated in fp32 on the vector ALUs (one
 * fp32 FMA per term, so within the d-term dot-product error bound; the
 * matrix cores are left to the expert GEMMs), then
 *  SOFTMAX_TOPK (Edge0 page, select_from_logits; blog page, route): the k
 *    most probable experts, highest first, ties to the lower index; weight
 *    p_i / sum of the kept p when norm_topk_prob, else p_i;
 *  SIGMOID_GROUP (Edge0 page, group_select_from_logits): s = sigmoid(L),
 *    selection score s + expert_bias, groups ranked by the sum of their
 *    top-two selection scores, best topk_group groups kept (ties to the
 *    lower group), top-k inside them (ties to the lower index); weight = raw
 *    s, divided by (sum + 1e-20) when norm_topk_prob, times routed_scaling.
 *  x          device [T,d] act dtype
 *  w_router   device [E,d] router dtype
 *  expert_bias device [E] fp32, SIGMOID_GROUP only, or NULL
 *               (non-NULL with SOFTMAX_TOPK is MOE_ERR_INVALID_ARG)
 *  topk_ids   device out [T,k] int32;  topk_w device out [T,k] fp32
 *  logits     device out [T,E] fp32 or NULL
 *  prob_sum   device out [E] fp32 (sum over tokens of softmax p) or NULL;
 *             SOFTMAX_TOPK only, summed in a fixed order (deterministic)
 *  errors     device [1] int32 or NULL: MOE_FLAG_NONFINITE_LOGIT is OR-ed in
 *  workspace  device, at least moe_workspace_size bytes */
moe_status moe_route(const moe_spec* spec, int64_t T, const void* x,
                     const void* w_router, const float* expert_bias,
                     int32_t* topk_ids, float* topk_w, float* logits,
                     float* prob_sum, int32_t* errors, void* workspace,
                     size_t ws_bytes, moe_stream_t stream);

/* Router replay (dockyard "Mixture-of-Experts" page, "Router replay (R3)"):
 * the expert ids of each token are given -- recorded when the tokens were
 * generated -- and only the gating weights come from the model's own gate
 * on the same logits L = x @ Wr^T as moe_route:
 *  SOFTMAX_TOPK: w_i = p[id_i] with p = softmax(L), divided by the given
 *    ids' total probability when norm_topk_prob;
 *  SIGMOID_GROUP: w_i = sigmoid(L)[id_i] (no bias, no group restriction:
 *    both only steer a selection), divided by (their sum + 1e-20) when
 *    norm_topk_prob, times routed_scaling.
 * Forcing the ids moe_route chose for the same x reproduces its weights
 * exactly.  A row that is not k distinct ids in [0,E) (a sentinel such as
 * -1 for a route that was never recorded, a repeat, an out-of-range id) is
 * rejected, not replayed: it gets the ids 0..k-1 with zero weights, so it
 * passes through dispatch and combine and contributes nothing, and it is
 * counted in *rejected.
 *  forced_ids device [T,k] int32, any values
 *  rejected   device out [1] int32, number of rejected rows
 *  other arguments as moe_route (prob_sum: softmax p over every token,
 *  rejected rows included)
 * Errors: the spec's; MOE_ERR_SHAPE for a missing x, w_router, forced_ids,
 * topk_ids, topk_w or rejected, or unaligned x / w_router;
 * MOE_ERR_WORKSPACE for a missing or short workspace.  T = 0 is a no-op
 * that writes nothing. */
moe_status moe_route_forced(const moe_spec* spec, int64_t T, const void* x,
                            const void* w_router, const int32_t* forced_ids,
                            int32_t* topk_ids, float* topk_w, float* logits,
                            float* prob_sum, int32_t* rejected,
                            void* workspace, size_t ws_bytes,
                            moe_stream_t stream);

/* Dispatch with capacity, blog page first program's moe_layer (arrival
 * order) and third program's route_and_sort (stable sort by expert):
 * slots (t,i) are visited in token order; expert e keeps its first
 * `capacity` slots, later ones are dropped.
 *  topk_ids     device [T,k] int32 (values must lie in [0,E))
 *  topk_w       device [T,k] fp32
 *  counts_pre   device out [E] int32, slots per expert before capacity
 *  offsets      device out [E+1] int32, exclusive prefix of kept counts
 *  sorted_token device out [T*k] int32, token of each kept row
 *               (expert-major, token order inside an expert); rows past
 *               offsets[E] are left untouched
 *  sorted_w     device out [T*k] fp32, routing weight of each kept row
 *  slot_row     device out [T,k] int32, row of slot (t,i) or -1 if dropped
 *  dropped      device out [1] int32 = T*k - offsets[E]
 *  x, x_perm    optional: when both non-NULL, x_perm[r] = x[sorted_token[r]]
 *               ([T*k, d] act dtype; the blog page's permuted copy)
 *  errors       device [1] int32 or NULL: MOE_FLAG_BAD_EXPERT_ID is OR-ed
 *               in when a topk_ids value lies outside [0,E) (that slot is
 *               dropped: slot_row -1, not counted in counts_pre)
 *  workspace    device, at least moe_workspace_size bytes */
moe_status moe_dispatch(const moe_spec* spec, int64_t T,
                        const int32_t* topk_ids, const float* topk_w,
                        int32_t* counts_pre, int32_t* offsets,
                        int32_t* sorted_token, float* sorted_w,
                        int32_t* slot_row, int32_t* dropped, const void* x,
                        void* x_perm, int32_t* errors, void* workspace,
                        size_t ws_bytes, moe_stream_t stream);

/* Grouped expert FFN over the ragged expert groups (dockyard page,
 * "The pipeline", grouped GEMM; blog page third program's moe_forward):
 * for every expert e and every kept row r in [offsets[e], offsets[e+1]),
 *   y_rows[r] = FFN_e(x[sorted_token[r]])                (sorted_w NULL)
 *   y_rows[r] = sorted_w[r] * FFN_e(x[sorted_token[r]])  (otherwise: the
 *     routing weight applied in the down product's epilogue, after its fp32
 *     accumulation, instead of in the combine)
 * and for every shared expert s and token t
 *   y_shared[s*T + t] = FFN_shared_s(x[t]).
 * SwiGLU: W_down (silu(W_gate x) * (W_up x)); ReLU: W_down relu(W_gate x).
 * bf16 activations use matrix cores with fp32 accumulation: bf16 x bf16
 * for the gate/up product, whose hidden activation is rounded to fp16
 * (saturating at +-65504), then fp16 x fp16 for the down product (the bf16
 * weights are rounded to the nearest fp16 in registers: exact for
 * magnitudes from 2^-17 to 65504); expert outputs stay fp32.
 * 4-bit weights (Edge0 page, QuantSpec): decode-sized groups (under 32 kept
 * rows per expert on average) stream each expert's codes once per 4 rows
 * with the affine term factored per group; larger groups run 256 x 256
 * matrix-core tiles that dequantise scale*q + bias to fp16 in the K loop,
 * against an fp16 copy of x (MOE_FLAG_X_SATURATED if x leaves fp16 range).
 *  offsets, sorted_token  device, as produced by moe_dispatch
 *  x         device [T,d] act dtype
 *  weights   host struct of device pointers
 *  sorted_w  device [T*k] fp32 (moe_dispatch's sorted_w), or NULL
 *  y_rows    device out [T*k, d] fp32 (rows >= offsets[E] untouched)
 *  y_shared  device out [S*T, d] fp32, or NULL when S = 0
 *  errors    device [1] int32 or NULL: MOE_FLAG_H_SATURATED is OR-ed in */
moe_status moe_grouped_ffn(const moe_spec* spec, int64_t T,
                           const int32_t* offsets, const int32_t* sorted_token,
                           const void* x, const moe_expert_weights* weights,
                           const float* sorted_w, void* y_rows, void* y_shared,
                           int32_t* errors,
                           void* workspace, size_t ws_bytes,
                           moe_stream_t stream);

/* Combine, dockyard page "The pipeline" (weighted scatter back) and blog
 * page third program (scatter-add; a token routed to k experts sums k
 * contributions):
 *   out[t] = sum_{i: slot_row[t,i] >= 0} topk_w[t,i] * y_rows[slot_row[t,i]]
 *            + sum_s y_shared[s*T + t]
 * accumulated in fp32 in the fixed order i = 0..k-1 then s (no atomics);
 * dropped slots add nothing and the kept weights are not renormalised.
 * With topk_w NULL each kept row is added unscaled: the rows already carry
 * their weights (moe_grouped_ffn with sorted_w).
 *  y_rows device [T*k, d] fp32, y_shared device [S*T, d] fp32 or NULL
 *  slot_row device [T,k] int32, topk_w device [T,k] fp32 or NULL
 *  out device out [T,d] out dtype */
moe_status moe_combine(const moe_spec* spec, int64_t T, const void* y_rows,
                       const int32_t* slot_row, const float* topk_w,
                       const void* y_shared, void* out, moe_stream_t stream);

/* The whole layer forward (dockyard page, "The pipeline"): moe_route ->
 * moe_dispatch -> moe_grouped_ffn -> moe_combine on one stream, with
 * ragged sizes kept on the device.  On the matrix-core kernels (bf16
 * layers, 4-bit layers on the tiled kernels) the expert rows pass from the
 * down product to the combine in fp16 (each part of a row rounded once,
 * saturating at +-65504 with MOE_FLAG_Y_SATURATED); the combine sums in
 * fp32.  Returns the MoE branch only (the
 * residual add belongs to the caller): a token whose slots were all
 * dropped and which has no shared expert gets exactly 0.
 *  x, w_router, expert_bias  as moe_route
 *  weights   host struct of device pointers (see moe_expert_weights)
 *  out       device out [T,d] out dtype
 *  stats     host struct of optional device outputs, or NULL
 *  workspace device, at least moe_workspace_size bytes */
moe_status moe_layer_forward(const moe_spec* spec, int64_t T, const void* x,
                             const void* w_router, const float* expert_bias,
                             const moe_expert_weights* weights, void* out,
                             const moe_layer_stats* stats, void* workspace,
                             size_t ws_bytes, moe_stream_t stream);

/* Bytes of the library's static scratch array on each GPU (64 MiB). */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_layer_forward without a workspace argument and without any device
 * allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The workspace is a static array of MOE_STATIC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends; the call
 * itself allocates nothing (no hipMalloc, no hipFree, no allocating library
 * routine).  Every call on one GPU uses that GPU's same array: calls that
 * overlap on one GPU (concurrent streams, or threads sharing a device) race
 * and must be serialised by the caller.  The array keeps the last call's
 * contents; nothing in the layer depends on them.
 * Arguments, results and errors as moe_layer_forward; a layer whose
 * moe_workspace_size exceeds MOE_STATIC_SCRATCH_BYTES returns
 * MOE_ERR_WORKSPACE with nothing launched (e.g. decode-shaped batches fit,
 * the 4096-token Mixtral-shaped layer does not).  MOE_ERR_HIP if the
 * array's device address cannot be obtained. */
moe_status moe_layer_forward_static(const moe_spec* spec, int64_t T, const void* x,
                                    const void* w_router, const float* expert_bias,
                                    const moe_expert_weights* weights, void* out,
                                    const moe_layer_stats* stats, moe_stream_t stream);

/* Routing health of one layer call, from its dispatch counts (device
 * struct, filled by moe_routing_health).  Definitions follow the "Mixture
 * of Experts" blog page (second program's RoutingHealth, third program's
 * routing_health and load_balancing_loss) with kept_e = offsets[e+1] -
 * offsets[e], shares s_e = kept_e / T and P_e = prob_sum[e] / T:
 *   aux        E * sum_e (kept_e / (T*k)) * P_e   (1 under uniform routing;
 *              0 when prob_sum is NULL, e.g. SIGMOID_GROUP)
 *   aux3       E * sum_e (kept_e / T) * P_e = k * aux (the pages' code)
 *   entropy    -sum_e q_e log q_e over q_e = s_e / sum s (q_e > 0)
 *   max_entropy log E;  entropy_ratio = entropy / max_entropy
 *   max_share  max_e q_e;  collapsed = entropy_ratio < 0.5
 *   dropped_fraction  dropped / (T*k)
 *   load_peak_over_mean  max_e count_pre_e / mean_e count_pre_e (pre-drop)
 * All zero-share cases give 0 (no division by zero). */
typedef struct moe_health {
  float aux;
  float aux3;
  float entropy;
  float max_entropy;
  float entropy_ratio;
  float max_share;
  float dropped_fraction;
  float load_peak_over_mean;
  int32_t collapsed;
  int32_t kept_total;
} moe_health;

/* Routing health and the aux-loss-free bias update (dockyard
 * "Mixture-of-Experts" page, "Aux-loss-free load balancing"; the blog page's
 * routing health), one small kernel on the stream.
 *   counts_pre [E], offsets [E+1], dropped [1]: int32, as written by
 *     moe_dispatch / moe_layer_forward for the same spec and T;
 *   prob_sum [E] fp32 or NULL (SOFTMAX_TOPK's sum of probabilities);
 *   health: device moe_health (written);
 *   bias [E] fp32 or NULL: when given, every expert's selection bias moves
 *     by bias_step -- up when its pre-drop load is below the mean load,
 *     down when above, unchanged when equal (the comparison is exact, in
 *     integers); bias_step = 0 leaves it unchanged.
 * Errors: the spec's; MOE_ERR_SHAPE for a missing counts_pre, offsets,
 * dropped or health pointer.  T = 0 is a no-op. */
moe_status moe_routing_health(const moe_spec* spec, int64_t T,
                              const int32_t* counts_pre, const int32_t* offsets,
                              const int32_t* dropped, const float* prob_sum,
                              float* bias, float bias_step,
                              moe_health* health, moe_stream_t stream);

/* Static description of a status code (never NULL). */
const char* moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
