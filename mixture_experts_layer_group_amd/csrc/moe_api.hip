// Host side of the C ABI (include/moe.h): spec validation, capacity,
// workspace layout, and the launch sequence of every entry point.  Nothing
// here synchronises with the device or copies data to the host; ragged sizes
// (per-expert counts, offsets, tile counts) stay on the device and the
// kernels size themselves from them.
#include <algorithm>
#include <climits>
#include <cmath>
#include <mutex>

#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

moe_status validate(const moe_spec* sp, int64_t T) {
  if (sp == nullptr) return MOE_ERR_SHAPE;
  const moe_spec& s = *sp;
  if (T < 0) return MOE_ERR_SHAPE;
  // "Mixture of Experts" blog page, second program: MoEConfig checks
  if (s.num_experts < 2) return MOE_ERR_INVALID_ARG;
  if (s.top_k < 1 || s.top_k > s.num_experts) return MOE_ERR_INVALID_TOPK;
  if (!(s.capacity_factor >= 0.0)) return MOE_ERR_INVALID_ARG;  // negative, NaN
  if (s.capacity_factor > 0.0 && s.capacity_factor < 1.0)
    return MOE_ERR_CAPACITY_TOO_TIGHT;
  if (s.hidden < 1 || s.ffn < 1) return MOE_ERR_INVALID_ARG;
  if (s.router != MOE_ROUTER_SOFTMAX_TOPK && s.router != MOE_ROUTER_SIGMOID_GROUP)
    return MOE_ERR_INVALID_ARG;
  if (s.act != MOE_ACT_SWIGLU && s.act != MOE_ACT_RELU) return MOE_ERR_INVALID_ARG;
  if (s.act_dtype != MOE_DTYPE_F32 && s.act_dtype != MOE_DTYPE_BF16)
    return MOE_ERR_INVALID_ARG;
  if (s.weight_dtype != MOE_DTYPE_F32 && s.weight_dtype != MOE_DTYPE_BF16 &&
      s.weight_dtype != MOE_DTYPE_U4_AFFINE)
    return MOE_ERR_INVALID_ARG;
  if (s.router_dtype != MOE_DTYPE_F32 && s.router_dtype != MOE_DTYPE_BF16)
    return MOE_ERR_INVALID_ARG;
  if (s.out_dtype != MOE_DTYPE_F32 && s.out_dtype != MOE_DTYPE_BF16)
    return MOE_ERR_INVALID_ARG;
  // Edge0 "MoE Spec and Routing" page, WeightLayout: the fused layout
  // stacks gate above up, so it needs the gated activation
  if (s.layout != MOE_LAYOUT_SEPARATE && s.layout != MOE_LAYOUT_FUSED_GATE_UP)
    return MOE_ERR_INVALID_ARG;
  if (s.layout == MOE_LAYOUT_FUSED_GATE_UP && s.act != MOE_ACT_SWIGLU)
    return MOE_ERR_INVALID_ARG;
  // Edge0 "MoE Spec and Routing" page: group-limited routing needs groups
  // of at least two experts (each group scores its top two)
  if (s.router == MOE_ROUTER_SIGMOID_GROUP) {
    if (s.n_group < 1 || s.num_experts % s.n_group != 0) return MOE_ERR_INVALID_ARG;
    const int G = s.num_experts / s.n_group;
    if (G < 2) return MOE_ERR_INVALID_ARG;
    if (s.topk_group < 1 || s.topk_group > s.n_group) return MOE_ERR_INVALID_ARG;
    if (s.top_k > s.topk_group * G) return MOE_ERR_INVALID_ARG;
    if (!std::isfinite(s.routed_scaling)) return MOE_ERR_INVALID_ARG;
  }
  if (s.shared_experts < 0) return MOE_ERR_INVALID_ARG;
  if (s.shared_experts > 0 && s.shared_ffn < 1) return MOE_ERR_INVALID_ARG;
  if (s.weight_dtype == MOE_DTYPE_U4_AFFINE) {
    if (s.quant_group != 64 || s.hidden % 64 != 0 || s.ffn % 64 != 0)
      return MOE_ERR_INVALID_ARG;
  }
  if (s.act_dtype == MOE_DTYPE_BF16 && s.weight_dtype == MOE_DTYPE_F32)
    return MOE_ERR_INVALID_ARG;
  // what this build has kernels for
  if (T > 0 && T * static_cast<int64_t>(s.top_k) > INT32_MAX) return MOE_ERR_SHAPE;
  if (s.act_dtype == MOE_DTYPE_F32 && s.weight_dtype != MOE_DTYPE_F32)
    return MOE_ERR_UNSUPPORTED;
  if (s.hidden % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (s.act_dtype == MOE_DTYPE_BF16 &&
      (s.hidden % 64 != 0 || s.ffn % 64 != 0 ||
       (s.shared_experts > 0 && s.shared_ffn % 64 != 0)))
    return MOE_ERR_UNSUPPORTED;
  if (s.weight_dtype == MOE_DTYPE_U4_AFFINE) {
    // the weight-stream kernels take SwiGLU with d, F powers of two up to
    // 2048; the tiled kernels any d, F that are multiples of 128 (an even
    // number of quantisation groups per row)
    const bool pow2 = s.hidden <= 2048 && s.ffn <= 2048 &&
                      (s.hidden & (s.hidden - 1)) == 0 && (s.ffn & (s.ffn - 1)) == 0;
    const bool stream_ok = s.act == MOE_ACT_SWIGLU && pow2;
    const bool tiled_ok = s.hidden % 128 == 0 && s.ffn % 128 == 0;
    if (!stream_ok && !tiled_ok) return MOE_ERR_UNSUPPORTED;
  }
  if (s.num_experts > 1024 || s.top_k > 64) return MOE_ERR_UNSUPPORTED;
  // the bf16 matrix-core kernels address activations, hidden rows and one
  // expert's matrix with 32-bit byte offsets (4-bit matrices are smaller)
  if (s.act_dtype == MOE_DTYPE_BF16 && s.weight_dtype != MOE_DTYPE_F32) {
    const int64_t lim = INT64_C(1) << 32;
    const int64_t slots = T * s.top_k;
    if (T * s.hidden * 2 >= lim || slots * s.ffn * 2 >= lim ||
        static_cast<int64_t>(s.ffn) * s.hidden * 2 >= lim ||
        T * static_cast<int64_t>(s.shared_ffn) * 2 >= lim ||
        static_cast<int64_t>(s.shared_ffn) * s.hidden * 2 >= lim)
      return MOE_ERR_UNSUPPORTED;
  }
  if (s.router == MOE_ROUTER_SIGMOID_GROUP && s.n_group > 64)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int64_t capacity_of(const moe_spec& s, int64_t T) {
  if (s.capacity_factor == 0.0) return INT64_MAX;
  // left to right, in double: T*k/E*cf, then truncation
  const double exact = static_cast<double>(T * s.top_k) /
                       static_cast<double>(s.num_experts) * s.capacity_factor;
  int64_t c = exact >= 9.0e18 ? INT64_MAX : static_cast<int64_t>(exact);
  return std::max<int64_t>(1, c);
}

Dims dims_of(const moe_spec& s, int64_t T) {
  Dims D{};
  D.T = T;
  D.E = s.num_experts;
  D.k = s.top_k;
  D.d = s.hidden;
  D.F = s.ffn;
  D.S = s.shared_experts;
  D.Fs = s.shared_ffn;
  D.slots = T * s.top_k;
  D.cap = std::min<int64_t>(capacity_of(s, T), std::max<int64_t>(D.slots, 1));
  D.bf16 = s.act_dtype == MOE_DTYPE_BF16;
  D.u4 = s.weight_dtype == MOE_DTYPE_U4_AFFINE;
  D.swiglu = s.act == MOE_ACT_SWIGLU;
  D.fused = s.layout == MOE_LAYOUT_FUSED_GATE_UP;
  D.out_bf16 = s.out_dtype == MOE_DTYPE_BF16;
  D.router_dtype = s.router_dtype;
  return D;
}

WsLayout layout_of(const Dims& D) {
  WsLayout L{};
  const size_t es = D.bf16 ? 2 : 4;
  const size_t T = static_cast<size_t>(D.T), E = D.E, S = D.slots;
  // one wave per token in flight: a token's selection is a chain of dependent
  // wave reductions, so throughput comes from many tokens at once
  L.route_blocks = static_cast<int>(std::min<int64_t>((D.T + kSelectWaves - 1) / kSelectWaves, 8192));
  if (L.route_blocks < 1) L.route_blocks = 1;
  L.dispatch_blocks = static_cast<int>((D.slots + kDispatchChunk - 1) / kDispatchChunk);
  if (L.dispatch_blocks < 1) L.dispatch_blocks = 1;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const RouterPlan rp = router_plan(D);
  L.logits = take(static_cast<size_t>(rp.S) * T * E * 4);
  L.probpart = take(static_cast<size_t>(L.route_blocks) * E * 4);
  L.hist = take(static_cast<size_t>(L.dispatch_blocks) * E * 4);
  L.tiles1 = take(tile_plan_entries(E) * 4);
  L.tiles2 = take(tile_plan_entries(E) * 4);
  L.topk_ids = take(S * 4);
  L.topk_w = take(S * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted_token = take(S * 4);
  L.sorted_w = take(S * 4);
  L.slot_row = take(S * 4);
  L.dropped = take(4);
  L.H = take(S * D.F * es);
  L.Hs = take(static_cast<size_t>(D.S) * T * D.Fs * es);
  L.Y = take(S * D.d * 4);
  L.Ypart = take(down_splits(D) > 1 ? S * D.d * 4 : 0);
  L.Ys = take(static_cast<size_t>(D.S) * T * D.d * 4);
  L.X16 = take(D.u4 && u4_tiled(D) ? T * D.d * 2 : 0);
  L.total = o;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<uint8_t*>(ws) + off);
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_weights(const moe_spec& sp, const moe_expert_weights* w) {
  if (w == nullptr || !w->gate || !w->down) return MOE_ERR_SHAPE;
  const bool fused = sp.layout == MOE_LAYOUT_FUSED_GATE_UP;
  if (fused) {
    // the up rows live inside the fused gate tensor
    if (w->up || w->up_scale || w->up_bias || w->shared_up) return MOE_ERR_INVALID_ARG;
    if (sp.weight_dtype == MOE_DTYPE_U4_AFFINE &&
        (!w->gate_scale || !w->gate_bias || !w->down_scale || !w->down_bias))
      return MOE_ERR_SHAPE;
    if (sp.shared_experts > 0 &&
        (!w->shared_gate || !w->shared_down || !aligned16(w->shared_gate) ||
         !aligned16(w->shared_down)))
      return MOE_ERR_SHAPE;
    return aligned16(w->gate) && aligned16(w->down) ? MOE_OK : MOE_ERR_SHAPE;
  }
  if (sp.act == MOE_ACT_SWIGLU && !w->up) return MOE_ERR_SHAPE;
  if (!aligned16(w->gate) || !aligned16(w->down) || (w->up && !aligned16(w->up)))
    return MOE_ERR_SHAPE;
  if (sp.weight_dtype == MOE_DTYPE_U4_AFFINE &&
      (!w->gate_scale || !w->gate_bias || !w->up_scale || !w->up_bias ||
       !w->down_scale || !w->down_bias))
    return MOE_ERR_SHAPE;
  if (sp.shared_experts > 0) {
    if (!w->shared_gate || !w->shared_down) return MOE_ERR_SHAPE;
    if (sp.act == MOE_ACT_SWIGLU && !w->shared_up) return MOE_ERR_SHAPE;
    if (!aligned16(w->shared_gate) || !aligned16(w->shared_down) ||
        (w->shared_up && !aligned16(w->shared_up)))
      return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

// ------------------------------------------------------------ stage bodies
moe_status do_route(const moe_spec& sp, const Dims& D, const WsLayout& L,
                    const void* x, const void* wr, const float* bias,
                    const int32_t* forced, int32_t* rejected,
                    int32_t* ids, float* w, float* logits, float* prob_sum,
                    int32_t* err, void* ws, hipStream_t s) {
  const RouterPlan rp = router_plan(D);
  // split reductions write partial planes to the workspace; the selection
  // adds them and hands the sums to the caller's buffer if one was given
  float* Lg = (rp.S > 1 || logits == nullptr) ? at<float>(ws, L.logits) : logits;
  float* Lout = rp.S > 1 ? logits : nullptr;
  hipError_t e = launch_router_logits(D, rp, sp.act_dtype, sp.router_dtype, x, wr, Lg, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  const bool want_p = prob_sum != nullptr && sp.router == MOE_ROUTER_SOFTMAX_TOPK;
  float* part = want_p ? at<float>(ws, L.probpart) : nullptr;
  if (forced != nullptr) {
    e = launch_zero_i32(rejected, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  e = launch_router_select(D, sp, Lg, rp.S, Lout, bias, forced,
                           rejected, ids, w, part, err, L.route_blocks, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (want_p) return hip_status(launch_prob_finalize(D, part, L.route_blocks, prob_sum, s));
  return MOE_OK;
}

// ev (may be null): three events recorded before the first expert kernel,
// between the routed gate/up and down kernels, and after the last one.
// fused: the layer's dispatch wrote the M-tile prefixes; layer: called by
// the layer, whose combine reads the matrix-core kernels' expert rows in
// fp16 and adds the down projection's second K split itself (the stage API
// returns whole fp32 rows)
moe_status do_ffn(const moe_spec& sp, const Dims& D, const WsLayout& L,
                  const int32_t* offsets, const int32_t* sorted_token,
                  const void* x, const moe_expert_weights& w, const float* row_scale,
                  void* y_rows,
                  void* y_shared, int32_t* err, void* const* ev, void* ws,
                  bool fused, bool layer, hipStream_t s) {
  void* H = at<void>(ws, L.H);
  void* Hs = at<void>(ws, L.Hs);
  hipEvent_t mid = ev ? static_cast<hipEvent_t>(ev[1]) : nullptr;
  hipError_t e = hipSuccess;
  if (!D.bf16 || D.u4) {
    // (the 4-bit tiled kernels, like the bf16 ones, read the M-tile
    // prefixes, which the fused layer's dispatch wrote)
    if (ev && (e = hipEventRecord(static_cast<hipEvent_t>(ev[0]), s)) != hipSuccess)
      return MOE_ERR_HIP;
    if (!D.bf16) {
      e = launch_ffn_f32(D, offsets, sorted_token, x, w, row_scale, H, Hs, y_rows, y_shared,
                         mid, s);
    } else if (!u4_tiled(D)) {
      e = launch_ffn_u4(D, sp.quant_group, offsets, sorted_token, x, w, row_scale, H, y_rows, err,
                        mid, s);
    } else {
      int32_t* t1 = at<int32_t>(ws, L.tiles1);
      int32_t* t2 = at<int32_t>(ws, L.tiles2);
      if (!fused) e = launch_tile_prefix(D, offsets, t1, t2, s);
      if (e == hipSuccess)
        e = launch_ffn_u4_tiled(D, offsets, t1, t2, sorted_token, x, at<void>(ws, L.X16), w,
                                row_scale, layer, H,
                                y_rows, err, mid, s);
    }
    if (e == hipSuccess && D.bf16 && D.S > 0)
      e = launch_shared_bf16(D, x, w, Hs, y_shared, err, s);
    if (e == hipSuccess && ev) e = hipEventRecord(static_cast<hipEvent_t>(ev[2]), s);
    return hip_status(e);
  }
  int32_t* t1 = at<int32_t>(ws, L.tiles1);
  int32_t* t2 = at<int32_t>(ws, L.tiles2);
  if (!fused) {  // the fused layer's dispatch already wrote the tile prefixes
    e = launch_tile_prefix(D, offsets, t1, t2, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (ev && (e = hipEventRecord(static_cast<hipEvent_t>(ev[0]), s)) != hipSuccess)
    return MOE_ERR_HIP;
  float* part = down_splits(D) > 1 ? at<float>(ws, L.Ypart) : nullptr;
  // inside the layer the expert rows go to the combine in fp16
  e = launch_ffn_bf16(D, offsets, t1, t2, sorted_token, x, w, row_scale, layer, H, Hs, y_rows,
                      part,
                      y_shared, err, mid, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (ev && (e = hipEventRecord(static_cast<hipEvent_t>(ev[2]), s)) != hipSuccess)
    return MOE_ERR_HIP;
  // the stage API returns whole expert rows; the layer lets the combine add
  // the second split instead
  if (part && !layer)
    return hip_status(launch_fold_split(D, offsets, static_cast<float*>(y_rows), part, s));
  return MOE_OK;
}

// The whole layer on a caller-owned workspace (or, for the no-allocation
// entry point, the library's static scratch array): `workspace` may be null
// only when ws_bytes is 0, which fails the size check below.
moe_status layer_forward(const moe_spec* spec, int64_t T, const void* x,
                         const void* w_router, const float* expert_bias,
                         const moe_expert_weights* weights, void* out,
                         const moe_layer_stats* stats, void* workspace,
                         size_t ws_bytes, moe_stream_t stream) {
  moe_status st = validate(spec, T);
  if (st != MOE_OK) return st;
  if (expert_bias != nullptr && spec->router == MOE_ROUTER_SOFTMAX_TOPK)
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !out || !aligned16(x) || !aligned16(w_router) || !aligned16(out))
    return MOE_ERR_SHAPE;
  st = check_weights(*spec, weights);
  if (st != MOE_OK) return st;
  const Dims D = dims_of(*spec, T);
  const WsLayout L = layout_of(D);
  if (!workspace || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = workspace;
  moe_layer_stats z{};
  const moe_layer_stats& o = stats ? *stats : z;
  int32_t* ids = o.topk_ids ? o.topk_ids : at<int32_t>(ws, L.topk_ids);
  float* tw = o.topk_w ? o.topk_w : at<float>(ws, L.topk_w);
  int32_t* counts = o.counts_pre ? o.counts_pre : at<int32_t>(ws, L.counts);
  int32_t* offsets = o.offsets ? o.offsets : at<int32_t>(ws, L.offsets);
  int32_t* dropped = o.dropped ? o.dropped : at<int32_t>(ws, L.dropped);
  int32_t* slot_row = o.slot_row ? o.slot_row : at<int32_t>(ws, L.slot_row);
  int32_t* sorted_token = o.sorted_token ? o.sorted_token : at<int32_t>(ws, L.sorted_token);
  float* sorted_w = at<float>(ws, L.sorted_w);

  st = do_route(*spec, D, L, x, w_router, expert_bias, nullptr, nullptr, ids,
                tw, o.logits, o.prob_sum, o.errors, ws, s);
  if (st != MOE_OK) return st;
  const bool mfma_path = D.bf16 && (!D.u4 || u4_tiled(D));
  hipError_t e = launch_dispatch(
      D, ids, tw, at<int32_t>(ws, L.hist), L.dispatch_blocks, counts, offsets,
      sorted_token, sorted_w, slot_row, dropped,
      mfma_path ? at<int32_t>(ws, L.tiles1) : nullptr,
      mfma_path ? at<int32_t>(ws, L.tiles2) : nullptr, o.errors, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  void* Y = at<void>(ws, L.Y);
  void* Ys = at<void>(ws, L.Ys);
  st = do_ffn(*spec, D, L, offsets, sorted_token, x, *weights, nullptr, Y, Ys, o.errors,
              o.ffn_events, ws, mfma_path, true, s);
  if (st != MOE_OK) return st;
  const void* part = (mfma_path && down_splits(D) > 1) ? at<void>(ws, L.Ypart) : nullptr;
  // the matrix-core kernels hand the layer's combine fp16 expert rows
  return hip_status(launch_combine(D, Y, part, mfma_path, slot_row, tw,
                                   D.S > 0 ? Ys : nullptr, out, s));
}

// Scratch of the no-allocation entry point: a file-scope device array, so
// each GPU the library runs on holds its own copy from the moment the code
// object is loaded there until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device memory: the device address is
// taken once per device with hipGetSymbolAddress and only that address is
// passed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// device address of the current device's scratch array (looked up on the
// first call on that device, with it current)
moe_status static_scratch(void** p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[dev] = ptr;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch[dev] == nullptr) return MOE_ERR_HIP;
  *p = g_scratch[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_spec_validate(const moe_spec* spec, int64_t T) {
  return validate(spec, T);
}

moe_status moe_capacity(const moe_spec* spec, int64_t T, int64_t* cap_out) {
  const moe_status st = validate(spec, T);
  if (st != MOE_OK) return st;
  if (cap_out == nullptr) return MOE_ERR_SHAPE;
  *cap_out = capacity_of(*spec, T);
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_spec* spec, int64_t T, size_t* bytes) {
  const moe_status st = validate(spec, T);
  if (st != MOE_OK) return st;
  if (bytes == nullptr) return MOE_ERR_SHAPE;
  *bytes = layout_of(dims_of(*spec, T)).total;
  return MOE_OK;
}

moe_status moe_route(const moe_spec* spec, int64_t T, const void* x,
                     const void* w_router, const float* expert_bias,
                     int32_t* topk_ids, float* topk_w, float* logits,
                     float* prob_sum, int32_t* errors, void* workspace,
                     size_t ws_bytes, moe_stream_t stream) {
  moe_status st = validate(spec, T);
  if (st != MOE_OK) return st;
  if (expert_bias != nullptr && spec->router == MOE_ROUTER_SOFTMAX_TOPK)
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_ids || !topk_w || !aligned16(x) || !aligned16(w_router))
    return MOE_ERR_SHAPE;
  const Dims D = dims_of(*spec, T);
  const WsLayout L = layout_of(D);
  if (!workspace || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return do_route(*spec, D, L, x, w_router, expert_bias, nullptr, nullptr,
                  topk_ids, topk_w, logits, prob_sum, errors, workspace,
                  static_cast<hipStream_t>(stream));
}

moe_status moe_route_forced(const moe_spec* spec, int64_t T, const void* x,
                            const void* w_router, const int32_t* forced_ids,
                            int32_t* topk_ids, float* topk_w, float* logits,
                            float* prob_sum, int32_t* rejected,
                            void* workspace, size_t ws_bytes,
                            moe_stream_t stream) {
  moe_status st = validate(spec, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !forced_ids || !topk_ids || !topk_w || !rejected ||
      !aligned16(x) || !aligned16(w_router))
    return MOE_ERR_SHAPE;
  const Dims D = dims_of(*spec, T);
  const WsLayout L = layout_of(D);
  if (!workspace || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return do_route(*spec, D, L, x, w_router, nullptr, forced_ids, rejected,
                  topk_ids, topk_w, logits, prob_sum, nullptr, workspace,
                  static_cast<hipStream_t>(stream));
}

moe_status moe_dispatch(const moe_spec* spec, int64_t T,
                        const int32_t* topk_ids, const float* topk_w,
                        int32_t* counts_pre, int32_t* offsets,
                        int32_t* sorted_token, float* sorted_w,
                        int32_t* slot_row, int32_t* dropped, const void* x,
                        void* x_perm, int32_t* errors, void* workspace,
                        size_t ws_bytes, moe_stream_t stream) {
  moe_status st = validate(spec, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !topk_w || !counts_pre || !offsets || !sorted_token ||
      !sorted_w || !slot_row || !dropped)
    return MOE_ERR_SHAPE;
  if ((x != nullptr) != (x_perm != nullptr)) return MOE_ERR_SHAPE;
  if (x && (!aligned16(x) || !aligned16(x_perm))) return MOE_ERR_SHAPE;
  const Dims D = dims_of(*spec, T);
  const WsLayout L = layout_of(D);
  if (!workspace || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_dispatch(D, topk_ids, topk_w, at<int32_t>(workspace, L.hist),
                                 L.dispatch_blocks, counts_pre, offsets,
                                 sorted_token, sorted_w, slot_row, dropped,
                                 nullptr, nullptr, errors, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (x) return hip_status(launch_gather_rows(D, offsets, sorted_token, x, x_perm, s));
  return MOE_OK;
}

moe_status moe_grouped_ffn(const moe_spec* spec, int64_t T,
                           const int32_t* offsets, const int32_t* sorted_token,
                           const void* x, const moe_expert_weights* weights,
                           const float* sorted_w, void* y_rows, void* y_shared, int32_t* errors,
                           void* workspace, size_t ws_bytes,
                           moe_stream_t stream) {
  moe_status st = validate(spec, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!offsets || !sorted_token || !x || !y_rows || !aligned16(x) || !aligned16(y_rows))
    return MOE_ERR_SHAPE;
  if (spec->shared_experts > 0 && (!y_shared || !aligned16(y_shared)))
    return MOE_ERR_SHAPE;
  st = check_weights(*spec, weights);
  if (st != MOE_OK) return st;
  const Dims D = dims_of(*spec, T);
  const WsLayout L = layout_of(D);
  if (!workspace || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return do_ffn(*spec, D, L, offsets, sorted_token, x, *weights, sorted_w, y_rows,
                y_shared, errors, nullptr, workspace, false, false,
                static_cast<hipStream_t>(stream));
}

moe_status moe_combine(const moe_spec* spec, int64_t T, const void* y_rows,
                       const int32_t* slot_row, const float* topk_w,
                       const void* y_shared, void* out, moe_stream_t stream) {
  moe_status st = validate(spec, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!y_rows || !slot_row || !out || !aligned16(y_rows) || !aligned16(out))
    return MOE_ERR_SHAPE;
  if (spec->shared_experts > 0 && (!y_shared || !aligned16(y_shared)))
    return MOE_ERR_SHAPE;
  const Dims D = dims_of(*spec, T);
  return hip_status(launch_combine(D, y_rows, nullptr, false, slot_row, topk_w,
                                   spec->shared_experts > 0 ? y_shared : nullptr,
                                   out, static_cast<hipStream_t>(stream)));
}

moe_status moe_layer_forward(const moe_spec* spec, int64_t T, const void* x,
                             const void* w_router, const float* expert_bias,
                             const moe_expert_weights* weights, void* out,
                             const moe_layer_stats* stats, void* workspace,
                             size_t ws_bytes, moe_stream_t stream) {
  return layer_forward(spec, T, x, w_router, expert_bias, weights, out, stats, workspace,
                       ws_bytes, stream);
}

moe_status moe_layer_forward_static(const moe_spec* spec, int64_t T, const void* x,
                                    const void* w_router, const float* expert_bias,
                                    const moe_expert_weights* weights, void* out,
                                    const moe_layer_stats* stats, moe_stream_t stream) {
  const moe_status st = validate(spec, T);
  if (st != MOE_OK) return st;
  if (T == 0) return layer_forward(spec, T, x, w_router, expert_bias, weights, out, stats,
                                   nullptr, 0, stream);
  void* ws = nullptr;
  const moe_status sc = static_scratch(&ws);
  if (sc != MOE_OK) return sc;
  // a layer whose workspace exceeds the array fails the size check
  // (MOE_ERR_WORKSPACE) before anything is launched
  return layer_forward(spec, T, x, w_router, expert_bias, weights, out, stats, ws,
                       MOE_STATIC_SCRATCH_BYTES, stream);
}

moe_status moe_routing_health(const moe_spec* spec, int64_t T,
                              const int32_t* counts_pre, const int32_t* offsets,
                              const int32_t* dropped, const float* prob_sum,
                              float* bias, float bias_step,
                              moe_health* health, moe_stream_t stream) {
  moe_status st = validate(spec, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!counts_pre || !offsets || !dropped || !health) return MOE_ERR_SHAPE;
  const Dims D = dims_of(*spec, T);
  return hip_status(launch_routing_health(D, counts_pre, offsets, dropped, prob_sum,
                                          bias, bias_step, health,
                                          static_cast<hipStream_t>(stream)));
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_INVALID_TOPK: return "top_k outside [1, num_experts]";
    case MOE_ERR_CAPACITY_TOO_TIGHT:
      return "capacity_factor below 1 drops tokens even under uniform routing";
    case MOE_ERR_SHAPE: return "missing or misaligned pointer, or bad token count";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_UNSUPPORTED: return "valid spec without a kernel in this build";
  }
  return "unknown status";
}

}  // extern "C"
