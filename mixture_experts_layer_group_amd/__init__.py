"""Python binding of the MI355X MoE layer library (``libmoe_mi355x.so``).

Argument marshalling only: every step of route -> dispatch -> grouped expert
FFN -> combine runs in the HIP kernels behind the C ABI of
``include/moe.h``; this module turns torch tensors into device pointers and
the current torch stream into a ``hipStream_t``.  There is no fallback: if
the library has not been built, importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK = 0
ROUTER = {"softmax_topk": 0, "sigmoid_group": 1}
ACT = {"swiglu": 0, "relu": 1}
DTYPE = {"f32": 0, "bf16": 1, "u4": 2}
LAYOUT = {"separate": 0, "fused_gate_up": 1}
# MOE_FLAG_* bits of the device error word
FLAG_BAD_EXPERT_ID = 1
FLAG_H_SATURATED = 2
FLAG_NONFINITE_LOGIT = 4
FLAG_X_SATURATED = 8
FLAG_Y_SATURATED = 16
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_INVALID_TOPK",
                3: "MOE_ERR_CAPACITY_TOO_TIGHT", 4: "MOE_ERR_SHAPE",
                5: "MOE_ERR_WORKSPACE", 6: "MOE_ERR_HIP", 7: "MOE_ERR_UNSUPPORTED"}
EXPORTS = ("moe_spec_validate", "moe_capacity", "moe_workspace_size", "moe_route",
           "moe_route_forced", "moe_dispatch", "moe_grouped_ffn", "moe_combine", "moe_layer_forward",
           "moe_layer_forward_static", "moe_routing_health", "moe_status_string")
# MOE_STATIC_SCRATCH_BYTES: the static scratch of moe_layer_forward_static
STATIC_SCRATCH_BYTES = 64 << 20


class MoESpec(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("router", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("capacity_factor", ctypes.c_double),
                ("shared_experts", ctypes.c_int32), ("shared_ffn", ctypes.c_int32),
                ("act", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("router_dtype", ctypes.c_int32),
                ("quant_group", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


_W_FIELDS = ["gate", "up", "down", "gate_scale", "gate_bias", "up_scale", "up_bias",
             "down_scale", "down_bias", "shared_gate", "shared_up", "shared_down"]


class MoEExpertWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _W_FIELDS]


_S_FIELDS = ["topk_ids", "topk_w", "logits", "counts_pre", "offsets", "dropped",
             "prob_sum", "slot_row", "sorted_token", "errors"]


class MoEHealth(ctypes.Structure):
    """Device struct filled by moe_routing_health (allocate it as a 40-byte
    tensor and read it back with ``health_from_bytes``)."""
    _fields_ = [("aux", ctypes.c_float), ("aux3", ctypes.c_float),
                ("entropy", ctypes.c_float), ("max_entropy", ctypes.c_float),
                ("entropy_ratio", ctypes.c_float), ("max_share", ctypes.c_float),
                ("dropped_fraction", ctypes.c_float),
                ("load_peak_over_mean", ctypes.c_float),
                ("collapsed", ctypes.c_int32), ("kept_total", ctypes.c_int32)]


class MoELayerStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _S_FIELDS] + [("ffn_events", ctypes.c_void_p)]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({status_string(status)})")


_lib = None


def library() -> ctypes.CDLL:
    """The loaded HIP library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mixture_experts_layer_group_amd.build` (there is no "
                "fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        sp = ctypes.POINTER(MoESpec)
        lib.moe_spec_validate.argtypes = [sp, i64]
        lib.moe_capacity.argtypes = [sp, i64, ctypes.POINTER(ctypes.c_int64)]
        lib.moe_workspace_size.argtypes = [sp, i64, ctypes.POINTER(ctypes.c_size_t)]
        lib.moe_route.argtypes = [sp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.moe_route_forced.argtypes = [sp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         sz, vp]
        lib.moe_dispatch.argtypes = [sp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     vp, vp, sz, vp]
        lib.moe_grouped_ffn.argtypes = [sp, i64, vp, vp, vp,
                                        ctypes.POINTER(MoEExpertWeights), vp, vp, vp, vp,
                                        vp, sz, vp]
        lib.moe_combine.argtypes = [sp, i64, vp, vp, vp, vp, vp, vp]
        lib.moe_layer_forward.argtypes = [sp, i64, vp, vp, vp,
                                          ctypes.POINTER(MoEExpertWeights), vp,
                                          ctypes.POINTER(MoELayerStats), vp, sz, vp]
        lib.moe_layer_forward_static.argtypes = [sp, i64, vp, vp, vp,
                                                 ctypes.POINTER(MoEExpertWeights), vp,
                                                 ctypes.POINTER(MoELayerStats), vp]
        lib.moe_routing_health.argtypes = [sp, i64, vp, vp, vp, vp, vp, ctypes.c_float,
                                           vp, vp]
        for n in EXPORTS[:-1]:
            getattr(lib, n).restype = ctypes.c_int
        lib.moe_status_string.argtypes = [ctypes.c_int]
        lib.moe_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().moe_status_string(int(status)).decode()


# ---------------------------------------------------------------- specs
def make_spec(E: int, top_k: int, d: int, F: int, router: str = "softmax_topk",
              norm_topk_prob: bool = True, routed_scaling: float = 1.0,
              n_group: int = 0, topk_group: int = 0, capacity_factor: float = 0.0,
              shared_experts: int = 0, shared_F: int = 0, act: str = "swiglu",
              act_dtype: str = "bf16", weight_dtype: str = "bf16",
              router_dtype: str = "f32", quant_group: int = 64,
              out_dtype: str = "f32", layout: str = "separate") -> MoESpec:
    return MoESpec(E, top_k, d, F, ROUTER[router], int(bool(norm_topk_prob)),
                   float(routed_scaling), n_group, topk_group, float(capacity_factor),
                   shared_experts, shared_F, ACT[act], DTYPE[act_dtype],
                   DTYPE[weight_dtype], DTYPE[router_dtype], quant_group,
                   DTYPE[out_dtype], LAYOUT[layout])


def spec_from_config(cfg) -> MoESpec:
    """A ``moe_spec`` from an object with the workload fields (E, top_k, d,
    F, router, ... as in ``synth.LayerConfig``)."""
    return make_spec(cfg.E, cfg.top_k, cfg.d, cfg.F, cfg.router, cfg.norm_topk_prob,
                     cfg.routed_scaling, cfg.n_group, cfg.topk_group,
                     cfg.capacity_factor, cfg.shared_experts, cfg.shared_F, cfg.act,
                     cfg.act_dtype, cfg.weight_dtype, cfg.router_dtype,
                     cfg.quant_group, getattr(cfg, "out_dtype", "f32"),
                     getattr(cfg, "layout", "separate"))


# ---------------------------------------------------------------- helpers
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoEError(status, where)


def expert_weights(w: Dict) -> MoEExpertWeights:
    """``moe_expert_weights`` from a dict of tensors keyed like the C struct
    (gate/up/down, *_scale/*_bias for 4-bit, shared_*).  Also accepts the
    keys w_gate/w_up/w_down, q_*/s_*/b_* and sh_*, and for the fused
    gate/up layout w_gate_up, q_gate_up/s_gate_up/b_gate_up and sh_gate_up
    (passed in the gate fields)."""
    alias = {"w_gate_up": "gate", "q_gate_up": "gate", "s_gate_up": "gate_scale",
             "b_gate_up": "gate_bias", "sh_gate_up": "shared_gate",
             "w_gate": "gate", "w_up": "up", "w_down": "down", "q_gate": "gate",
             "q_up": "up", "q_down": "down", "s_gate": "gate_scale",
             "b_gate": "gate_bias", "s_up": "up_scale", "b_up": "up_bias",
             "s_down": "down_scale", "b_down": "down_bias", "sh_gate": "shared_gate",
             "sh_up": "shared_up", "sh_down": "shared_down"}
    out = MoEExpertWeights()
    for k, v in w.items():
        if v is None:
            continue
        name = alias.get(k, k)
        if name in _W_FIELDS:
            setattr(out, name, _ptr(v))
    return out


def layer_stats(ffn_events=None, **tensors) -> MoELayerStats:
    """``moe_layer_stats`` from device tensors keyed like the C struct;
    ``ffn_events``: three hipEvent_t handles (ints) or None."""
    s = MoELayerStats()
    for k, v in tensors.items():
        if k not in _S_FIELDS:
            raise KeyError(k)
        setattr(s, k, _ptr(v))
    if ffn_events is not None:
        arr = (ctypes.c_void_p * 3)(*[int(e) for e in ffn_events])
        s._events_keepalive = arr
        s.ffn_events = ctypes.cast(arr, ctypes.c_void_p)
    return s


# ---------------------------------------------------------------- C ABI
def moe_spec_validate(spec: MoESpec, T: int) -> int:
    return library().moe_spec_validate(ctypes.byref(spec), T)


def moe_capacity(spec: MoESpec, T: int) -> int:
    c = ctypes.c_int64()
    _check(library().moe_capacity(ctypes.byref(spec), T, ctypes.byref(c)), "moe_capacity")
    return c.value


def moe_workspace_size(spec: MoESpec, T: int) -> int:
    n = ctypes.c_size_t()
    _check(library().moe_workspace_size(ctypes.byref(spec), T, ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


def moe_route(spec, T, x, w_router, expert_bias, topk_ids, topk_w, logits=None,
              prob_sum=None, workspace=None, ws_bytes=None, stream=None,
              errors=None) -> None:
    ws_bytes = ws_bytes if ws_bytes is not None else (workspace.numel() if workspace is not None else 0)
    _check(library().moe_route(ctypes.byref(spec), T, _ptr(x), _ptr(w_router),
                               _ptr(expert_bias), _ptr(topk_ids), _ptr(topk_w),
                               _ptr(logits), _ptr(prob_sum), _ptr(errors),
                               _ptr(workspace), ws_bytes, _stream(stream)), "moe_route")


def moe_route_forced(spec, T, x, w_router, forced_ids, topk_ids, topk_w, rejected,
                     logits=None, prob_sum=None, workspace=None, ws_bytes=None,
                     stream=None) -> None:
    ws_bytes = ws_bytes if ws_bytes is not None else (workspace.numel() if workspace is not None else 0)
    _check(library().moe_route_forced(ctypes.byref(spec), T, _ptr(x), _ptr(w_router),
                                      _ptr(forced_ids), _ptr(topk_ids), _ptr(topk_w),
                                      _ptr(logits), _ptr(prob_sum), _ptr(rejected),
                                      _ptr(workspace), ws_bytes, _stream(stream)),
           "moe_route_forced")


def moe_dispatch(spec, T, topk_ids, topk_w, counts_pre, offsets, sorted_token,
                 sorted_w, slot_row, dropped, x=None, x_perm=None, workspace=None,
                 ws_bytes=None, stream=None, errors=None) -> None:
    ws_bytes = ws_bytes if ws_bytes is not None else (workspace.numel() if workspace is not None else 0)
    _check(library().moe_dispatch(ctypes.byref(spec), T, _ptr(topk_ids), _ptr(topk_w),
                                  _ptr(counts_pre), _ptr(offsets), _ptr(sorted_token),
                                  _ptr(sorted_w), _ptr(slot_row), _ptr(dropped),
                                  _ptr(x), _ptr(x_perm), _ptr(errors), _ptr(workspace),
                                  ws_bytes, _stream(stream)), "moe_dispatch")


def moe_grouped_ffn(spec, T, offsets, sorted_token, x, weights, y_rows,
                    y_shared=None, workspace=None, ws_bytes=None, stream=None,
                    errors=None, sorted_w=None) -> None:
    """sorted_w (moe_dispatch's [T*k] fp32, or None): when given, each routed
    row comes out multiplied by its routing weight (then combine with
    topk_w=None)."""
    w = weights if isinstance(weights, MoEExpertWeights) else expert_weights(weights)
    ws_bytes = ws_bytes if ws_bytes is not None else (workspace.numel() if workspace is not None else 0)
    _check(library().moe_grouped_ffn(ctypes.byref(spec), T, _ptr(offsets),
                                     _ptr(sorted_token), _ptr(x), ctypes.byref(w),
                                     _ptr(sorted_w), _ptr(y_rows), _ptr(y_shared), _ptr(errors),
                                     _ptr(workspace), ws_bytes, _stream(stream)),
           "moe_grouped_ffn")


def moe_combine(spec, T, y_rows, slot_row, topk_w, y_shared, out, stream=None) -> None:
    _check(library().moe_combine(ctypes.byref(spec), T, _ptr(y_rows), _ptr(slot_row),
                                 _ptr(topk_w), _ptr(y_shared), _ptr(out),
                                 _stream(stream)), "moe_combine")


def moe_layer_forward(spec, T, x, w_router, expert_bias, weights, out, stats=None,
                      workspace=None, ws_bytes=None, stream=None) -> None:
    w = weights if isinstance(weights, MoEExpertWeights) else expert_weights(weights)
    st = stats if (stats is None or isinstance(stats, MoELayerStats)) else layer_stats(**stats)
    ws_bytes = ws_bytes if ws_bytes is not None else (workspace.numel() if workspace is not None else 0)
    _check(library().moe_layer_forward(ctypes.byref(spec), T, _ptr(x), _ptr(w_router),
                                       _ptr(expert_bias), ctypes.byref(w), _ptr(out),
                                       ctypes.byref(st) if st is not None else None,
                                       _ptr(workspace), ws_bytes, _stream(stream)),
           "moe_layer_forward")


def moe_layer_forward_static(spec, T, x, w_router, expert_bias, weights, out, stats=None,
                             stream=None) -> None:
    """moe_layer_forward on the library's static scratch (no allocation)."""
    w = weights if isinstance(weights, MoEExpertWeights) else expert_weights(weights)
    st = stats if (stats is None or isinstance(stats, MoELayerStats)) else layer_stats(**stats)
    _check(library().moe_layer_forward_static(ctypes.byref(spec), T, _ptr(x), _ptr(w_router),
                                              _ptr(expert_bias), ctypes.byref(w), _ptr(out),
                                              ctypes.byref(st) if st is not None else None,
                                              _stream(stream)),
           "moe_layer_forward_static")


def moe_routing_health(spec, T, counts_pre, offsets, dropped, prob_sum, health,
                       bias=None, bias_step: float = 0.0, stream=None) -> None:
    _check(library().moe_routing_health(ctypes.byref(spec), T, _ptr(counts_pre),
                                        _ptr(offsets), _ptr(dropped), _ptr(prob_sum),
                                        _ptr(bias), ctypes.c_float(bias_step),
                                        _ptr(health), _stream(stream)),
           "moe_routing_health")


def health_buffer(device="cuda"):
    """Device bytes for one moe_health struct."""
    import torch
    return torch.zeros(ctypes.sizeof(MoEHealth), dtype=torch.uint8, device=device)


def health_from_bytes(buf) -> dict:
    """The moe_health fields of a device buffer, as a dict (copies to host)."""
    raw = bytes(buf.detach().to("cpu").numpy().tobytes())
    h = MoEHealth.from_buffer_copy(raw[:ctypes.sizeof(MoEHealth)])
    return {name: getattr(h, name) for name, _ in MoEHealth._fields_}


def workspace(spec: MoESpec, T: int, device="cuda"):
    """A device byte buffer of ``moe_workspace_size`` bytes (torch is used
    only to allocate it)."""
    import torch
    return torch.empty(max(1, moe_workspace_size(spec, T)), dtype=torch.uint8,
                       device=device)
