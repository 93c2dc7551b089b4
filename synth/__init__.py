"""Seeded synthetic inputs for the sparse MoE layer forward.

This module only draws numbers: it holds none of the layer's arithmetic
(no routing, dispatch, expert FFN or combine).  Both sides of every parity
check -- the CPU oracle and the HIP path -- receive tensors made here, and
the oracle always gets a host copy of exactly the tensor the device used.

Recipe (one rule for every tensor):
  * a 64-bit seed comes from ``numpy.random.SeedSequence([base, cfg_id,
    tensor_id, expert_id])`` so any tensor or any single expert can be
    regenerated on its own;
  * Gaussians are drawn in fp32 by ``torch.randn`` with a ``torch.Generator``
    on the target device, scaled by ``1/sqrt(fan_in)`` (hidden states use
    std 1), and rounded to bf16 with round-to-nearest-even when the tensor
    is bf16.  The CPU and the GPU generators are different streams, so the
    values depend on the device they are drawn on; tests never mix them.

Workload shapes follow the Mixtral expert shape (hidden 4096, FFN 14336,
8 experts, top-2) of the "moe-architecture" skill page, the DeepSeek-V3
sigmoid-group routing of the Edge0 "MoE Spec and Routing" page, and the
tiny ReLU layer of the "Mixture of Experts" blog page.  The 4-bit weights use
that Edge0 page's format (4 bits, group 64, affine); the quantiser below only
prepares inputs in that format -- the pages define the format, not how a
checkpoint was quantised.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch

# router kinds / activations / dtypes (plain strings; the binding maps them)
SOFTMAX_TOPK = "softmax_topk"
SIGMOID_GROUP = "sigmoid_group"
SWIGLU = "swiglu"
RELU = "relu"
F32 = "f32"
BF16 = "bf16"
U4 = "u4"
SEPARATE = "separate"
FUSED_GATE_UP = "fused_gate_up"

# tensor ids used in the seed sequence
TID_X, TID_WR, TID_BIAS, TID_GATE, TID_UP, TID_DOWN = 0, 1, 2, 3, 4, 5
TID_SH_GATE, TID_SH_UP, TID_SH_DOWN = 6, 7, 8
SEED_BASE = 1234


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape and routing of one MoE layer workload."""

    name: str
    cfg_id: int
    T: int
    d: int
    E: int
    top_k: int
    F: int
    router: str = SOFTMAX_TOPK
    norm_topk_prob: bool = True
    routed_scaling: float = 1.0
    n_group: int = 0
    topk_group: int = 0
    capacity_factor: float = 0.0  # 0 = unlimited
    shared_experts: int = 0
    shared_F: int = 0
    act: str = SWIGLU
    act_dtype: str = BF16
    weight_dtype: str = BF16
    router_dtype: str = F32
    quant_group: int = 64
    out_dtype: str = F32  # layer output (fp32 accumulation result by default)
    layout: str = "separate"  # or FUSED_GATE_UP: gate rows above up rows
    # generation recipe only
    bias_range: float = 0.0  # U(-r, r) selection bias (sigmoid-group)
    zipf_s: float = 0.0  # > 0: fold a Zipf popularity prior into router rows

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[int, LayerConfig] = {
    1: LayerConfig("tiny-fp32-relu", 1, T=64, d=32, E=8, top_k=2, F=64,
                   capacity_factor=1.25, act=RELU, act_dtype=F32,
                   weight_dtype=F32, router_dtype=F32),
    2: LayerConfig("mixtral-8x-top2-4096x14336", 2, T=4096, d=4096, E=8,
                   top_k=2, F=14336),
    3: LayerConfig("deepseek-v3-256x-top8-group", 3, T=8192, d=7168, E=256,
                   top_k=8, F=2048, router=SIGMOID_GROUP, routed_scaling=2.5,
                   n_group=8, topk_group=4, shared_experts=1, shared_F=2048,
                   router_dtype=BF16, bias_range=0.05),
    4: LayerConfig("qwen-moe-128x-top8-zipf-skew", 4, T=16384, d=2048, E=128,
                   top_k=8, F=768, capacity_factor=1.0, zipf_s=1.1),
    5: LayerConfig("decode-u4-256x-top8", 5, T=32, d=2048, E=256, top_k=8,
                   F=512, weight_dtype=U4),
}


def seed_for(cfg_id: int, tensor_id: int, expert_id: int = 0,
             base: int = SEED_BASE) -> int:
    ss = np.random.SeedSequence([base, cfg_id, tensor_id, expert_id])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def gaussian(shape, std: float, seed: int, device) -> torch.Tensor:
    """fp32 N(0, std^2) draw."""
    t = torch.randn(shape, generator=_gen(seed, device), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def uniform(shape, lo: float, hi: float, seed: int, device) -> torch.Tensor:
    t = torch.rand(shape, generator=_gen(seed, device), device=device,
                   dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def _torch_dtype(name: str) -> torch.dtype:
    return {F32: torch.float32, BF16: torch.bfloat16}[name]


def _stacked(cfg: LayerConfig, tid: int, E: int, N: int, K: int, dtype,
             device, base: int) -> torch.Tensor:
    """[E, N, K] stack, expert e drawn from its own seed, std 1/sqrt(K)."""
    out = torch.empty((E, N, K), dtype=dtype, device=device)
    std = 1.0 / math.sqrt(K)
    for e in range(E):
        out[e] = gaussian((N, K), std, seed_for(cfg.cfg_id, tid, e, base),
                          device).to(dtype)
    return out


def quantize_u4_affine(w: torch.Tensor, group: int = 64):
    """Prepare 4-bit affine weights (input generation only).

    Per group of ``group`` consecutive K elements of one row: scale =
    (max-min)/15 and bias = min, both rounded to bf16; q = clamp(rint((w -
    bias)/scale), 0, 15) (q = 0 where scale is 0).  Eight codes are packed
    per 32-bit word, element 8j+i in nibble i (low nibble first).

    Returns (packed int32 [..., N, K/8], scale bf16 [..., N, K/group],
    bias bf16 [..., N, K/group]).
    """
    *lead, N, K = w.shape
    assert K % group == 0 and K % 8 == 0
    wf = w.float().reshape(*lead, N, K // group, group)
    mn = wf.amin(dim=-1)
    mx = wf.amax(dim=-1)
    scale = ((mx - mn) / 15.0).to(torch.bfloat16)
    bias = mn.to(torch.bfloat16)
    sf = scale.float().unsqueeze(-1)
    bf = bias.float().unsqueeze(-1)
    safe = torch.where(sf == 0, torch.ones_like(sf), sf)
    q = torch.round((wf - bf) / safe).clamp_(0, 15)
    q = torch.where(sf == 0, torch.zeros_like(q), q).to(torch.int64)
    q = q.reshape(*lead, N, K // 8, 8)
    shifts = torch.arange(8, device=w.device, dtype=torch.int64) * 4
    words = (q << shifts).sum(dim=-1)  # < 2^32
    words = torch.where(words >= 2**31, words - 2**32, words).to(torch.int32)
    return words, scale, bias


def make_layer_inputs(cfg: LayerConfig, device="cpu", base: int = SEED_BASE,
                      with_weights: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """All tensors of one layer workload on ``device``.

    Keys: x [T,d], w_router [E,d], expert_bias [E] or None, and when
    ``with_weights``: w_gate [E,F,d] (w_in for ReLU), w_up [E,F,d] or None,
    w_down [E,d,F]; for 4-bit weights q_gate/q_up/q_down (int32 packed) with
    s_*/b_* (bf16 scale/bias); for shared experts sh_gate/sh_up/sh_down.
    """
    c = cfg
    out: Dict[str, Optional[torch.Tensor]] = {}
    adt = _torch_dtype(c.act_dtype)
    x = gaussian((c.T, c.d), 1.0, seed_for(c.cfg_id, TID_X, 0, base), device)
    wr = gaussian((c.E, c.d), 1.0 / math.sqrt(c.d),
                  seed_for(c.cfg_id, TID_WR, 0, base), device)
    if c.zipf_s > 0.0:
        # popularity prior folded into the router rows through a constant
        # input channel: logit_e gets ln p_e, p_e ~ (e+1)^-s
        ranks = torch.arange(1, c.E + 1, dtype=torch.float64)
        p = ranks.pow(-c.zipf_s)
        p = p / p.sum()
        x[:, 0] = 1.0
        wr[:, 0] = torch.log(p).to(torch.float32).to(device)
    out["x"] = x.to(adt)
    out["w_router"] = wr.to(_torch_dtype(c.router_dtype))
    out["expert_bias"] = None
    if c.bias_range > 0.0:
        out["expert_bias"] = uniform((c.E,), -c.bias_range, c.bias_range,
                                     seed_for(c.cfg_id, TID_BIAS, 0, base),
                                     device)
    if not with_weights:
        return out
    if c.weight_dtype == U4:
        for name, tid, N, K in (("gate", TID_GATE, c.F, c.d),
                                ("up", TID_UP, c.F, c.d),
                                ("down", TID_DOWN, c.d, c.F)):
            qs, ss, bs = [], [], []
            for e in range(c.E):
                w = gaussian((N, K), 1.0 / math.sqrt(K),
                             seed_for(c.cfg_id, tid, e, base), device)
                q, s, b = quantize_u4_affine(w, c.quant_group)
                qs.append(q)
                ss.append(s)
                bs.append(b)
            out["q_" + name] = torch.stack(qs)
            out["s_" + name] = torch.stack(ss)
            out["b_" + name] = torch.stack(bs)
        out["w_gate"] = out["w_up"] = out["w_down"] = None
    else:
        wdt = _torch_dtype(c.weight_dtype)
        out["w_gate"] = _stacked(c, TID_GATE, c.E, c.F, c.d, wdt, device, base)
        out["w_up"] = (_stacked(c, TID_UP, c.E, c.F, c.d, wdt, device, base)
                       if c.act == SWIGLU else None)
        out["w_down"] = _stacked(c, TID_DOWN, c.E, c.d, c.F, wdt, device, base)
    if c.shared_experts > 0:
        sdt = adt
        S, Fs = c.shared_experts, c.shared_F
        out["sh_gate"] = _stacked(c, TID_SH_GATE, S, Fs, c.d, sdt, device, base)
        out["sh_up"] = (_stacked(c, TID_SH_UP, S, Fs, c.d, sdt, device, base)
                        if c.act == SWIGLU else None)
        out["sh_down"] = _stacked(c, TID_SH_DOWN, S, c.d, Fs, sdt, device, base)
    if c.layout == FUSED_GATE_UP:
        out = fuse_gate_up(out)
    return out


def fuse_gate_up(inp: Dict[str, Optional[torch.Tensor]]) -> Dict[str, Optional[torch.Tensor]]:
    """The same weights in the fused gate/up storage: for every pair
    (w_gate, w_up), (q_gate, q_up), (s_gate, s_up), (b_gate, b_up) and
    (sh_gate, sh_up) of [E, F, K] stacks, one [E, 2F, K] stack under
    <prefix>_gate_up holding each expert's gate rows followed by its up
    rows; the separate keys are dropped."""
    out = dict(inp)
    for pre in ("w", "q", "s", "b", "sh"):
        g, u = out.pop(pre + "_gate", None), out.pop(pre + "_up", None)
        if g is None:
            continue
        assert u is not None and u.shape == g.shape
        out[pre + "_gate_up"] = torch.cat([g, u], dim=1)
    return out


def host_array(t: Optional[torch.Tensor]):
    """Exact host copy as numpy: bf16 -> uint16 bit pattern, int32 packed
    words -> uint32 bit pattern, fp32 stays fp32."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()
