"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare every stage with the CPU oracle, to the bars of the parity protocol:

  * router logits within the dot-product forward error bound
    |L_gpu - L| <= gamma_d * sum_j |x_j Wr_ej|, gamma_d = d u / (1 - d u),
    u = 2^-24 (fp32 accumulation of exact products);
  * routing ids bit-exact against the oracle's selection run on the GPU's
    own fp32 logits (near-tie tokens, margin < 1e-6, are reported; softmax
    ranking is decided on identical fp32 values, so all tokens must agree);
    weights within 1e-6;
  * dispatch (counts, offsets, permutation, slot rows, drops) bit-exact;
  * layer output max |err| <= 2e-2 * RMS(ref) for bf16 arithmetic and
    <= 1e-4 * RMS(ref) for fp32; when the output itself is stored in bf16,
    each element may further differ by the half-ulp of that final rounding
    (2^-8 |ref|); fully dropped tokens exactly 0.
"""
from __future__ import annotations

import math
import sys
import time
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import mixture_experts_layer_group_amd as moe
import oracle
import synth

BF16_TOL = 2e-2
F32_TOL = 1e-4


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def spec_dict(cfg) -> Dict:
    return {"router": cfg.router, "E": cfg.E, "top_k": cfg.top_k, "act": cfg.act,
            "capacity_factor": cfg.capacity_factor, "shared_experts": cfg.shared_experts,
            "norm_topk_prob": cfg.norm_topk_prob, "routed_scaling": cfg.routed_scaling,
            "n_group": cfg.n_group, "topk_group": cfg.topk_group}


def make_inputs(cfg, base=synth.SEED_BASE, device="cuda"):
    return synth.make_layer_inputs(cfg, device, base=base)


def run_layer(cfg, inp, T: Optional[int] = None):
    """moe_layer_forward with every optional output requested."""
    T = cfg.T if T is None else T
    spec = moe.spec_from_config(cfg)
    dev = "cuda"
    odt = torch.bfloat16 if cfg.out_dtype == synth.BF16 else torch.float32
    E, k = cfg.E, cfg.top_k
    r = {
        "out": torch.full((T, cfg.d), float("nan"), dtype=odt, device=dev),
        "topk_ids": torch.full((T, k), -7, dtype=torch.int32, device=dev),
        "topk_w": torch.zeros((T, k), dtype=torch.float32, device=dev),
        "logits": torch.zeros((T, E), dtype=torch.float32, device=dev),
        "counts_pre": torch.zeros(E, dtype=torch.int32, device=dev),
        "offsets": torch.zeros(E + 1, dtype=torch.int32, device=dev),
        "dropped": torch.zeros(1, dtype=torch.int32, device=dev),
        "prob_sum": torch.zeros(E, dtype=torch.float32, device=dev)
        if cfg.router == synth.SOFTMAX_TOPK else None,
        "slot_row": torch.full((T, k), -7, dtype=torch.int32, device=dev),
        "sorted_token": torch.full((max(1, T * k),), -7, dtype=torch.int32, device=dev),
        "errors": torch.zeros(1, dtype=torch.int32, device=dev),
    }
    ws = moe.workspace(spec, T)
    stats = moe.layer_stats(**{n: r[n] for n in moe._S_FIELDS})
    moe.moe_layer_forward(spec, T, inp["x"], inp["w_router"], inp["expert_bias"],
                          inp, r["out"], stats=stats, workspace=ws)
    torch.cuda.synchronize()
    # seeded inputs of the workloads are finite and O(1): no condition of
    # the device error word may be raised
    assert int(r["errors"].item()) == 0, f"device error word {int(r['errors'].item())}"
    return r


def bank_for(cfg, inp, experts: Optional[Sequence[int]] = None,
             threads: int = 8) -> oracle.ExpertBank:
    """Oracle expert bank over exact host copies of what the GPU read.

    Without ``experts`` each stored tensor is copied to the host on demand.
    With ``experts`` (the routed experts in the order the oracle visits
    them, i.e. ascending) a pool of ``threads`` copies and decodes them to
    fp64 ahead of the oracle, a bounded number at a time: the oracle's
    arithmetic is unchanged (it receives the matrices its own ``as_f64``
    decoded), only the decoding of large expert stacks runs in parallel."""
    cache: Dict = {}

    def raw(name, e):
        return synth.host_array(inp[name][e])

    if experts is None:
        def fetch(name, e):
            key = (name, e)
            if key not in cache:
                if len(cache) > 48:
                    cache.clear()
                cache[key] = raw(name, e)
            return cache[key]
    else:
        import concurrent.futures
        import threading
        u4 = cfg.weight_dtype == synth.U4
        fused = cfg.layout == synth.FUSED_GATE_UP
        if u4:
            names = ["q_gate_up", "s_gate_up", "b_gate_up"] if fused else \
                [p + m for m in ("gate", "up") for p in ("q_", "s_", "b_")]
            names += ["q_down", "s_down", "b_down"]
        else:
            names = ["w_gate_up"] if fused else \
                ["w_gate"] + (["w_up"] if cfg.act == synth.SWIGLU else [])
            names += ["w_down"]
        order = [(n, e) for e in experts for n in names]
        pos = {key: i for i, key in enumerate(order)}
        pool = concurrent.futures.ThreadPoolExecutor(threads)
        futs: Dict = {}
        lock = threading.Lock()
        ahead = 4 * threads
        nxt = [0]

        def decode(key):
            a = raw(*key)
            return a if u4 else oracle.as_f64(a)

        def submit_upto(i):
            with lock:
                while nxt[0] < len(order) and nxt[0] <= i + ahead:
                    key = order[nxt[0]]
                    futs[key] = pool.submit(decode, key)
                    nxt[0] += 1

        def fetch(name, e):
            key = (name, e)
            if key in pos:
                submit_upto(pos[key])
                fut = futs.pop(key, None)
                if fut is not None:
                    return fut.result()
            if name.startswith("sh_") or key not in pos:
                return raw(name, e)
            return decode(key)

    return oracle.ExpertBank(fetch, cfg.act, u4=cfg.weight_dtype == synth.U4,
                             group=cfg.quant_group,
                             fused=cfg.layout == synth.FUSED_GATE_UP)


def fp16_rows_bound(y_rows, slot_row, topk_w, parts: int = 1):
    """Elementwise bound on what keeping the expert rows in fp16 (as the
    layer does on the matrix-core path) changes in the combined output:
    each of a row's `parts` fp16 parts is off by at most 2^-11 of its
    magnitude, taken here as the whole row's with headroom for parts that
    partly cancel (4x when the down projection's K halves are stored apart),
    weighted by |w| and summed over the token's kept slots."""
    import torch
    f = 2.0 ** -11 * (1.0 if parts == 1 else 4.0)
    T, k = slot_row.shape
    bound = torch.zeros((T, y_rows.shape[1]), dtype=torch.float32, device=y_rows.device)
    for i in range(k):
        r = slot_row[:, i].long()
        kept = (r >= 0)
        rows = y_rows[r.clamp(min=0)].abs() * topk_w[:, i:i + 1].abs()
        bound += torch.where(kept[:, None], rows, torch.zeros_like(rows))
    return bound * f


def last_tile_tokens(disp, per_expert: int = 1, bm: int = 256):
    """Tokens whose rows lie in the last M tile of each expert's group (the
    ragged tail the grouped GEMM handles specially), up to ``per_expert``
    of them per expert."""
    off = disp["offsets"]
    st = disp["sorted_token"]
    out = []
    for e in range(len(off) - 1):
        n = int(off[e + 1] - off[e])
        if n == 0:
            continue
        start = int(off[e]) + (n - 1) // bm * bm
        rows = list(range(int(off[e + 1]) - 1, start - 1, -1))[:per_expert]
        out += [int(st[r]) for r in rows]
    return out


def logits_bound(x_h, wr_h, d):
    """Forward error bound of an fp32-accumulated dot product of d exact
    products, in any summation order: gamma_d * sum |x||w|, gamma_d =
    d u / (1 - d u), u = 2^-24."""
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    X = np.abs(oracle.as_f64(x_h))
    W = np.abs(oracle.as_f64(wr_h))
    return gamma * (X @ W.T)


def check_route(cfg, inp, r, full_logits_check=True):
    """Logits bound, ids bit-exact vs the oracle on the GPU logits, weights
    within 1e-6.  Returns (ids_gpu, w_oracle (fp64), flags)."""
    spec = spec_dict(cfg)
    L_gpu = r["logits"].cpu().numpy()
    x_h, wr_h = synth.host_array(inp["x"]), synth.host_array(inp["w_router"])
    bias_h = synth.host_array(inp["expert_bias"])
    if full_logits_check:
        L_ref = oracle.router_logits(x_h, wr_h)
        bound = logits_bound(x_h, wr_h, cfg.d)
        err = np.abs(L_gpu.astype(np.float64) - L_ref)
        assert np.all(err <= bound), f"logits outside the fp32 dot bound: {(err - bound).max()}"
    ids_o, w_o, p_o = oracle.route_from_logits(L_gpu, spec, bias_h)
    flags = oracle.near_tie_flags(L_gpu, spec, bias_h)
    ids_g = r["topk_ids"].cpu().numpy()
    w_g = r["topk_w"].cpu().numpy().astype(np.float64)
    bad = np.any(ids_g != ids_o, axis=1)
    log(f"  route: {int(flags.sum())} near-tie tokens, {int(bad.sum())} id mismatches "
        f"({int((bad & ~flags).sum())} unflagged)")
    assert not np.any(bad & ~flags), "routing ids differ on unflagged tokens"
    if cfg.router == synth.SOFTMAX_TOPK:
        assert not np.any(bad), "softmax ranking is decided on identical fp32 values"
    ok = ~bad
    assert np.all(np.abs(w_g[ok] - w_o[ok]) <= 1e-6), \
        f"routing weights off by {np.abs(w_g[ok] - w_o[ok]).max()}"
    # downstream stages follow the GPU routing: a flagged token whose ids
    # differ keeps the GPU's ids and weights together
    w_o = w_o.copy()
    w_o[bad] = w_g[bad]
    if r.get("prob_sum") is not None and p_o is not None:
        ps = r["prob_sum"].cpu().numpy().astype(np.float64)
        ref = p_o.sum(axis=0)
        assert np.all(np.abs(ps - ref) <= 1e-6 * cfg.T + 1e-5 * np.abs(ref)), \
            f"prob_sum off by {np.abs(ps - ref).max()}"
    return ids_g, w_o, flags


def check_dispatch(cfg, ids_g, r):
    T, k, E = cfg.T, cfg.top_k, cfg.E
    cap = oracle.capacity_for(T, k, E, cfg.capacity_factor)
    d = oracle.dispatch(ids_g, E, cap)
    n = int(d["offsets"][E])
    assert np.array_equal(r["counts_pre"].cpu().numpy(), d["count_pre"]), "counts_pre"
    assert np.array_equal(r["offsets"].cpu().numpy(), d["offsets"]), "offsets"
    assert int(r["dropped"].cpu().item()) == d["dropped"], "dropped"
    assert np.array_equal(r["sorted_token"].cpu().numpy()[:n], d["sorted_token"]), "sorted_token"
    assert np.array_equal(r["slot_row"].cpu().numpy(), d["slot_row"]), "slot_row"
    log(f"  dispatch: capacity {cap}, kept {n}, dropped {d['dropped']} (bit-exact)")
    return d


def check_output(cfg, inp, r, ids_g, w_o, disp, tokens: Optional[Sequence[int]] = None,
                 prefetch: bool = False):
    tol = BF16_TOL if cfg.act_dtype == synth.BF16 else F32_TOL
    toks = list(range(cfg.T)) if tokens is None else list(tokens)
    experts = None
    if prefetch:
        sr = disp["slot_row"]
        experts = sorted({int(ids_g[t, i]) for t in toks for i in range(cfg.top_k)
                          if sr[t, i] >= 0})
    bank = bank_for(cfg, inp, experts)
    t0 = time.time()
    ref = oracle.ffn_and_combine(synth.host_array(inp["x"]), ids_g, w_o, disp, bank,
                                 spec_dict(cfg), toks)
    got = r["out"].float().cpu().numpy().astype(np.float64)[toks]
    rms = math.sqrt(float(np.mean(ref ** 2)))
    # bf16 output: the same bar, the final rounding to bf16 included
    absdiff = np.abs(got - ref)
    err = float(absdiff.max())
    log(f"  output: {len(toks)} tokens, max|err| {err:.3e}, RMS(ref) {rms:.3e}, "
        f"ratio {err / max(rms, 1e-300):.2e} (bar {tol}), oracle {time.time() - t0:.1f}s")
    assert err <= tol * rms, f"max|err| {err} > {tol} * RMS {rms}"
    # fully dropped tokens with no shared expert are exactly zero
    if cfg.shared_experts == 0:
        sr = disp["slot_row"]
        dead = [j for j, t in enumerate(toks) if np.all(sr[t] < 0)]
        if dead:
            assert np.all(got[dead] == 0.0), "fully dropped tokens must give exactly 0"
            log(f"  {len(dead)} fully dropped tokens are exactly 0")
    return err, rms


def logit_error_flags(cfg, L, B, bias):
    """Tokens whose top-k set could change when every logit moves by up to
    B[t] (the GPU's fp32 logits differ from the fp64 ones by at most that
    much -- the measured difference, itself checked against the
    dot-product error bound): the boundary gap of the ranked scores is
    within twice the largest possible score change.  Softmax ranks logits directly; sigmoid scores move by at
    most B/4 (the sigmoid's slope is at most 1/4) and group scores, sums of
    two of them, by at most B/2."""
    T, E = L.shape
    k = cfg.top_k
    flags = np.zeros(T, dtype=bool)
    if cfg.router == synth.SOFTMAX_TOPK:
        if k < E:
            srt = -np.sort(-L, axis=1)
            flags |= (srt[:, k - 1] - srt[:, k]) <= 2 * B
        return flags
    s = 1.0 / (1.0 + np.exp(-L))
    sel = s + (bias.astype(np.float64)[None, :] if bias is not None else 0.0)
    G = E // cfg.n_group
    grp = -np.sort(-sel.reshape(T, cfg.n_group, G), axis=2)
    gs = grp[:, :, 0] + grp[:, :, 1]
    if cfg.topk_group < cfg.n_group:
        gsrt = -np.sort(-gs, axis=1)
        flags |= (gsrt[:, cfg.topk_group - 1] - gsrt[:, cfg.topk_group]) <= 2 * (B / 2)
        drop = oracle.rank_descending(gs)[:, cfg.topk_group:]
        m = sel.reshape(T, cfg.n_group, G).copy()
        m[np.arange(T)[:, None], drop, :] = -np.inf
        sel = m.reshape(T, E)
    if k < cfg.topk_group * G:
        srt = -np.sort(-sel, axis=1)
        flags |= (srt[:, k - 1] - srt[:, k]) <= 2 * (B / 4)
    return flags


def check_end_to_end_routing(cfg, inp, ids_g, L_gpu):
    """The set of experts each token chose from the oracle's own fp64 logits
    agrees with the GPU's except on tokens that are near ties (margin < 1e-6
    of the oracle's selection scores) or whose decision lies within the
    GPU's logit rounding (see logit_error_flags).  The order inside the
    top-k is compared bit-exactly on shared fp32 logits in check_route."""
    spec = spec_dict(cfg)
    x_h, wr_h = synth.host_array(inp["x"]), synth.host_array(inp["w_router"])
    bias_h = synth.host_array(inp["expert_bias"])
    L = oracle.router_logits(x_h, wr_h)
    ids_o, _, _ = oracle.route_from_logits(L, spec, bias_h)
    B = np.abs(L_gpu.astype(np.float64) - L).max(axis=1)
    flags = oracle.near_tie_flags(L, spec, bias_h) | logit_error_flags(cfg, L, B, bias_h)
    bad = np.any(np.sort(ids_o, axis=1) != np.sort(ids_g, axis=1), axis=1)
    log(f"  end-to-end routing: {int(bad.sum())} tokens differ, {int((bad & ~flags).sum())} "
        f"unflagged (flagged {int(flags.sum())} of {cfg.T})")
    assert not np.any(bad & ~flags)


def full_check(cfg, inp, r, tokens=None, full_logits_check=True, choose_tokens=None):
    """Route, dispatch and output parity.  ``choose_tokens(disp)`` may pick
    the output sample from the dispatch (e.g. the tokens of every expert's
    last M tile); their expert matrices are then decoded in parallel."""
    ids_g, w_o, flags = check_route(cfg, inp, r, full_logits_check)
    disp = check_dispatch(cfg, ids_g, r)
    if choose_tokens is not None:
        tokens = choose_tokens(disp)
    check_output(cfg, inp, r, ids_g, w_o, disp, tokens, prefetch=choose_tokens is not None)
    return ids_g, disp
