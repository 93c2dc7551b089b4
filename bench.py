#!/usr/bin/env python3
"""MoE layer forward benchmark on one MI355X.

A step is one whole moe_layer_forward (route -> dispatch -> grouped expert
FFN -> combine) over one batch of seeded synthetic tokens already resident
in HBM.  The default workload is the Mixtral-shaped layer (T=4096 tokens,
d=4096, 8 experts, top-2, SwiGLU FFN 14336, bf16 with fp32 accumulation,
fp32 router, no capacity limit).

Printed: ONE JSON line with tokens/s (value), the grouped expert GEMM
TFLOP/s and its fraction of the bf16 matrix-core peak, a roofline object for
the grouped FFN (both expert GEMMs, timed per call with HIP events on the
stream they run on), and the CPU oracle timed on a bounded sample of the same
workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/s + grouped-GEMM TFLOP/s (% bf16 MFMA peak), 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0


def expert_flops(cfg, n_kept: int) -> float:
    """Algorithmic FLOPs of the expert FFN: 2*d*F per matrix per row (3
    matrices for SwiGLU, 2 for ReLU), routed kept rows plus shared experts
    on every token."""
    mats = 3 if cfg.act == "swiglu" else 2
    f = 2.0 * mats * cfg.d * cfg.F * n_kept
    if cfg.shared_experts:
        f += 2.0 * mats * cfg.d * cfg.shared_F * cfg.T * cfg.shared_experts
    return f


def cpu_baseline(cfg, inp, sample: int):
    """The oracle as it stands, on the host cores: routing and dispatch of
    the whole batch plus the expert FFN of `sample` seeded tokens."""
    import numpy as np
    import oracle
    import synth
    from threadpoolctl import threadpool_info
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    host = {k: synth.host_array(v) for k, v in inp.items() if v is not None
            and k in ("x", "w_router", "expert_bias")}
    cache = {}

    def fetch(name, e):
        if (name, e) not in cache:
            cache[(name, e)] = synth.host_array(inp[name][e])
        return cache[(name, e)]

    bank = oracle.ExpertBank(fetch, cfg.act, u4=cfg.weight_dtype == "u4",
                             group=cfg.quant_group)
    spec = {"router": cfg.router, "E": cfg.E, "top_k": cfg.top_k, "act": cfg.act,
            "capacity_factor": cfg.capacity_factor, "shared_experts": cfg.shared_experts,
            "norm_topk_prob": cfg.norm_topk_prob, "routed_scaling": cfg.routed_scaling,
            "n_group": cfg.n_group, "topk_group": cfg.topk_group}
    toks = sorted(np.random.default_rng(0).choice(cfg.T, size=min(sample, cfg.T),
                                                  replace=False).tolist())
    # copy the expert tensors to the host before the clock starts (the oracle
    # works on host memory; the copy is not part of its arithmetic)
    for name in ("w_gate", "w_up", "w_down", "q_gate", "s_gate", "b_gate", "q_up",
                 "s_up", "b_up", "q_down", "s_down", "b_down", "sh_gate", "sh_up",
                 "sh_down"):
        if inp.get(name) is not None:
            for e in range(inp[name].shape[0]):
                fetch(name, e)
    t0 = time.perf_counter()
    oracle.layer(host["x"], host["w_router"], bank, spec, host.get("expert_bias"),
                 tokens=toks)
    dt = time.perf_counter() - t0
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"routing+dispatch of all {cfg.T} tokens, expert FFN+combine of "
                      f"{len(toks)} seeded tokens (fp64 NumPy), {dt:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload id (1-5)")
    ap.add_argument("--cpu-sample", type=int, default=2048,
                    help="tokens whose expert FFN the CPU oracle evaluates")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        return 2

    import torch
    import synth
    import mixture_experts_layer_group_amd as moe

    torch.cuda.set_device(0)
    cfg = synth.CONFIGS[args.config]
    inp = synth.make_layer_inputs(cfg, "cuda")
    spec = moe.spec_from_config(cfg)
    T = cfg.T
    odt = torch.bfloat16 if cfg.out_dtype == "bf16" else torch.float32
    out = torch.empty((T, cfg.d), dtype=odt, device="cuda")
    ws = moe.workspace(spec, T)
    w = moe.expert_weights(inp)
    dev = "cuda"
    offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
    sorted_token = torch.empty(T * cfg.top_k, dtype=torch.int32, device=dev)
    stats = moe.layer_stats(offsets=offsets, sorted_token=sorted_token)

    def step():
        moe.moe_layer_forward(spec, T, inp["x"], inp["w_router"], inp["expert_bias"],
                              w, out, stats=stats, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    tokens_per_s = T / (ms_step / 1e3)

    # the grouped expert FFN alone (both GEMMs), each call timed with HIP
    # events on the stream the kernels run on
    n_kept = int(offsets[-1].item())
    y = torch.empty((T * cfg.top_k, cfg.d), dtype=torch.float32, device=dev)
    ysh = (torch.empty((cfg.shared_experts * T, cfg.d), dtype=torch.float32, device=dev)
           if cfg.shared_experts else None)
    for _ in range(2):
        moe.moe_grouped_ffn(spec, T, offsets, sorted_token, inp["x"], w, y, ysh, ws)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        moe.moe_grouped_ffn(spec, T, offsets, sorted_token, inp["x"], w, y, ysh, ws)
        b.record()
    torch.cuda.synchronize()
    ffn_ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    flops = expert_flops(cfg, n_kept)
    tflops = flops / (ffn_ms / 1e3) / 1e12

    res = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "wall_s": wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act_dtype if cfg.weight_dtype != "u4" else "bf16+u4",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "d": cfg.d, "E": cfg.E,
                   "top_k": cfg.top_k, "F": cfg.F, "router": cfg.router,
                   "capacity_factor": cfg.capacity_factor,
                   "shared_experts": cfg.shared_experts,
                   "weights": cfg.weight_dtype, "parallelism": "none (1 GPU)"},
        "grouped_gemm_tflops": tflops,
        "grouped_gemm_frac_peak": tflops / PEAK_BF16_TFLOPS,
        "kept_rows": n_kept,
        "roofline": {"bound": "mfma", "kernel": "grouped expert FFN (GEMM1 gate/up + "
                     "SwiGLU, GEMM2 down)", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                     "flops_per_launch": flops, "avg_launch_ms": ffn_ms,
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
