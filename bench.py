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
import csv
import glob
import hashlib
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


def _median(v):
    s = sorted(v)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def u4_expert_bytes(cfg) -> int:
    """Bytes of one routed expert's 4-bit weights: packed codes (half a byte
    per weight) plus a bf16 scale and bias per 64 weights of a row, for the
    gate, up and down matrices (1,769,472 B at d=2048, F=512)."""
    per_matrix = cfg.d * cfg.F // 2 + 2 * 2 * cfg.d * cfg.F // cfg.quant_group
    return 3 * per_matrix


def expert_flops(cfg, n_kept: int) -> float:
    """Algorithmic FLOPs of the expert FFN: 2*d*F per matrix per row (3
    matrices for SwiGLU, 2 for ReLU), routed kept rows plus shared experts
    on every token."""
    mats = 3 if cfg.act == "swiglu" else 2
    f = 2.0 * mats * cfg.d * cfg.F * n_kept
    if cfg.shared_experts:
        f += 2.0 * mats * cfg.d * cfg.shared_F * cfg.T * cfg.shared_experts
    return f


# sources of the kernels one grouped-FFN call runs (tile prefix, both expert
# GEMMs, the fold of a split down projection; the two 4-bit kernels): a
# traffic summary measured on other sources is stale
TRAFFIC_SOURCES = {"bf16": ("csrc/gemm_bf16.hip", "csrc/dispatch.hip", "csrc/combine.hip"),
                   "u4": ("csrc/gemm_u4.hip",)}
COPY_BYTES = 1 << 30  # calibration kernel: reads and writes 1 GiB
# counters are collected for the calibration copy and the FFN kernels only
TRAFFIC_REGEX = "neg_kernel|grouped_gemm|tile_prefix|fold_split|u4s_kernel"


def sources_digest(weight_dtype: str = "bf16") -> str:
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES["u4" if weight_dtype == "u4" else "bf16"]:
        with open(os.path.join(ROOT, "mixture_experts_layer_group_amd", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_summary_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"grouped_ffn_{workload}_hbm_traffic.md")


def measured_traffic(workload: str, weight_dtype: str = "bf16"):
    """HBM bytes per grouped-FFN call from the committed counter summary, or
    None when there is none or it was taken on other kernel sources."""
    path = traffic_summary_path(workload)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                vals[k.strip("`")] = v.strip().strip("`")
    if vals.get("sources_sha256") != sources_digest(weight_dtype):
        return None
    try:
        return float(vals["bytes_per_call"])
    except (KeyError, ValueError):
        return None


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
    # repeat whole oracle calls until about 10 s of CPU work (at most 4)
    reps, dt = 0, 0.0
    while reps < 4 and (reps == 0 or dt < 10.0):
        t0 = time.perf_counter()
        oracle.layer(host["x"], host["w_router"], bank, spec, host.get("expert_bias"),
                     tokens=toks)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": reps * len(toks) / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{reps} oracle layer calls, each routing+dispatch of all {cfg.T} tokens "
                      f"and expert FFN+combine of {len(toks)} seeded tokens (fp64 NumPy), "
                      f"{dt:.1f} s in total",
            "host_cpus": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(),
            "cpu_model": _cpu_model()}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload id (1-5)")
    ap.add_argument("--cpu-sample", type=int, default=4096,
                    help="tokens whose expert FFN the CPU oracle evaluates")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a 1 GiB copy and three grouped-FFN calls, for rocprofv3 --pmc")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two --pmc runs of --traffic-probe into the profiles/ summary")
    args = ap.parse_args()
    if args.summarize_traffic:
        return summarize_traffic(args)
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        return 2

    import torch
    import synth
    import mixture_experts_layer_group_amd as moe

    torch.cuda.set_device(0)
    cfg = synth.CONFIGS[args.config]
    u4 = cfg.weight_dtype == "u4"
    # the 4-bit decode layer touches ~290 MB of weights, about the size of
    # the 256 MB last-level cache: its timed steps rotate through three
    # independently drawn copies of the inputs (1.4 GB) so no step finds the
    # previous step's weights cached; larger layers exceed the cache anyway
    n_rep = 3 if u4 else 1
    reps = [synth.make_layer_inputs(cfg, "cuda", base=synth.SEED_BASE + r)
            for r in range(n_rep)]
    inp = reps[0]
    spec = moe.spec_from_config(cfg)
    T = cfg.T
    odt = torch.bfloat16 if cfg.out_dtype == "bf16" else torch.float32
    out = torch.empty((T, cfg.d), dtype=odt, device="cuda")
    ws = moe.workspace(spec, T)
    ws_all = [moe.expert_weights(r) for r in reps]
    w = ws_all[0]
    dev = "cuda"
    offs_all = [torch.empty(cfg.E + 1, dtype=torch.int32, device=dev) for _ in reps]
    st_all = [torch.empty(T * cfg.top_k, dtype=torch.int32, device=dev) for _ in reps]
    stats_all = [moe.layer_stats(offsets=o, sorted_token=t) for o, t in zip(offs_all, st_all)]
    offsets, sorted_token = offs_all[0], st_all[0]

    def step(i=0):
        r = i % n_rep
        moe.moe_layer_forward(spec, T, reps[r]["x"], reps[r]["w_router"],
                              reps[r]["expert_bias"], ws_all[r], out, stats=stats_all[r],
                              workspace=ws)

    if args.traffic_probe:
        return traffic_probe(torch, moe, spec, cfg, inp, w, offsets, sorted_token, ws, step)

    for i in range(max(args.warmup, n_rep)):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    tokens_per_s = T / (ms_step / 1e3)

    # the grouped expert FFN alone (both GEMMs), each call timed with HIP
    # events on the stream the kernels run on (rotating copies as above)
    kept = [int(o[-1].item()) for o in offs_all]
    touched = [int((o[1:] - o[:-1] > 0).sum().item()) for o in offs_all]
    n_kept = kept[0]
    y = torch.empty((T * cfg.top_k, cfg.d), dtype=torch.float32, device=dev)
    ysh = (torch.empty((cfg.shared_experts * T, cfg.d), dtype=torch.float32, device=dev)
           if cfg.shared_experts else None)

    def ffn(i):
        r = i % n_rep
        moe.moe_grouped_ffn(spec, T, offs_all[r], st_all[r], reps[r]["x"], ws_all[r], y, ysh,
                            ws)

    for i in range(max(2, n_rep)):
        ffn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        ffn(i)
        b.record()
    torch.cuda.synchronize()
    ffn_times = [a.elapsed_time(b) for a, b in evs]
    ffn_ms = sum(ffn_times) / len(ffn_times)
    flops = sum(expert_flops(cfg, kept[i % n_rep]) for i in range(args.steps)) / args.steps
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
        "roofline": {"bound": "mfma", "kernel": "grouped expert FFN call (tile prefix, "
                     "GEMM1 gate/up + SwiGLU, GEMM2 down, split fold)", "achieved": tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_BF16_TFLOPS, "flops_per_launch": flops,
                     "avg_launch_ms": ffn_ms, "median_launch_ms": _median(ffn_times),
                     "min_launch_ms": min(ffn_times), "traffic": measured_traffic(cfg.name)},
    }
    if u4:
        # bound by HBM: the touched experts' packed weights, the token rows
        # read and the fp32 expert rows written, per call (touched experts
        # counted on each copy's own routing)
        def ffn_bytes(r):
            return (touched[r] * u4_expert_bytes(cfg) + T * cfg.d * 2 + kept[r] * cfg.d * 4)
        byts = sum(ffn_bytes(i % n_rep) for i in range(args.steps)) / args.steps
        gbs = byts / (ffn_ms / 1e3) / 1e9
        res["roofline"] = {"bound": "hbm", "kernel": "grouped expert FFN call (both "
                           "4-bit expert kernels)", "achieved": gbs, "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                           "bytes_per_launch": byts, "avg_launch_ms": ffn_ms,
                           "median_launch_ms": _median(ffn_times),
                           "min_launch_ms": min(ffn_times),
                           "traffic": measured_traffic(cfg.name, "u4")}
        # the whole layer against HBM: the FFN's bytes plus the router
        # weights and the layer output
        layer_bytes = byts + cfg.E * cfg.d * (4 if cfg.router_dtype == "f32" else 2) \
            + T * cfg.d * (4 if cfg.out_dtype == "f32" else 2)
        res["layer_hbm_gbs"] = layer_bytes / (ms_step / 1e3) / 1e9
        res["touched_experts"] = touched
        res["input_copies_rotated"] = n_rep
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample)
    print(json.dumps(res), flush=True)
    return 0


def traffic_probe(torch, moe, spec, cfg, inp, w, offsets, sorted_token, ws, step) -> int:
    """Kernels for the HBM-traffic counters: an elementwise negation that
    reads and writes COPY_BYTES (the calibration of FETCH_SIZE and
    WRITE_SIZE), then three grouped-FFN calls on the routed batch."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    step()  # routing and dispatch for the FFN calls
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    y = torch.empty((cfg.T * cfg.top_k, cfg.d), dtype=torch.float32, device="cuda")
    ysh = (torch.empty((cfg.shared_experts * cfg.T, cfg.d), dtype=torch.float32,
                       device="cuda") if cfg.shared_experts else None)
    for _ in range(3):
        moe.moe_grouped_ffn(spec, cfg.T, offsets, sorted_token, inp["x"], w, y, ysh, ws)
    torch.cuda.synchronize()
    print("traffic probe done", flush=True)
    return 0


FFN_KERNELS = ("grouped_gemm_kernel", "tile_prefix_kernel", "fold_split_kernel", "u4s_kernel")


def _counter_rows(d):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize_traffic(args) -> int:
    """profiles/ summary of HBM traffic per grouped-FFN call: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) of the FFN kernels, each scaled by the
    ratio of the calibration kernel's known bytes to what the same counter
    read for it."""
    import synth
    cfg = synth.CONFIGS[args.config]
    res = {}
    for counter, d in (("FETCH_SIZE", args.summarize_traffic[0]),
                       ("WRITE_SIZE", args.summarize_traffic[1])):
        copy_kib, ffn = [], {}
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == counter]
        copies = [r for r in rows if "neg_kernel" in r["Kernel_Name"]]
        # the FFN calls are the dispatches after the last calibration copy
        last_copy = max((int(r["Dispatch_Id"]) for r in copies), default=None)
        for r in copies:
            copy_kib.append(float(r["Counter_Value"]))
        for r in rows:
            if last_copy is None or int(r["Dispatch_Id"]) <= last_copy:
                continue
            name = r["Kernel_Name"]
            for k in FFN_KERNELS:
                if k in name:
                    key = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
                    ffn.setdefault(key, []).append(float(r["Counter_Value"]))
        if not copy_kib or not ffn:
            print(f"no calibration or FFN dispatches for {counter} in {d}", file=sys.stderr)
            return 1
        factor = COPY_BYTES / (sum(copy_kib) / len(copy_kib) * 1024.0)
        # per call: every FFN kernel's mean per dispatch times its dispatches per call
        per_call = 0.0
        per_kernel = {}
        for k, vs in ffn.items():
            calls = 3
            kib = sum(vs) / calls
            per_kernel[k] = kib * 1024.0 * factor
            per_call += per_kernel[k]
        res[counter] = {"factor": factor, "copy_kib": copy_kib, "per_call": per_call,
                        "per_kernel": per_kernel}
    total = res["FETCH_SIZE"]["per_call"] + res["WRITE_SIZE"]["per_call"]
    path = traffic_summary_path(cfg.name)
    rel = os.path.relpath(path, ROOT)
    with open(path, "w") as f:
        f.write(f"# HBM traffic of one grouped-FFN call, {cfg.name}\n\n")
        f.write("Commands (repository root, one MI355X; the probe runs a 1 GiB elementwise "
                "negation for calibration, then three grouped-FFN calls):\n\n```\n")
        f.write("cd /tmp && export TMPDIR=/tmp\n")
        for c, dd in (("FETCH_SIZE", "pmc_fetch"), ("WRITE_SIZE", "pmc_write")):
            f.write(f"timeout -s KILL 120 rocprofv3 --kernel-include-regex '{TRAFFIC_REGEX}' "
                    f"--pmc {c} --output-format csv -d $REPO/gpurun_out/{dd} "
                    f"-o p -- python3 $REPO/bench.py --config {cfg.cfg_id} --traffic-probe\n")
        f.write(f"python3 $REPO/bench.py --config {cfg.cfg_id} --summarize-traffic "
                "$REPO/gpurun_out/pmc_fetch $REPO/gpurun_out/pmc_write\n```\n\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            r = res[c]
            f.write(f"{c}: calibration read {sum(r['copy_kib']) / len(r['copy_kib']):.0f} KiB for "
                    f"{COPY_BYTES >> 10} KiB moved, factor {r['factor']:.4f}\n\n")
            f.write("| kernel | bytes per call (scaled) |\n|---|---|\n")
            for k, b in sorted(res[c]["per_kernel"].items()):
                f.write(f"| `{k}` | {b:.4g} |\n")
            f.write("\n")
        f.write(f"- fetch_bytes_per_call: {res['FETCH_SIZE']['per_call']:.6g}\n")
        f.write(f"- write_bytes_per_call: {res['WRITE_SIZE']['per_call']:.6g}\n")
        f.write(f"- bytes_per_call: {total:.6g}\n")
        f.write(f"- sources_sha256: {sources_digest(cfg.weight_dtype)}\n")
    print(f"wrote {rel}: {total / 1e9:.3f} GB per call", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
