#!/usr/bin/env python3
"""MoE layer forward benchmark on one MI355X.

A step is one whole moe_layer_forward (route -> dispatch -> grouped expert
FFN -> combine) over one batch of seeded synthetic tokens already resident
in HBM.  The default workload is the Mixtral-shaped layer (T=4096 tokens,
d=4096, 8 experts, top-2, SwiGLU FFN 14336, bf16 with fp32 accumulation,
fp32 router, no capacity limit).

Printed: ONE JSON line with tokens/s (value); the grouped expert GEMM
TFLOP/s (gate/up + down, both launches as the layer issues them) and its
fraction of the bf16 matrix-core peak; a roofline object for the dominant
kernel (the gate/up grouped GEMM; the 4-bit FFN against HBM on the decode
workload); a `decode` object from the decode-shaped 4-bit layer timed in the
same run (its HBM roofline); and the CPU oracle timed on a bounded sample of
the same workload (cpu_baseline).  Every kernel time comes from HIP events
that moe_layer_forward records on its own stream inside the timed steps
(moe_layer_stats.ffn_events).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import subprocess
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


# sources of the kernels whose HBM traffic the roofline quotes (the bf16
# grouped GEMMs; the two 4-bit kernels): a traffic summary measured on other
# sources is stale
TRAFFIC_SOURCES = {"bf16": ("csrc/gemm_bf16.hip",), "u4": ("csrc/gemm_u4.hip",)}
COPY_BYTES = 1 << 30  # calibration kernel: reads and writes 1 GiB
# counters are collected for the calibration copy and the expert kernels only
TRAFFIC_REGEX = "neg_kernel|grouped_gemm|u4s_kernel"
# the router, dispatch and combine kernels (their HBM traffic, summarised
# with --side)
SIDE_KERNELS = ("logits_", "select_kernel", "count_kernel", "scan_kernel", "scatter_kernel",
                "dispatch_small_kernel", "combine_kernel")
SIDE_REGEX = "neg_kernel|" + "|".join(SIDE_KERNELS)
SIDE_SOURCES = ("csrc/router.hip", "csrc/dispatch.hip", "csrc/combine.hip")
# kernel-name fragments of the dominant kernels in the profiler's summaries:
# the routed bf16 gate/up GEMM (SwiGLU mode, gathered rows; any tile size)
# and the 4-bit weight-stream kernels
GATE_UP_KEY = "grouped_gemm_kernel<0, true,"
U4_STREAM_KEY = "u4s_kernel"
# matrix-core counters of the bf16 expert GEMMs (one rocprofv3 pass)
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                 "SQ_INSTS_VALU_MFMA_MOPS_F16 GRBM_GUI_ACTIVE")
SIMDS = 4 * 256  # MI355X: 256 CUs of 4 SIMDs


def kernel_label(name: str) -> str:
    """A profiler's kernel name as a readable template id without the
    argument list.  rocprofv3 leaves a name mangled when it holds the
    _Float16 builtin type (Itanium code DF16_), which c++filt cannot read;
    that code is demangled here as the half type (Dh) and printed back as
    _Float16."""
    if name.startswith("_Z"):
        try:
            r = subprocess.run(["c++filt", name.replace("DF16_", "Dh")],
                               capture_output=True, text=True, timeout=30)
            if r.returncode == 0 and not r.stdout.startswith("_Z"):
                name = re.sub(r"\bhalf\b", "_Float16", r.stdout.strip())
        except (OSError, subprocess.SubprocessError):
            pass
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[len("void "):]
    depth, out = 0, ""
    for ch in name:
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out += ch
    return out


def sources_digest(weight_dtype: str = "bf16") -> str:
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES["u4" if weight_dtype == "u4" else "bf16"]:
        with open(os.path.join(ROOT, "mixture_experts_layer_group_amd", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_summary_path(workload: str, side: bool = False) -> str:
    if side:
        return os.path.join(ROOT, "profiles", f"side_kernels_{workload}_hbm_traffic.md")
    return os.path.join(ROOT, "profiles", f"expert_gemms_{workload}_hbm_traffic.md")


def side_sources_digest() -> str:
    h = hashlib.sha256()
    for rel in SIDE_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_group_amd", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes (read + written) per layer call of the expert kernels whose
    name contains `kernel`, from the committed counter summary; None when
    there is none or it was taken on other kernel sources."""
    path = traffic_summary_path(workload)
    if not os.path.exists(path):
        return None
    digest, total, found = None, 0.0, False
    with open(path) as f:
        for line in f:
            if line.startswith("- sources_sha256: "):
                digest = line.split(": ", 1)[1].strip()
            elif line.startswith("- per_call[") and "]: " in line:
                key, v = line[len("- per_call["):].rsplit("]: ", 1)
                if kernel in key:
                    total += float(v)
                    found = True
    wd = "u4" if "u4s" in kernel else "bf16"
    if digest != sources_digest(wd) or not found:
        return None
    return total


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded (ctypes),
    for the library to record on its stream."""

    def __init__(self, n: int):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h.value)

    def ms(self, a: int, b: int) -> float:
        t = self.ct.c_float()
        self.hip.hipEventSynchronize(self.ev[b])
        if self.hip.hipEventElapsedTime(self.ct.byref(t), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def time_layer(torch, moe, cfg, steps: int, warmup: int, n_rep: int, graph: bool = False,
               split: bool = True):
    """Warm-up, then two timed passes of `steps` moe_layer_forward calls of
    workload `cfg`, rotating through `n_rep` independently drawn input
    copies: the first, plain, gives the per-step layer time (torch events
    around the loop, nothing else recorded); the second has the layer record
    HIP events around its expert kernels (moe_layer_stats.ffn_events), which
    give the gate/up and down (+ shared) kernel times of every step.
    Also returns kept rows and touched experts of each copy."""
    import synth
    reps = [synth.make_layer_inputs(cfg, "cuda", base=synth.SEED_BASE + r)
            for r in range(n_rep)]
    spec = moe.spec_from_config(cfg)
    T = cfg.T
    odt = torch.bfloat16 if cfg.out_dtype == "bf16" else torch.float32
    out = torch.empty((T, cfg.d), dtype=odt, device="cuda")
    ws = moe.workspace(spec, T)
    wts = [moe.expert_weights(r) for r in reps]
    offs = [torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda") for _ in reps]
    ev = HipEvents(3 * steps)
    plain = [moe.layer_stats(offsets=o) for o in offs]
    # split=False: no event between the two expert kernels (for layers of a
    # few tens of µs, where recording one costs a visible share)
    timed = [moe.layer_stats(offsets=offs[i % n_rep],
                             ffn_events=[ev.ev[3 * i], ev.ev[3 * i + 1] if split else 0,
                                         ev.ev[3 * i + 2]]) for i in range(steps)]

    def step(i, st):
        r = i % n_rep
        moe.moe_layer_forward(spec, T, reps[r]["x"], reps[r]["w_router"],
                              reps[r]["expert_bias"], wts[r], out, stats=st, workspace=ws)

    def timed_pass(stats_of):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            step(i, stats_of(i))
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, time.perf_counter() - t0

    for i in range(max(warmup, n_rep)):
        step(i, plain[i % n_rep])
    ms_step, wall = timed_pass(lambda i: plain[i % n_rep])
    ms_step_ev, _ = timed_pass(lambda i: timed[i])
    ms_graph = None
    if graph:
        # one HIP graph per input copy, captured from the same C-ABI call
        # (kernels only: no memset, allocation or host synchronisation)
        graphs = []
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            for r in range(n_rep):
                step(r, plain[r])
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        for r in range(n_rep):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(r, plain[r])
            graphs.append(gr)
        torch.cuda.synchronize()
        for i in range(max(warmup, n_rep)):
            graphs[i % n_rep].replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for i in range(steps):
            graphs[i % n_rep].replay()
        g1.record()
        torch.cuda.synchronize()
        ms_graph = g0.elapsed_time(g1) / steps
    if split:
        up = [ev.ms(3 * i, 3 * i + 1) for i in range(steps)]
        down = [ev.ms(3 * i + 1, 3 * i + 2) for i in range(steps)]
    else:  # the whole expert FFN as "up", nothing as "down"
        up = [ev.ms(3 * i, 3 * i + 2) for i in range(steps)]
        down = [0.0] * steps
    ev.close()
    kept = [int(o[-1].item()) for o in offs]
    touched = [int((o[1:] - o[:-1] > 0).sum().item()) for o in offs]
    return {"ms_step": ms_step, "ms_step_events": ms_step_ev, "ms_step_graph": ms_graph,
            "wall": wall, "up": up, "down": down, "kept": kept, "touched": touched,
            "inp": reps[0]}


def decode_leg(torch, moe, steps: int, warmup: int):
    """The decode-shaped 4-bit layer (T=32, d=2048, 256 experts, top-8,
    SwiGLU 512), timed like the headline workload over three rotated input
    copies (its ~290 MB of touched weights would otherwise sit in the
    256 MB last-level cache between steps); HBM roofline of the layer and of
    its two 4-bit expert kernels (timed together, between two events the
    layer records before the first and after the second); the layer also
    replayed from HIP graphs."""
    import synth
    cfg = synth.CONFIGS[5]
    n_rep = 3
    r = time_layer(torch, moe, cfg, steps, warmup, n_rep, graph=True, split=False)
    ffn = r["up"]

    def ffn_bytes(j):
        return (r["touched"][j] * u4_expert_bytes(cfg) + cfg.T * cfg.d * 2
                + r["kept"][j] * cfg.d * 4)
    byts = sum(ffn_bytes(i % n_rep) for i in range(steps)) / steps
    ffn_ms = sum(ffn) / len(ffn)
    layer_bytes = byts + cfg.E * cfg.d * 4 + cfg.T * cfg.d * 4
    return {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "top_k": cfg.top_k,
            "F": cfg.F, "weights": "u4-affine-g64", "steps": steps,
            "input_copies_rotated": n_rep,
            "layer_us": r["ms_step"] * 1e3, "tokens_per_s": cfg.T / (r["ms_step"] / 1e3),
            "layer_us_with_events": r["ms_step_events"] * 1e3,
            "layer_us_graph_replay": r["ms_step_graph"] * 1e3,
            "tokens_per_s_graph_replay": cfg.T / (r["ms_step_graph"] / 1e3),
            "ffn_us": ffn_ms * 1e3,
            "touched_experts": r["touched"],
            "ffn_bytes_per_call": byts,
            "ffn_hbm_gbs": byts / (ffn_ms / 1e3) / 1e9,
            "ffn_frac_hbm": byts / (ffn_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
            "layer_bytes": layer_bytes,
            "layer_hbm_gbs": layer_bytes / (r["ms_step"] / 1e3) / 1e9,
            "layer_frac_hbm": layer_bytes / (r["ms_step"] / 1e3) / 1e9 / PEAK_HBM_GBS,
            "peak_hbm_gbs": PEAK_HBM_GBS}


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
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-shaped 4-bit layer's object")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a 1 GiB copy and three layer calls, for rocprofv3 --pmc")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two --pmc runs of --traffic-probe into the profiles/ summary")
    ap.add_argument("--side", action="store_true",
                    help="with --summarize-traffic: the router, dispatch and combine kernels")
    ap.add_argument("--vendor-compare", action="store_true",
                    help="time torch.matmul per expert on the workload's kept-row counts "
                         "against this library's expert kernels; writes profiles/")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_DIR", "BENCH_LOG"),
                    help="turn a rocprofv3 --kernel-trace --stats run of bench.py and that "
                         "run's output into the profiles/ kernel-time summary")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="turn a --pmc run of --traffic-probe with the matrix-core counters "
                         "into the profiles/ summary")
    args = ap.parse_args()
    if args.summarize_traffic:
        return summarize_traffic(args)
    if args.summarize_mfma:
        return summarize_mfma(args)
    if args.summarize_stats:
        return summarize_stats(args)
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
    if args.traffic_probe:
        return traffic_probe(torch, moe, cfg)
    if args.vendor_compare:
        return vendor_compare(torch, moe, cfg, args.steps, args.warmup)
    # the 4-bit decode layer touches ~290 MB of weights, about the size of
    # the 256 MB last-level cache: its timed steps rotate through three
    # independently drawn copies of the inputs (1.4 GB) so no step finds the
    # previous step's weights cached; larger layers exceed the cache anyway
    n_rep = 3 if u4 else 1
    r = time_layer(torch, moe, cfg, args.steps, args.warmup, n_rep)
    T = cfg.T
    ms_step = r["ms_step"]
    tokens_per_s = T / (ms_step / 1e3)
    steps = args.steps
    up_ms = sum(r["up"]) / steps
    down_ms = sum(r["down"]) / steps
    ffn_times = [a + b for a, b in zip(r["up"], r["down"])]
    ffn_ms = sum(ffn_times) / steps
    kept = r["kept"]
    n_kept = kept[0]
    flops = sum(expert_flops(cfg, kept[i % n_rep]) for i in range(steps)) / steps
    tflops = flops / (ffn_ms / 1e3) / 1e12
    mats = 3 if cfg.act == "swiglu" else 2
    up_flops = sum(2.0 * (mats - 1) * cfg.d * cfg.F * kept[i % n_rep]
                   for i in range(steps)) / steps
    up_tflops = up_flops / (up_ms / 1e3) / 1e12
    if cfg.act_dtype == "f32":
        dtype = "f32"
    elif u4:
        dtype = "bf16 x u4-affine (codes as exact fp16 on the matrix cores), fp32 accumulate"
    else:
        dtype = "bf16 (gate/up products), fp16 (down products: fp16 hidden x bf16 weights converted to fp16), fp32 accumulate"

    res = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "wall_s": r["wall"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "d": cfg.d, "E": cfg.E,
                   "top_k": cfg.top_k, "F": cfg.F, "router": cfg.router,
                   "capacity_factor": cfg.capacity_factor,
                   "shared_experts": cfg.shared_experts,
                   "weights": cfg.weight_dtype, "parallelism": "none (1 GPU)"},
        "grouped_gemm_tflops": tflops,
        "grouped_gemm_frac_peak": tflops / PEAK_BF16_TFLOPS,
        "grouped_gemm": {"kernels": "routed gate/up GEMM + down GEMM (+ shared expert "
                         "GEMMs), timed between HIP events the layer records around them "
                         "in every step of a second timed pass", "flops_per_step": flops,
                         "layer_ms_per_step_with_events": r["ms_step_events"],
                         "avg_ms": ffn_ms, "median_ms": _median(ffn_times),
                         "min_ms": min(ffn_times), "up_avg_ms": up_ms,
                         "down_avg_ms": down_ms, "tflops": tflops,
                         "frac_peak_bf16": tflops / PEAK_BF16_TFLOPS},
        "kept_rows": n_kept,
        "roofline": {"bound": "mfma",
                     "kernel": "grouped_gemm_kernel<SwiGLU> (routed gate/up GEMM + SwiGLU "
                               "epilogue, the dominant kernel)",
                     "achieved": up_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": up_tflops / PEAK_BF16_TFLOPS,
                     "flops_per_launch": up_flops, "avg_launch_ms": up_ms,
                     "median_launch_ms": _median(r["up"]), "min_launch_ms": min(r["up"]),
                     "traffic": measured_traffic(cfg.name, GATE_UP_KEY)},
    }
    if u4:
        def ffn_bytes(j):
            return (r["touched"][j] * u4_expert_bytes(cfg) + T * cfg.d * 2
                    + kept[j] * cfg.d * 4)
        byts = sum(ffn_bytes(i % n_rep) for i in range(steps)) / steps
        gbs = byts / (ffn_ms / 1e3) / 1e9
        res["roofline"] = {"bound": "hbm", "kernel": "both 4-bit expert kernels "
                           "(u4s_kernel gate/up, down) as the layer issues them",
                           "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": gbs / PEAK_HBM_GBS, "bytes_per_launch": byts,
                           "avg_launch_ms": ffn_ms, "median_launch_ms": _median(ffn_times),
                           "min_launch_ms": min(ffn_times),
                           "traffic": measured_traffic(cfg.name, U4_STREAM_KEY)}
        res["touched_experts"] = r["touched"]
        res["input_copies_rotated"] = n_rep
    elif not args.no_decode:
        res["decode"] = decode_leg(torch, moe, args.steps, args.warmup)
    inp = r["inp"]
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample)
    print(json.dumps(res), flush=True)
    return 0


def vendor_compare(torch, moe, cfg, steps: int, warmup: int) -> int:
    """The vendor library on the layer's own expert products: torch.matmul
    (hipBLASLt) once per expert, with the kept-row counts this library's
    routing gives the workload, on contiguous bf16 rows (no gather, no
    SwiGLU, no weighting), against this library's routed gate/up and down
    kernels timed between the layer's events.  Writes
    profiles/vendor_gemm_<workload>.md.  bf16 weights only."""
    import synth
    if cfg.weight_dtype != "bf16" or cfg.act_dtype != "bf16":
        print("--vendor-compare needs a bf16 workload", file=sys.stderr)
        return 2
    r = time_layer(torch, moe, cfg, steps, warmup, 1)
    # per-expert kept rows of the same inputs
    spec = moe.spec_from_config(cfg)
    inp = r["inp"]
    offs = torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda")
    out = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    moe.moe_layer_forward(spec, cfg.T, inp["x"], inp["w_router"], inp["expert_bias"], inp,
                          out, stats=moe.layer_stats(offsets=offs),
                          workspace=moe.workspace(spec, cfg.T))
    torch.cuda.synchronize()
    o = offs.cpu().tolist()
    cnt = [o[e + 1] - o[e] for e in range(cfg.E)]
    del inp, out
    r["inp"] = None
    torch.cuda.empty_cache()
    d, F = cfg.d, cfg.F
    nup = 2 * F if cfg.act == "swiglu" else F
    g = torch.Generator(device="cuda").manual_seed(7)
    X = [torch.randn(c, d, device="cuda", dtype=torch.bfloat16, generator=g) for c in cnt if c]
    H = [torch.randn(c, F, device="cuda", dtype=torch.bfloat16, generator=g) for c in cnt if c]
    # [N][K] row-major weights as the layer stores them, passed transposed
    # (a 2-D product: K-contiguous B, no batch)
    W1 = [torch.randn(nup, d, device="cuda", dtype=torch.bfloat16, generator=g) * 0.02
          for c in cnt if c]
    W2 = [torch.randn(d, F, device="cuda", dtype=torch.bfloat16, generator=g) * 0.02
          for c in cnt if c]
    rows = sum(cnt)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def up():
        for x, w in zip(X, W1):
            torch.matmul(x, w.t())

    def down():
        for h, w in zip(H, W2):
            torch.matmul(h, w.t())

    def graphed(fn):
        # the same per-expert loop captured once and replayed: the GPU time
        # without the host's per-call launch cost
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            fn()
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        return timed(gr.replay)

    v_up, v_down = timed(up), timed(down)
    g_up, g_down = graphed(up), graphed(down)
    ours_up = sum(r["up"]) / len(r["up"])
    ours_down = sum(r["down"]) / len(r["down"])
    f_up, f_down = 2.0 * rows * nup * d, 2.0 * rows * d * F
    lines = [f"# Vendor GEMM against this library's expert kernels, {cfg.name}", "",
             "Command (repository root, one MI355X):", "", "```",
             f"python3 bench.py --config {cfg.cfg_id} --vendor-compare --steps {steps} "
             f"--warmup {warmup}",
             "```", "",
             f"Kept rows per expert (this library's routing of the seeded inputs): "
             f"{min(cnt)}-{max(cnt)}, {rows} in total over {sum(1 for c in cnt if c)} experts.", "",
             "Vendor: one torch.matmul (hipBLASLt) per expert on contiguous bf16 rows with "
             "random data of the same shapes, no gather, no activation; this library: the "
             "routed kernels between the layer's HIP events (gate/up with the gathered rows "
             "and the SwiGLU / ReLU epilogue; down" +
             (" plus the shared experts' products" if cfg.shared_experts else "") + ").", "",
             "The vendor loop is timed as issued from the host and as one captured HIP "
             "graph (its GPU time without the per-call launch cost).", "",
             "| product | this library (µs) | TFLOP/s | vendor loop (µs) | TFLOP/s "
             "| vendor loop in a graph (µs) | TFLOP/s |",
             "|---|---|---|---|---|---|---|",
             f"| gate/up | {ours_up * 1e3:.1f} | {f_up / ours_up / 1e9:.0f} | "
             f"{v_up * 1e3:.1f} | {f_up / v_up / 1e9:.0f} | "
             f"{g_up * 1e3:.1f} | {f_up / g_up / 1e9:.0f} |",
             f"| down | {ours_down * 1e3:.1f} | "
             f"{'-' if cfg.shared_experts else f'{f_down / ours_down / 1e9:.0f}'} | "
             f"{v_down * 1e3:.1f} | {f_down / v_down / 1e9:.0f} | "
             f"{g_down * 1e3:.1f} | {f_down / g_down / 1e9:.0f} |", ""]
    path = os.path.join(ROOT, "profiles", f"vendor_gemm_{cfg.name}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps({"workload": cfg.name, "ours_up_us": ours_up * 1e3,
                      "vendor_up_us": v_up * 1e3, "vendor_graph_up_us": g_up * 1e3,
                      "ours_down_us": ours_down * 1e3, "vendor_down_us": v_down * 1e3,
                      "vendor_graph_down_us": g_down * 1e3}))
    print(f"wrote {os.path.relpath(path, ROOT)}")
    return 0


def traffic_probe(torch, moe, cfg) -> int:
    """Kernels for the HBM-traffic counters: an elementwise negation that
    reads and writes COPY_BYTES (the calibration of FETCH_SIZE and
    WRITE_SIZE), then three layer calls of the workload."""
    import synth
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    inp = synth.make_layer_inputs(cfg, "cuda")
    spec = moe.spec_from_config(cfg)
    out = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    ws = moe.workspace(spec, cfg.T)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    for _ in range(3):
        moe.moe_layer_forward(spec, cfg.T, inp["x"], inp["w_router"], inp["expert_bias"],
                              inp, out, workspace=ws)
    torch.cuda.synchronize()
    print("traffic probe done", flush=True)
    return 0


FFN_KERNELS = ("grouped_gemm_kernel", "u4s_kernel")


def _counter_rows(d):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize_traffic(args) -> int:
    """profiles/ summary of HBM traffic per layer call of each expert kernel:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the ratio of
    the calibration kernel's known bytes to what the same counter read for
    it."""
    import synth
    cfg = synth.CONFIGS[args.config]
    kernels_of_interest = SIDE_KERNELS if args.side else FFN_KERNELS
    regex = SIDE_REGEX if args.side else TRAFFIC_REGEX
    res = {}
    for counter, d in (("FETCH_SIZE", args.summarize_traffic[0]),
                       ("WRITE_SIZE", args.summarize_traffic[1])):
        copy_kib, ffn = [], {}
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == counter]
        copies = [r for r in rows if "neg_kernel" in r["Kernel_Name"]]
        # the layer calls are the dispatches after the last calibration copy
        last_copy = max((int(r["Dispatch_Id"]) for r in copies), default=None)
        for r in copies:
            copy_kib.append(float(r["Counter_Value"]))
        for r in rows:
            if last_copy is None or int(r["Dispatch_Id"]) <= last_copy:
                continue
            name = r["Kernel_Name"]
            for k in kernels_of_interest:
                if k in name:
                    key = kernel_label(name)
                    ffn.setdefault(key, []).append(float(r["Counter_Value"]))
        if not copy_kib or not ffn:
            print(f"no calibration or kernel dispatches for {counter} in {d}",
                  file=sys.stderr)
            return 1
        factor = COPY_BYTES / (sum(copy_kib) / len(copy_kib) * 1024.0)
        # per layer call: every kernel's dispatches over the 3 calls
        per_kernel = {k: sum(vs) / 3 * 1024.0 * factor for k, vs in ffn.items()}
        res[counter] = {"factor": factor, "copy_kib": copy_kib, "per_kernel": per_kernel}
    path = traffic_summary_path(cfg.name, args.side)
    rel = os.path.relpath(path, ROOT)
    kernels = sorted(set(res["FETCH_SIZE"]["per_kernel"]) | set(res["WRITE_SIZE"]["per_kernel"]))
    with open(path, "w") as f:
        what = "router, dispatch and combine kernels" if args.side else "expert kernels"
        f.write(f"# HBM traffic of the {what} per layer call, {cfg.name}\n\n")
        f.write("Commands (repository root, one MI355X; the probe runs a 1 GiB elementwise "
                "negation for calibration, then three layer calls):\n\n```\n")
        f.write("export REPO=$PWD OUT=/tmp/moe_profiles TMPDIR=/tmp && mkdir -p $OUT && cd /tmp\n")
        for c, dd in (("FETCH_SIZE", "pmc_fetch"), ("WRITE_SIZE", "pmc_write")):
            f.write(f"timeout -s KILL 120 rocprofv3 --kernel-include-regex '{regex}' "
                    f"--pmc {c} --output-format csv -d $OUT/{dd} "
                    f"-o p -- python3 $REPO/bench.py --config {cfg.cfg_id} --traffic-probe\n")
        f.write(f"python3 $REPO/bench.py --config {cfg.cfg_id} --summarize-traffic "
                f"$OUT/pmc_fetch $OUT/pmc_write"
                f"{' --side' if args.side else ''}\n```\n\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            r = res[c]
            f.write(f"{c}: calibration read {sum(r['copy_kib']) / len(r['copy_kib']):.0f} KiB "
                    f"for {COPY_BYTES >> 10} KiB moved, factor {r['factor']:.4f}\n\n")
        f.write("| kernel | fetched bytes per call | written bytes per call |\n|---|---|---|\n")
        for k in kernels:
            f.write(f"| `{k}` | {res['FETCH_SIZE']['per_kernel'].get(k, 0.0):.4g} | "
                    f"{res['WRITE_SIZE']['per_kernel'].get(k, 0.0):.4g} |\n")
        f.write("\n")
        for k in kernels:
            tot = res["FETCH_SIZE"]["per_kernel"].get(k, 0.0) + \
                res["WRITE_SIZE"]["per_kernel"].get(k, 0.0)
            f.write(f"- per_call[{k}]: {tot:.6g}\n")
        f.write(f"- sources_sha256: "
                f"{side_sources_digest() if args.side else sources_digest(cfg.weight_dtype)}\n")
    total = sum(res["FETCH_SIZE"]["per_kernel"].values()) + \
        sum(res["WRITE_SIZE"]["per_kernel"].values())
    print(f"wrote {rel}: {total / 1e9:.3f} GB per layer call", flush=True)
    return 0


STATS_WORKLOADS = {
    2: "the Mixtral-shaped layer forward (T=4096, d=4096, E=8, top-2, SwiGLU F=14336, bf16)",
    3: "the DeepSeek-style layer forward (T=8192, d=7168, E=256 in 8 groups, top-4 groups, "
       "top-8, sigmoid router with selection bias, routed scaling 2.5, one shared expert, "
       "SwiGLU F=2048, bf16)",
    4: "the Qwen-style layer forward (T=16384, d=2048, E=128, top-8, Zipf-skewed router "
       "s=1.1, capacity factor 1.0, SwiGLU F=768, bf16)",
    5: "the decode layer forward with 4-bit experts (T=32, d=2048, E=256, top-8, SwiGLU "
       "F=512; timed steps rotate three input copies)",
}


def summarize_stats(args) -> int:
    """profiles/<workload>_layer_kernel_stats.md: the library's kernels from
    a rocprofv3 kernel_stats.csv (calls, average, min, max, share of all GPU
    time) and the bench.py line of the same run."""
    import synth
    cfg = synth.CONFIGS[args.config]
    d, log = args.summarize_stats
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if len(files) != 1:
        print(f"expected one kernel_stats.csv under {d}, found {len(files)}", file=sys.stderr)
        return 1
    with open(files[0]) as fh:
        rows = list(csv.DictReader(fh))
    labels = {r["Name"]: kernel_label(r["Name"]) for r in rows}
    ours = [r for r in rows if labels[r["Name"]].startswith("moe::")]
    others = [r for r in rows if not labels[r["Name"]].startswith("moe::")]
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    with open(log) as fh:
        lines = [ln for ln in fh if ln.startswith("{")]
    if not lines or not ours:
        print(f"no bench.py line in {log} or no library kernels in {files[0]}", file=sys.stderr)
        return 1
    res = json.loads(lines[-1])
    c = cfg.cfg_id
    out = [f"# Kernel time of {STATS_WORKLOADS.get(c, cfg.name)}", "",
           "Commands (repository root, one MI355X):", "", "```",
           f"export REPO=$PWD OUT=/tmp/moe_profiles TMPDIR=/tmp && mkdir -p $OUT && cd /tmp",
           f"rocprofv3 --kernel-trace --stats --output-format "
           f"csv -d $OUT/prof_c{c} -o bench -- python3 $REPO/bench.py --config {c} "
           f"--steps 20 --warmup 2 --no-cpu-baseline > $OUT/prof_c{c}.log",
           f"python3 $REPO/bench.py --config {c} --summarize-stats $OUT/prof_c{c} "
           f"$OUT/prof_c{c}.log",
           "```", "",
           "| kernel | calls | avg (us) | min (us) | max (us) | share of GPU time |",
           "|---|---|---|---|---|---|"]
    for r in sorted(ours, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"| `{labels[r['Name']]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{100 * float(r['TotalDurationNs']) / total:.2f}% |")
    out += ["", f"{len(others)} kernels of torch that draw the seeded synthetic inputs before "
            "the timed steps (random number generation, scaling, casts, copies) are omitted "
            "from the table (they are in the share's denominator)."]
    if "decode" in res and cfg.weight_dtype != "u4":
        out += ["", "The run includes bench.py's decode leg (the 4-bit decode layer, T=32): the "
                "`u4s_kernel_*`, `logits_rowdot_kernel`, `select_kernel<4, 0, false>` and "
                "`dispatch_small_kernel` calls and the `combine_kernel<float, float>` calls are "
                "that leg's."]
    rf = res["roofline"]
    s = (f"The same run's bench.py line: {res['ms_per_step']:.3f} ms per layer step, "
         f"{res['value']:.4g} tokens/s; roofline kernel ({rf['kernel']}) averaged "
         f"{rf['avg_launch_ms'] * 1e3:.1f} us per launch between HIP events recorded by the "
         f"layer on its stream, {rf['achieved']:.4g} {rf['unit']} = {100 * rf['frac']:.1f}% of "
         f"{rf['peak']:.4g} {rf['unit']}.")
    if "decode" in res:
        dd = res["decode"]
        s += (f" Decode leg: {dd.get('layer_us', float('nan')):.1f} us per layer, expert FFN "
              f"{dd.get('ffn_us', float('nan')):.1f} us.")
    out += ["", s]
    path = os.path.join(ROOT, "profiles", f"{cfg.name}_layer_kernel_stats.md")
    with open(path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    print(f"wrote {os.path.relpath(path, ROOT)}", flush=True)
    return 0


def summarize_mfma(args) -> int:
    """profiles/ summary of the bf16 expert GEMMs' matrix-core counters per
    layer call: MFMA busy cycles over the GPU's busy cycles and SIMDs (the
    definition of rocprofv3's MfmaUtil, with the XCDs' mean busy cycles),
    the MFMA operations counted (bf16 and fp16, 512 per unit), and the
    shader clock the busy-cycle count implies over the dispatch's
    duration."""
    import synth
    cfg = synth.CONFIGS[args.config]
    rows = _counter_rows(args.summarize_mfma)
    copies = [r for r in rows if "neg_kernel" in r["Kernel_Name"]]
    last_copy = max((int(r["Dispatch_Id"]) for r in copies), default=-1)
    per = {}  # kernel -> dispatch -> {counter: value, "ns": duration}
    for r in rows:
        if int(r["Dispatch_Id"]) <= last_copy or "grouped_gemm" not in r["Kernel_Name"]:
            continue
        key = kernel_label(r["Kernel_Name"])
        dd = per.setdefault(key, {}).setdefault(int(r["Dispatch_Id"]), {})
        dd[r["Counter_Name"]] = float(r["Counter_Value"])
        dd["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    if not per:
        print(f"no grouped-GEMM dispatches in {args.summarize_mfma}", file=sys.stderr)
        return 1
    path = os.path.join(ROOT, "profiles", f"expert_gemms_{cfg.name}_mfma_counters.md")
    with open(path, "w") as f:
        f.write(f"# Matrix-core counters of the bf16 expert GEMMs, {cfg.name}\n\n")
        f.write("Commands (repository root, one MI355X; three layer calls after a calibration "
                "copy):\n\n```\nexport REPO=$PWD OUT=/tmp/moe_profiles TMPDIR=/tmp && "
                "mkdir -p $OUT && cd /tmp\n")
        f.write(f"timeout -s KILL 120 rocprofv3 --kernel-trace --kernel-include-regex "
                f"'neg_kernel|grouped_gemm' --pmc {MFMA_COUNTERS} --output-format csv "
                f"-d $OUT/pmc_mfma -o p -- python3 $REPO/bench.py --config "
                f"{cfg.cfg_id} --traffic-probe\n")
        f.write(f"python3 $REPO/bench.py --config {cfg.cfg_id} --summarize-mfma "
                "$OUT/pmc_mfma\n```\n\n")
        f.write("MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); "
                "MFMA FLOPs = 512 x SQ_INSTS_VALU_MFMA_MOPS_*; the clock is GRBM_GUI_ACTIVE "
                "summed over the 8 XCDs, / 8, over the dispatch's duration (under counter "
                "collection).\n\n")
        f.write("| kernel | dispatches | µs per dispatch | MFMA busy | MFMA TFLOP per dispatch "
                "(bf16 / fp16) | TFLOP/s by counters | implied clock (GHz) |\n|---|---|---|---|---|---|---|\n")
        for k in sorted(per):
            ds = list(per[k].values())
            ns = sum(d["ns"] for d in ds) / len(ds)
            util = sum(100.0 * d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) /
                       max(1.0, d.get("GRBM_GUI_ACTIVE", 0.0) / 8 * SIMDS) for d in ds) / len(ds)
            fb = sum(d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for d in ds) / len(ds) * 512
            fh = sum(d.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) for d in ds) / len(ds) * 512
            gui = sum(d.get("GRBM_GUI_ACTIVE", 0.0) for d in ds) / len(ds)
            f.write(f"| `{k}` | {len(ds)} | {ns / 1e3:.1f} | {util:.1f}% | {fb / 1e12:.3f} / "
                    f"{fh / 1e12:.3f} | {(fb + fh) / ns / 1e3:.0f} | {gui / 8 / ns:.2f} |\n")
        f.write(f"\n- sources_sha256: {sources_digest('bf16')}\n")
    print(f"wrote {os.path.relpath(path, ROOT)}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
