"""Host logic of bench.py that needs no GPU: the committed counter summaries
under profiles/ are found by the kernel-name fragments the benchmark line
looks them up with, so a kernel renamed (a template parameter added, say)
cannot silently turn the roofline's `traffic` into null."""
import glob
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def per_call_keys(path):
    keys = []
    with open(path) as f:
        for line in f:
            if line.startswith("- per_call[") and "]: " in line:
                keys.append(line[len("- per_call["):].rsplit("]: ", 1)[0])
    return keys


def test_expert_traffic_summaries_hold_the_dominant_kernel():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "expert_gemms_*_hbm_traffic.md")))
    assert paths
    for p in paths:
        keys = per_call_keys(p)
        want = bench.U4_STREAM_KEY if "decode-u4" in os.path.basename(p) else bench.GATE_UP_KEY
        assert any(want in k for k in keys), (p, want, keys)


def test_headline_traffic_is_found_when_the_sources_match():
    """The lookup returns the summary's per-call bytes exactly when the
    digest recorded in it equals the digest of the current kernel source."""
    w = "mixtral-8x-top2-4096x14336"
    path = bench.traffic_summary_path(w)
    digest = None
    with open(path) as f:
        for line in f:
            if line.startswith("- sources_sha256: "):
                digest = line.split(": ", 1)[1].strip()
    got = bench.measured_traffic(w, bench.GATE_UP_KEY)
    if digest == bench.sources_digest("bf16"):
        total = sum(float(open(path).read().split(f"- per_call[{k}]: ")[1].split()[0])
                    for k in per_call_keys(path) if bench.GATE_UP_KEY in k)
        assert got == total and got > 0
    else:
        assert got is None


def test_kernel_stats_name_the_dominant_kernels():
    for p in glob.glob(os.path.join(ROOT, "profiles", "*_layer_kernel_stats.md")):
        text = open(p).read()
        assert bench.GATE_UP_KEY in text or bench.U4_STREAM_KEY in text, p


def test_kernel_labels_are_readable():
    """rocprofv3 leaves names holding _Float16 mangled; the summaries print
    them as template ids, like the names it demangles itself."""
    assert bench.kernel_label(
        "_ZN3moe12_GLOBAL__N_114combine_kernelIfDF16_EEvPKT0_S4_PKiPKfS8_PT_liii"
    ) == "moe::combine_kernel<float, _Float16>"
    assert bench.kernel_label(
        "void moe::(anonymous namespace)::grouped_gemm_kernel<0, true, false, 256>"
        "(moe::(anonymous namespace)::GemmArgs)") == "moe::grouped_gemm_kernel<0, true, false, 256>"
    for p in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        assert "_ZN3moe" not in open(p).read(), p
