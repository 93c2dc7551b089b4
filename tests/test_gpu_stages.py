"""GPU parity of the whole path and of each C-ABI stage against the CPU
oracle, at sizes the oracle finishes in seconds that still span several
256-row M tiles, ragged N and M tails, drops, both routing kinds, both
activations, fp32 and bf16, and 4-bit weights; plus the degenerate cases.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

C = synth.LayerConfig
MEDIUM = {
    # several M tiles per expert with a ragged tail; N tails in both GEMMs
    "swiglu-bf16-ragged": C("swiglu-bf16-ragged", 101, T=2000, d=576, E=4, top_k=2, F=704),
    # Zipf-skewed popularity with capacity: heavy drops
    "swiglu-bf16-zipf-capacity": C("swiglu-bf16-zipf-capacity", 102, T=1500, d=512, E=8,
                                   top_k=2, F=512, capacity_factor=1.0, zipf_s=1.1),
    # sigmoid group routing, selection bias, routed scaling, a shared expert
    "sigmoid-group-shared": C("sigmoid-group-shared", 103, T=700, d=512, E=32, top_k=4,
                              F=256, router=synth.SIGMOID_GROUP, routed_scaling=2.5,
                              n_group=4, topk_group=2, shared_experts=1, shared_F=384,
                              router_dtype=synth.BF16, bias_range=0.05),
    # ReLU experts in bf16 with capacity
    "relu-bf16-capacity": C("relu-bf16-capacity", 104, T=900, d=256, E=6, top_k=3, F=320,
                            capacity_factor=1.25, act=synth.RELU),
    # top-1 (Switch) with many small experts
    "top1": C("top1", 105, T=333, d=128, E=16, top_k=1, F=128),
    # k = E: every expert on every token
    "k-equals-E": C("k-equals-E", 106, T=100, d=64, E=4, top_k=4, F=64),
    # softmax without renormalisation
    "no-norm": C("no-norm", 107, T=257, d=192, E=8, top_k=2, F=192, norm_topk_prob=False),
    # sigmoid group with every group kept and norm off
    "sigmoid-all-groups-no-norm": C("sigmoid-all-groups-no-norm", 108, T=300, d=256, E=16,
                                    top_k=3, F=128, router=synth.SIGMOID_GROUP,
                                    routed_scaling=1.5, n_group=4, topk_group=4,
                                    norm_topk_prob=False, bias_range=0.05),
    # 4-bit affine weights, decode-shaped; K % 128 == 0 and == 64 variants
    "u4-decode": C("u4-decode", 109, T=20, d=512, E=64, top_k=4, F=256, weight_dtype=synth.U4),
    "u4-small-k": C("u4-small-k", 110, T=37, d=256, E=16, top_k=2, F=64, weight_dtype=synth.U4),
    # 4-bit weights with 64 rows per expert (16 four-row chunks each, weights
    # streamed once per chunk) and the largest expert count (1024 experts,
    # 64 of them touched at most)
    "u4-many-rows": C("u4-many-rows", 116, T=256, d=256, E=8, top_k=2, F=128,
                      weight_dtype=synth.U4),
    "u4-1024-experts": C("u4-1024-experts", 117, T=8, d=64, E=1024, top_k=8, F=64,
                         weight_dtype=synth.U4),
    # the other reduction lengths of the 4-bit kernels: gate/up over
    # K = 1024 and 128, down over K = 2048 and 1024 (1, 2, 8 and 16 K slices
    # per unit group)
    "u4-k1024-f2048": C("u4-k1024-f2048", 118, T=24, d=1024, E=8, top_k=2, F=2048,
                        weight_dtype=synth.U4),
    "u4-k128-f1024": C("u4-k128-f1024", 119, T=40, d=128, E=16, top_k=3, F=1024,
                       weight_dtype=synth.U4),
    # fp32 path, SwiGLU and a shared expert
    "f32-swiglu-shared": C("f32-swiglu-shared", 111, T=150, d=48, E=5, top_k=2, F=40,
                           act_dtype=synth.F32, weight_dtype=synth.F32, shared_experts=2,
                           shared_F=24, capacity_factor=1.5),
    # down projection long enough (F >= 1024) and with few enough tiles that
    # its reduction is split in two K halves, with capacity drops
    "swiglu-bf16-splitk": C("swiglu-bf16-splitk", 113, T=600, d=256, E=4, top_k=2,
                            F=1024, capacity_factor=1.25),
    # router tile widths of the matrix-core logits: 37 experts with fp32
    # router weights (three bf16 parts, 64-wide tile, ragged expert tail) and
    # 100 experts with bf16 router weights (128-wide tile)
    "router-e37-fp32": C("router-e37-fp32", 114, T=400, d=192, E=37, top_k=3, F=64),
    "router-e100-bf16": C("router-e100-bf16", 115, T=300, d=128, E=100, top_k=5, F=64,
                          router_dtype=synth.BF16),
    # bf16 shared expert with ReLU and many tokens (several M tiles)
    "relu-shared-tiles": C("relu-shared-tiles", 112, T=1100, d=256, E=8, top_k=2, F=256,
                           act=synth.RELU, shared_experts=1, shared_F=320),
    # bf16 layer output
    "bf16-output": C("bf16-output", 113, T=800, d=320, E=8, top_k=2, F=448,
                     out_dtype=synth.BF16, capacity_factor=1.25),
}


@pytest.mark.parametrize("name", list(MEDIUM))
def test_layer_parity_medium(name):
    cfg = MEDIUM[name]
    gu.log(f"[layer parity] {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.top_k} F={cfg.F}")
    inp = gu.make_inputs(cfg)
    r = gu.run_layer(cfg, inp)
    ids_g, disp = gu.full_check(cfg, inp, r)
    gu.check_end_to_end_routing(cfg, inp, ids_g, r["logits"].cpu().numpy())


@pytest.mark.parametrize("base", range(1234, 1242))
def test_tiny_fp32_config_seeds(base):
    """The tiny fp32 ReLU layer (capacity 20) over seeds 1234..1241."""
    cfg = synth.CONFIGS[1]
    gu.log(f"[tiny fp32] seed base {base}")
    inp = gu.make_inputs(cfg, base=base)
    r = gu.run_layer(cfg, inp)
    gu.full_check(cfg, inp, r)


def test_zero_router_drops_are_exact_zero():
    """Wr = 0: every token picks experts 0..k-1 (lower-index ties); with
    capacity c the tokens t >= c lose both slots and give exactly 0."""
    cfg = C("zero-router", 120, T=300, d=128, E=8, top_k=2, F=128, capacity_factor=1.0)
    inp = gu.make_inputs(cfg)
    inp["w_router"].zero_()
    r = gu.run_layer(cfg, inp)
    ids = r["topk_ids"].cpu().numpy()
    assert np.all(ids == np.array([0, 1]))
    ids_g, disp = gu.full_check(cfg, inp, r)
    out = r["out"].float().cpu().numpy()
    assert np.all(out[75:] == 0.0) and np.all(np.any(out[:75] != 0.0, axis=1))


def test_single_token_and_empty_batch():
    cfg = C("one-token", 121, T=1, d=256, E=8, top_k=2, F=128)
    inp = gu.make_inputs(cfg)
    r = gu.run_layer(cfg, inp)
    gu.full_check(cfg, inp, r)
    # T = 0 is a no-op that touches nothing
    import mixture_experts_layer_group_amd as moe
    spec = moe.spec_from_config(cfg)
    out = torch.full((1, cfg.d), 7.0, dtype=torch.float32, device="cuda")
    moe.moe_layer_forward(spec, 0, inp["x"], inp["w_router"], None, inp, out,
                          workspace=torch.empty(1, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


@pytest.mark.parametrize("name", ["sigmoid-group-shared", "swiglu-bf16-splitk"])
def test_stagewise_api_matches_layer(name):
    """moe_route -> moe_dispatch (with the permuted copy) -> moe_grouped_ffn
    -> moe_combine, called one by one, equal the fused moe_layer_forward
    bit for bit, and each stage matches the oracle.  The second case splits
    the down projection's reduction: the stage API folds the halves into
    its expert rows, the fused layer adds them in the combine."""
    import mixture_experts_layer_group_amd as moe
    cfg = MEDIUM[name]
    inp = gu.make_inputs(cfg)
    spec = moe.spec_from_config(cfg)
    T, k, E, d = cfg.T, cfg.top_k, cfg.E, cfg.d
    dev = "cuda"
    ws = moe.workspace(spec, T)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    moe.moe_route(spec, T, inp["x"], inp["w_router"], inp["expert_bias"], ids, tw,
                  logits, None, ws)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    st = torch.empty(T * k, dtype=torch.int32, device=dev)
    sw = torch.empty(T * k, dtype=torch.float32, device=dev)
    sr = torch.empty((T, k), dtype=torch.int32, device=dev)
    dropped = torch.empty(1, dtype=torch.int32, device=dev)
    xp = torch.zeros((T * k, d), dtype=torch.bfloat16, device=dev)
    moe.moe_dispatch(spec, T, ids, tw, counts, offsets, st, sw, sr, dropped,
                     inp["x"], xp, ws)
    y = torch.zeros((T * k, d), dtype=torch.float32, device=dev)
    ysh = torch.zeros((T, d), dtype=torch.float32, device=dev)
    moe.moe_grouped_ffn(spec, T, offsets, st, inp["x"], inp, y, ysh, ws)
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    moe.moe_combine(spec, T, y, sr, tw, ysh, out)
    torch.cuda.synchronize()
    r = gu.run_layer(cfg, inp)
    assert torch.equal(out, r["out"])
    assert torch.equal(ids, r["topk_ids"]) and torch.equal(sr, r["slot_row"])
    n = int(offsets[-1].item())
    # permuted copy, sorted weights
    assert torch.equal(xp[:n], inp["x"][st[:n].long()])
    ids_h = ids.cpu().numpy()
    disp = gu.check_dispatch(cfg, ids_h, {"counts_pre": counts, "offsets": offsets,
                                          "dropped": dropped, "sorted_token": st,
                                          "slot_row": sr})
    assert torch.equal(sw[:n].cpu(), tw.reshape(-1)[torch.as_tensor(disp["sorted_slot"])].cpu())


def test_determinism_bitwise():
    cfg = MEDIUM["swiglu-bf16-zipf-capacity"]
    inp = gu.make_inputs(cfg)
    a = gu.run_layer(cfg, inp)
    b = gu.run_layer(cfg, inp)
    for key in ("out", "topk_ids", "topk_w", "slot_row", "prob_sum"):
        assert torch.equal(a[key], b[key]), key


def _health_case(cfg, inp, step):
    import mixture_experts_layer_group_amd as moe
    r = gu.run_layer(cfg, inp)
    spec = moe.spec_from_config(cfg)
    T, k, E = cfg.T, cfg.top_k, cfg.E
    h = moe.health_buffer()
    bias0 = torch.linspace(-0.1, 0.1, E, dtype=torch.float32, device="cuda")
    bias = bias0.clone()
    moe.moe_routing_health(spec, T, r["counts_pre"], r["offsets"], r["dropped"],
                           r["prob_sum"], h, bias, step)
    torch.cuda.synchronize()
    got = moe.health_from_bytes(h)
    counts = r["counts_pre"].cpu().numpy().astype(np.int64)
    off = r["offsets"].cpu().numpy().astype(np.int64)
    kept = np.diff(off)
    dropped = int(r["dropped"].item())
    P = (r["prob_sum"].cpu().numpy().astype(np.float64) / T
         if r["prob_sum"] is not None else None)
    ref = oracle.layer_stats(counts, kept, dropped, P, T, k, E)
    gu.log(f"  health: {got}")
    assert got["kept_total"] == int(kept.sum())
    for key in ("entropy", "max_entropy", "entropy_ratio", "max_share",
                "dropped_fraction", "load_peak_over_mean"):
        assert abs(got[key] - ref[key]) <= 2e-6 * max(1.0, abs(ref[key])), key
    if P is not None:
        for key in ("aux", "aux3"):
            assert abs(got[key] - ref[key]) <= 2e-6 * max(1.0, abs(ref[key])), key
    else:
        assert got["aux"] == 0.0 and got["aux3"] == 0.0
    if abs(ref["entropy_ratio"] - 0.5) > 1e-5:
        assert got["collapsed"] == int(ref["collapsed"])
    ref_b = oracle.bias_update(bias0.cpu().numpy(), counts, step)
    got_b = bias.cpu().numpy().astype(np.float64)
    # one fp32 addition of +-step or 0
    assert np.all(np.abs(got_b - ref_b) <= 1e-7 + 2.0 ** -24 * np.abs(ref_b))
    return got, ref


@pytest.mark.parametrize("name", ["swiglu-bf16-zipf-capacity", "sigmoid-group-shared",
                                  "relu-bf16-capacity"])
def test_routing_health_and_bias_update(name):
    """moe_routing_health on a layer's own dispatch counts equals the
    oracle's health fields (fp32 against fp64) and its bias update."""
    cfg = MEDIUM[name]
    _health_case(cfg, gu.make_inputs(cfg), 1e-3)


def test_routing_health_collapsed_and_equal_loads():
    """Zero router: every token picks experts 0 and 1, so the kept shares
    are two equal halves (entropy log 2, ratio 1/3, collapsed); the other
    six experts are below the mean load and move up, the two busy ones down."""
    cfg = C("zero-router-health", 122, T=256, d=128, E=8, top_k=2, F=128)
    inp = gu.make_inputs(cfg)
    inp["w_router"].zero_()
    got, ref = _health_case(cfg, inp, 0.25)
    assert got["collapsed"] == 1 and abs(got["max_share"] - 0.5) < 1e-7
    assert abs(got["entropy_ratio"] - 1.0 / 3.0) < 1e-6
