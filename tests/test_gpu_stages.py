"""GPU parity of the whole path and of each C-ABI stage against the CPU
oracle, at sizes the oracle finishes in seconds that still span several
256-row M tiles, ragged N and M tails, drops, both routing kinds, both
activations, fp32 and bf16, and 4-bit weights; plus the degenerate cases.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_group_amd as moe
import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

C = synth.LayerConfig
MEDIUM = {
    # several M tiles per expert with a ragged tail; N tails in both GEMMs
    "swiglu-bf16-ragged": C("swiglu-bf16-ragged", 101, T=2000, d=576, E=4, top_k=2, F=704),
    # about 250 rows per expert in one ragged M tile: each of the tile's two
    # 128-row halves holds 0 to 4 non-empty 32-row blocks, so the K loop's
    # specialisations by block count all run, on both GEMMs
    "swiglu-bf16-partial-blocks": C("swiglu-bf16-partial-blocks", 139, T=1000, d=320, E=8,
                                    top_k=2, F=320),
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
    # the spec's limits: 1024 experts with k = 64 (bf16 and 4-bit weights),
    # and sigmoid-group routing over 64 groups
    "limits-e1024-k64": C("limits-e1024-k64", 140, T=33, d=64, E=1024, top_k=64, F=64),
    "limits-u4-e1024-k64": C("limits-u4-e1024-k64", 141, T=17, d=128, E=1024, top_k=64, F=128,
                             weight_dtype=synth.U4),
    # capacity max(1, int(3 * 2 / 8 * 1.0)) = 1: one kept row per expert
    "capacity-one": C("capacity-one", 143, T=3, d=64, E=8, top_k=2, F=64, capacity_factor=1.0),
    "limits-sigmoid-64-groups": C("limits-sigmoid-64-groups", 142, T=50, d=128, E=1024,
                                  top_k=16, F=64, router=synth.SIGMOID_GROUP,
                                  routed_scaling=2.5, n_group=64, topk_group=8,
                                  bias_range=0.05),
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
    # 4-bit weights on the weight-stream kernels with about 30 rows per
    # expert (8 four-row chunks each, weights streamed once per chunk; below
    # the 32 rows per expert from which the tiled kernels take over) and
    # the largest expert count (1024 experts, 64 of them touched at most)
    "u4-many-rows": C("u4-many-rows", 116, T=120, d=256, E=8, top_k=2, F=128,
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
    # 4-bit weights on the tiled matrix-core kernels (dequantised in the K
    # loop): F not a power of two with a bf16 shared expert; ReLU with
    # capacity drops (a shape only the tiled kernels take); a power-of-two
    # shape with hundreds of rows per expert
    "u4-tiled-swiglu-shared": C("u4-tiled-swiglu-shared", 132, T=1024, d=512, E=8, top_k=2,
                                F=384, weight_dtype=synth.U4, shared_experts=1, shared_F=256),
    "u4-tiled-relu-capacity": C("u4-tiled-relu-capacity", 133, T=600, d=256, E=8, top_k=2,
                                F=256, act=synth.RELU, weight_dtype=synth.U4,
                                capacity_factor=1.25),
    "u4-tiled-pow2": C("u4-tiled-pow2", 134, T=2048, d=1024, E=16, top_k=4, F=512,
                       weight_dtype=synth.U4),
    # 128-row 4-bit tiles (under 64 rows per expert): 50 rows per expert on
    # a power-of-two shape, and 8 rows per expert where the stream kernels
    # cannot take the shape (d = 384)
    "u4-tiled-128-rows": C("u4-tiled-128-rows", 137, T=400, d=512, E=32, top_k=4, F=256,
                           weight_dtype=synth.U4),
    "u4-tiled-few-rows": C("u4-tiled-few-rows", 138, T=64, d=384, E=16, top_k=2, F=256,
                           weight_dtype=synth.U4),
    # fp32 path, SwiGLU and a shared expert
    "f32-swiglu-shared": C("f32-swiglu-shared", 111, T=150, d=48, E=5, top_k=2, F=40,
                           act_dtype=synth.F32, weight_dtype=synth.F32, shared_experts=2,
                           shared_F=24, capacity_factor=1.5),
    # down projection long enough (F >= 1024) and with few enough tiles that
    # its reduction is split in two K halves, with capacity drops
    "swiglu-bf16-splitk": C("swiglu-bf16-splitk", 113, T=600, d=256, E=4, top_k=2,
                            F=1024, capacity_factor=1.25),
    # 128 x 128 vector-ALU logits tiles with ragged expert and token tails:
    # 37 experts with fp32 router weights and 100 experts with bf16 router
    # weights, one reduction split each
    "router-e37-fp32": C("router-e37-fp32", 114, T=400, d=192, E=37, top_k=3, F=64),
    "router-e100-bf16": C("router-e100-bf16", 115, T=300, d=128, E=100, top_k=5, F=64,
                          router_dtype=synth.BF16),
    # the reduction over d split in 4 partial planes, the last one shorter
    # (d = 1088: splits of 288, 288, 288, 224), fp32 and bf16 router weights,
    # two expert tiles
    "router-split-fp32": C("router-split-fp32", 123, T=300, d=1088, E=40, top_k=3, F=64),
    "router-split-bf16": C("router-split-bf16", 124, T=260, d=1024, E=150, top_k=4, F=64,
                           router_dtype=synth.BF16),
    # fp32 activations through the tiled logits kernel (two splits)
    "router-f32-tiled": C("router-f32-tiled", 125, T=200, d=512, E=64, top_k=2, F=32,
                          act_dtype=synth.F32, weight_dtype=synth.F32),
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
    -> moe_combine, called one by one, match the fused moe_layer_forward --
    routing and dispatch bit for bit, the output up to the layer keeping
    its expert rows in fp16 -- and each stage matches the oracle.  The
    second case splits the down projection's reduction: the stage API folds
    the halves into its expert rows, the fused layer adds them in the
    combine."""
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
    split = name.endswith("splitk")
    bound = gu.fp16_rows_bound(y, sr, tw, parts=2 if split else 1)
    # the split halves are partial sums, which may cancel far more than the
    # bound's headroom allows: their fp16 rounding is held to 0.2% of the
    # output RMS on top (the layer itself meets the oracle's bar elsewhere)
    rms = r["out"].float().pow(2).mean().sqrt().item()
    slack = 2e-3 * rms if split else 0.0
    excess = ((out - r["out"]).abs() - bound - 1e-6 * out.abs() - slack).max().item()
    gu.log(f"  stage vs layer: max excess over the fp16-row bound {excess:.3e} (RMS {rms:.3e})")
    assert excess <= 0, excess
    assert torch.equal(ids, r["topk_ids"]) and torch.equal(sr, r["slot_row"])
    r2 = dict(r)
    r2["out"] = out
    gu.full_check(cfg, inp, r2)
    n = int(offsets[-1].item())
    # permuted copy, sorted weights
    assert torch.equal(xp[:n], inp["x"][st[:n].long()])
    ids_h = ids.cpu().numpy()
    disp = gu.check_dispatch(cfg, ids_h, {"counts_pre": counts, "offsets": offsets,
                                          "dropped": dropped, "sorted_token": st,
                                          "slot_row": sr})
    assert torch.equal(sw[:n].cpu(), tw.reshape(-1)[torch.as_tensor(disp["sorted_slot"])].cpu())


@pytest.mark.parametrize("name", ["swiglu-bf16-splitk", "sigmoid-group-shared",
                                  "f32-swiglu-shared", "u4-decode", "u4-tiled-swiglu-shared"])
def test_routing_weights_applied_in_the_ffn(name):
    """moe_grouped_ffn with sorted_w writes each routed row times its routing
    weight (the down product's epilogue scales the fp32 accumulation; shared
    rows stay unweighted), and moe_combine with topk_w=NULL adds the rows
    unscaled: the same layer output up to rounding order, within the oracle's
    bar.  Covers the bf16 MFMA path (split and unsplit down product), the
    fp32 path, the 4-bit stream and the 4-bit tiled kernels."""
    import mixture_experts_layer_group_amd as moe
    cfg = MEDIUM[name]
    gu.log(f"[weighted rows] {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.top_k} F={cfg.F}")
    inp = gu.make_inputs(cfg)
    spec = moe.spec_from_config(cfg)
    T, k, E, d = cfg.T, cfg.top_k, cfg.E, cfg.d
    dev = "cuda"
    ws = moe.workspace(spec, T)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    moe.moe_route(spec, T, inp["x"], inp["w_router"], inp["expert_bias"], ids, tw,
                  None, None, ws)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    st = torch.empty(T * k, dtype=torch.int32, device=dev)
    sw = torch.empty(T * k, dtype=torch.float32, device=dev)
    sr = torch.empty((T, k), dtype=torch.int32, device=dev)
    dropped = torch.empty(1, dtype=torch.int32, device=dev)
    moe.moe_dispatch(spec, T, ids, tw, counts, offsets, st, sw, sr, dropped, None, None, ws)
    S = cfg.shared_experts
    y_u = torch.zeros((T * k, d), dtype=torch.float32, device=dev)
    y_w = torch.zeros((T * k, d), dtype=torch.float32, device=dev)
    ysh_u = torch.zeros((max(S, 1) * T, d), dtype=torch.float32, device=dev)
    ysh_w = torch.zeros((max(S, 1) * T, d), dtype=torch.float32, device=dev)
    moe.moe_grouped_ffn(spec, T, offsets, st, inp["x"], inp, y_u, ysh_u if S else None, ws)
    moe.moe_grouped_ffn(spec, T, offsets, st, inp["x"], inp, y_w, ysh_w if S else None, ws,
                        sorted_w=sw)
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    moe.moe_combine(spec, T, y_w, sr, None, ysh_w if S else None, out)
    torch.cuda.synchronize()
    n = int(offsets[-1].item())
    # the scaled rows: one fp32 rounding of the product (a few when the down
    # product's K halves are scaled before they are added)
    ref = y_u[:n] * sw[:n, None]
    err = (y_w[:n] - ref).abs().max().item()
    assert err <= 1e-6 * max(ref.abs().max().item(), 1e-30), err
    if S:
        assert torch.equal(ysh_w, ysh_u)
    r = gu.run_layer(cfg, inp)
    diff = (out - r["out"]).abs().max().item()
    rms = r["out"].float().pow(2).mean().sqrt().item()
    gu.log(f"  {n} rows; max|out - layer out| = {diff:.3e} (RMS {rms:.3e})")
    # the layer's matrix-core path keeps fp16 expert rows; the others fp32
    split = name.endswith("splitk")
    bound = gu.fp16_rows_bound(y_u, sr, tw, parts=2 if split else 1)
    excess = ((out - r["out"]).abs() - bound - (2e-3 if split else 1e-5) * rms).max().item()
    assert excess <= 0, excess
    r2 = dict(r)
    r2["out"] = out
    gu.full_check(cfg, inp, r2)


def test_grouped_ffn_skewed_loads_clamped_xcd_ranges():
    """One expert takes 2041 of 2048 rows (8 M tiles per N column), seven
    take one row each (one-row tiles).  The grouped GEMMs' XCD ranges, cut at
    equal estimated cost, would give the XCDs holding the one-row tiles more
    tiles than the 16 workgroups each XCD receives (120 gate/up tiles on a
    grid of 128): the boundaries are clamped, the down product's list is
    doubled by its K split, and the last quarters are claimed at run time.
    Every token of the stage API's output must still meet the oracle's bar,
    and every dispatched row must come back."""
    import mixture_experts_layer_group_amd as moe
    cfg = C("skew-one-expert", 144, T=2048, d=512, E=8, top_k=1, F=1024)
    T, k, E, d = cfg.T, cfg.top_k, cfg.E, cfg.d
    gu.log(f"[skewed loads] T={T} d={d} E={E} F={cfg.F}: 2041 rows on expert 0")
    inp = gu.make_inputs(cfg)
    spec = moe.spec_from_config(cfg)
    dev = "cuda"
    ws = moe.workspace(spec, T)
    ids = torch.zeros((T, k), dtype=torch.int32, device=dev)
    ids[T - 7:, 0] = torch.arange(1, 8, dtype=torch.int32, device=dev)
    g = torch.Generator(device="cpu").manual_seed(144)
    tw = (0.5 + torch.rand((T, k), generator=g)).to(dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    st = torch.empty(T * k, dtype=torch.int32, device=dev)
    sw = torch.empty(T * k, dtype=torch.float32, device=dev)
    sr = torch.empty((T, k), dtype=torch.int32, device=dev)
    dropped = torch.empty(1, dtype=torch.int32, device=dev)
    moe.moe_dispatch(spec, T, ids, tw, counts, offsets, st, sw, sr, dropped, None, None, ws)
    y = torch.full((T * k, d), float("nan"), dtype=torch.float32, device=dev)
    moe.moe_grouped_ffn(spec, T, offsets, st, inp["x"], inp, y, None, ws)
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    moe.moe_combine(spec, T, y, sr, tw, None, out)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [T - 7] + [1] * 7
    assert bool(torch.isfinite(y).all())  # every row written (no tile skipped)
    ids_h = ids.cpu().numpy()
    disp = gu.check_dispatch(cfg, ids_h, {"counts_pre": counts, "offsets": offsets,
                                          "dropped": dropped, "sorted_token": st,
                                          "slot_row": sr})
    gu.check_output(cfg, inp, {"out": out}, ids_h, tw.cpu().numpy().astype(np.float64), disp)


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


def _route_only(cfg, inp, errors=None):
    spec = moe.spec_from_config(cfg)
    T, k = cfg.T, cfg.top_k
    ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    tw = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    L = torch.zeros((T, cfg.E), dtype=torch.float32, device="cuda")
    moe.moe_route(spec, T, inp["x"], inp["w_router"], inp["expert_bias"], ids, tw, L,
                  workspace=moe.workspace(spec, T), errors=errors)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), tw.cpu().numpy().astype(np.float64), L.cpu().numpy()


@pytest.mark.parametrize("E,n_group,topk_group,k", [(256, 8, 4, 8), (32, 4, 2, 3)])
def test_sigmoid_group_exact_ties(E, n_group, topk_group, k):
    """Zero router weights and zero bias: every logit is 0, every sigmoid
    score 0.5, every group score 1.0.  Groups and experts tie everywhere, so
    the lower groups and then the lower experts win: ids 0..k-1 and weights
    0.5 / (k * 0.5 + 1e-20) * routed_scaling (0.3125 at k = 8, scaling 2.5)
    -- the oracle's closed-form pin, now on the GPU's group tie-break.  A
    bias that lifts one later group's experts moves the choice to that
    group's first k experts, with the same weights."""
    cfg = C("sigmoid-ties", 126, T=96, d=256, E=E, top_k=k, F=64,
            router=synth.SIGMOID_GROUP, routed_scaling=2.5, n_group=n_group,
            topk_group=topk_group, router_dtype=synth.BF16, bias_range=0.05)
    inp = gu.make_inputs(cfg)
    inp["w_router"].zero_()
    inp["expert_bias"].zero_()
    ids, w, L = _route_only(cfg, inp)
    assert np.all(L == 0.0)
    w_closed = 0.5 / (k * 0.5 + 1e-20) * 2.5
    assert np.all(ids == np.arange(k)[None, :])
    assert np.all(np.abs(w - w_closed) <= 1e-6)
    # the oracle on the same (zero) logits agrees bit for bit
    ids_o, w_o, _ = oracle.route_from_logits(L, gu.spec_dict(cfg),
                                             synth.host_array(inp["expert_bias"]))
    assert np.array_equal(ids, ids_o) and np.all(np.abs(w - w_o) <= 1e-6)
    # lift the experts of group g: the tie inside the group picks its first k
    G = E // n_group
    g = n_group - 2
    inp["expert_bias"][g * G:(g + 1) * G] = 0.125
    ids, w, L = _route_only(cfg, inp)
    assert np.all(ids == g * G + np.arange(k)[None, :])
    assert np.all(np.abs(w - w_closed) <= 1e-6)  # raw sigmoid: the bias is not a weight
    ids_o, _, _ = oracle.route_from_logits(L, gu.spec_dict(cfg),
                                           synth.host_array(inp["expert_bias"]))
    assert np.array_equal(ids, ids_o)
    gu.log(f"  exact ties: ids 0..{k - 1}, w {w_closed}; lifted group {g}: ids "
           f"{g * G}..{g * G + k - 1}")


def test_error_word_bad_ids_and_clean_runs():
    """moe_dispatch flags expert ids outside [0,E) (MOE_FLAG_BAD_EXPERT_ID)
    and drops those slots; every other slot is dispatched as the oracle
    dispatches the valid ids.  Clean calls leave the word at 0."""
    cfg = C("bad-ids", 127, T=700, d=128, E=16, top_k=2, F=64, capacity_factor=1.5)
    spec = moe.spec_from_config(cfg)
    T, k, E = cfg.T, cfg.top_k, cfg.E
    rs = np.random.default_rng(5)
    ids_h = np.stack([rs.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    dev = "cuda"
    for T_run in (T, 40):  # the multi-block and the one-block dispatch
        ids_t = torch.from_numpy(ids_h[:T_run].copy()).to(dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        out = {n: torch.full(shape, -7, dtype=dt, device=dev) for n, shape, dt in (
            ("counts", (E,), torch.int32), ("offsets", (E + 1,), torch.int32),
            ("st", (T_run * k,), torch.int32), ("sw", (T_run * k,), torch.float32),
            ("sr", (T_run, k), torch.int32), ("dropped", (1,), torch.int32))}
        tw = torch.ones((T_run, k), dtype=torch.float32, device=dev)
        ws = moe.workspace(spec, T_run)

        def run(ids_dev):
            moe.moe_dispatch(spec, T_run, ids_dev, tw, out["counts"], out["offsets"],
                             out["st"], out["sw"], out["sr"], out["dropped"], workspace=ws,
                             errors=err)
            torch.cuda.synchronize()

        run(ids_t)
        assert int(err.item()) == 0, "a clean dispatch sets no flag"
        bad = ids_h[:T_run].copy()
        bad[3, 1] = E
        bad[T_run - 1, 0] = -1
        bad[T_run // 2, 1] = 1 << 20
        run(torch.from_numpy(bad).to(dev))
        assert int(err.item()) & moe.FLAG_BAD_EXPERT_ID
        sr = out["sr"].cpu().numpy()
        assert sr[3, 1] == -1 and sr[T_run - 1, 0] == -1 and sr[T_run // 2, 1] == -1
        valid = (bad >= 0) & (bad < E)
        counts = np.bincount(bad[valid], minlength=E)
        assert np.array_equal(out["counts"].cpu().numpy(), counts)
        cap = oracle.capacity_for(T_run, k, E, cfg.capacity_factor)
        # the oracle's queue rule restricted to the valid slots
        kept = np.zeros(E, dtype=np.int64)
        rows = {}
        for t in range(T_run):
            for i in range(k):
                e = int(bad[t, i])
                if 0 <= e < E and kept[e] < cap:
                    rows[(t, i)] = (e, int(kept[e]))
                    kept[e] += 1
        offs = np.concatenate([[0], np.cumsum(kept)])
        assert np.array_equal(out["offsets"].cpu().numpy(), offs)
        assert int(out["dropped"].item()) == T_run * k - int(offs[-1])
        for (t, i), (e, rank) in rows.items():
            assert sr[t, i] == offs[e] + rank
        gu.log(f"  T={T_run}: 3 bad ids flagged and dropped, {int(offs[-1])} slots kept")


def test_error_word_saturation_and_nonfinite():
    """A hidden activation beyond the fp16 range sets MOE_FLAG_H_SATURATED
    (bf16 and 4-bit paths) and is stored as +-65504; a NaN token row sets
    MOE_FLAG_NONFINITE_LOGIT.  The normal inputs set neither."""
    for cfg in (C("sat-bf16", 128, T=300, d=256, E=8, top_k=2, F=128),
                C("sat-u4", 129, T=24, d=256, E=16, top_k=2, F=128,
                  weight_dtype=synth.U4),
                C("sat-u4-tiled", 136, T=600, d=256, E=8, top_k=2, F=256,
                  weight_dtype=synth.U4)):
        inp = gu.make_inputs(cfg)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        spec = moe.spec_from_config(cfg)
        out = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
        ws = moe.workspace(spec, cfg.T)
        moe.moe_layer_forward(spec, cfg.T, inp["x"], inp["w_router"], None, inp, out,
                              stats=moe.layer_stats(errors=err), workspace=ws)
        torch.cuda.synchronize()
        assert int(err.item()) == 0, f"{cfg.name}: normal inputs set {int(err.item())}"
        # tokens 300x larger: gate and up ~ N(0, 300^2), so silu(g)*u passes
        # 65504 for some hidden units
        x_big = (inp["x"].float() * 300.0).to(torch.bfloat16)
        moe.moe_layer_forward(spec, cfg.T, x_big, inp["w_router"], None, inp, out,
                              stats=moe.layer_stats(errors=err), workspace=ws)
        torch.cuda.synchronize()
        # the clamped hidden rows may carry fp16 expert rows past the range
        # too (matrix-core kernels)
        allowed = moe.FLAG_H_SATURATED | (0 if cfg.name == "sat-u4" else moe.FLAG_Y_SATURATED)
        got = int(err.item())
        assert got & moe.FLAG_H_SATURATED and got & ~allowed == 0, f"{cfg.name}: {got}"
        gu.log(f"  {cfg.name}: saturation flagged")
        if cfg.name == "sat-u4-tiled":
            # an activation beyond fp16's range: the tiled 4-bit products read
            # an fp16 copy of x
            x_wide = inp["x"].clone()
            x_wide[5, 3] = 1.0e5
            err.zero_()
            moe.moe_layer_forward(spec, cfg.T, x_wide, inp["w_router"], None, inp, out,
                                  stats=moe.layer_stats(errors=err), workspace=ws)
            torch.cuda.synchronize()
            assert int(err.item()) & moe.FLAG_X_SATURATED, f"{int(err.item())}"
    # a NaN token: its logits are NaN; the other tokens route as before
    cfg = C("nonfinite", 130, T=200, d=256, E=40, top_k=2, F=64)
    inp = gu.make_inputs(cfg)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids0, w0, _ = _route_only(cfg, inp, errors=err)
    assert int(err.item()) == 0
    inp["x"][17] = float("nan")
    ids1, w1, _ = _route_only(cfg, inp, errors=err)
    assert int(err.item()) == moe.FLAG_NONFINITE_LOGIT
    keep = np.ones(cfg.T, dtype=bool)
    keep[17] = False
    assert np.array_equal(ids0[keep], ids1[keep]) and np.array_equal(w0[keep], w1[keep])


def test_error_word_expert_rows_beyond_fp16():
    """Inside moe_layer_forward the matrix-core kernels keep the expert rows
    in fp16: down weights scaled by 2^16 (exact in bf16) push expert outputs
    past 65504 with every hidden activation in range, which sets
    MOE_FLAG_Y_SATURATED alone; the stage API's fp32 rows set nothing."""
    import mixture_experts_layer_group_amd as moe
    cfg = C("sat-y", 144, T=300, d=256, E=8, top_k=2, F=128)
    inp = gu.make_inputs(cfg)
    inp["w_down"] = (inp["w_down"].float() * 65536.0).to(torch.bfloat16)
    spec = moe.spec_from_config(cfg)
    out = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    ws = moe.workspace(spec, cfg.T)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda")
    st = torch.empty(cfg.T * cfg.top_k, dtype=torch.int32, device="cuda")
    moe.moe_layer_forward(spec, cfg.T, inp["x"], inp["w_router"], None, inp, out,
                          stats=moe.layer_stats(errors=err, offsets=offsets, sorted_token=st),
                          workspace=ws)
    torch.cuda.synchronize()
    assert int(err.item()) == moe.FLAG_Y_SATURATED, int(err.item())
    err.zero_()
    y = torch.zeros((cfg.T * cfg.top_k, cfg.d), dtype=torch.float32, device="cuda")
    moe.moe_grouped_ffn(spec, cfg.T, offsets, st, inp["x"], inp, y, None, ws, errors=err)
    torch.cuda.synchronize()
    n = int(offsets[-1].item())
    assert int(err.item()) == 0
    assert y[:n].abs().max().item() > 65504.0
    gu.log("  expert rows past fp16: flagged in the layer, exact in the stage API")


def test_routing_health_counts_beyond_fp32_integers():
    """Pre-drop counts above 2^24 (not all representable in fp32): the
    totals and the bias sign rule are exact.  E = 4, counts 2^24 + (1, 1,
    3, -1): total 2^26 + 4, mean 2^24 + 1, so experts 0 and 1 stay, 2 moves
    down and 3 up.  In fp32 the counts would read 2^24 + (0, 0, 4, -1) and
    the total could not be 2^26 + 4, which moves experts 0 and 1."""
    cfg = C("big-counts", 131, T=(1 << 24) + 1, d=64, E=4, top_k=4, F=64,
            act_dtype=synth.F32, weight_dtype=synth.F32)
    spec = moe.spec_from_config(cfg)
    base = 1 << 24
    counts_h = np.array([base + 1, base + 1, base + 3, base - 1], dtype=np.int32)
    dev = "cuda"
    counts = torch.from_numpy(counts_h).to(dev)
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts_h)]).astype(np.int32)).to(dev)
    dropped = torch.zeros(1, dtype=torch.int32, device=dev)
    bias = torch.zeros(4, dtype=torch.float32, device=dev)
    h = moe.health_buffer()
    moe.moe_routing_health(spec, cfg.T, counts, offsets, dropped, None, h, bias=bias,
                           bias_step=0.5)
    torch.cuda.synchronize()
    got = moe.health_from_bytes(h)
    assert got["kept_total"] == 4 * base + 4
    assert bias.cpu().tolist() == [0.0, 0.0, -0.5, 0.5]
    ref = oracle.bias_update(np.zeros(4), counts_h.astype(np.int64), 0.5)
    assert np.array_equal(bias.cpu().numpy().astype(np.float64), ref)
    st = oracle.layer_stats(counts_h, counts_h, 0, None, cfg.T, 4, 4)
    assert abs(got["load_peak_over_mean"] - st["load_peak_over_mean"]) <= 1e-6


U4_LARGE = {
    # the DeepSeek-style expert shape in 4 bits (d = 7168, F = 2048) with
    # about 256 rows per expert
    "u4-deepseek-shape": C("u4-deepseek-shape", 135, T=2048, d=7168, E=16, top_k=2, F=2048,
                           weight_dtype=synth.U4),
    # a prefill batch over the decode-shaped layer's experts (4096 tokens,
    # 256 experts, top-8: 128 rows per expert)
    "u4-decode-experts-prefill": synth.CONFIGS[5].replace(name="u4-decode-experts-prefill",
                                                          T=4096),
}


@pytest.mark.parametrize("name", list(U4_LARGE))
def test_u4_tiled_large(name):
    """The tiled 4-bit kernels at full-size expert shapes: routing and
    dispatch in full, the output on 256 tokens (every expert's last M tile
    first)."""
    cfg = U4_LARGE[name]
    gu.log(f"[u4 tiled] {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.top_k} F={cfg.F}")
    inp = gu.make_inputs(cfg)
    r = gu.run_layer(cfg, inp)

    def choose(disp):
        toks = set(gu.last_tile_tokens(disp, 1))
        for t in np.random.default_rng(cfg.cfg_id).permutation(cfg.T):
            if len(toks) >= 256:
                break
            toks.add(int(t))
        return sorted(toks)

    gu.full_check(cfg, inp, r, choose_tokens=choose)
