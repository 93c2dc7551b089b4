"""GPU parity of router replay (moe_route_forced) against the oracle's
route_forced, on the GPU's own logits: ids bit-exact, weights within 1e-6,
the rejected-row count exact; forcing the router's own choice reproduces
moe_route bit for bit; and a replayed route carried through dispatch, the
grouped FFN and the combine matches the oracle's layer on the same ids.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_group_amd as moe
import oracle
import synth
from tests import gpu_util as gu
from tests.test_gpu_stages import MEDIUM

pytestmark = pytest.mark.gpu

CASES = ["swiglu-bf16-zipf-capacity", "sigmoid-group-shared", "router-e100-bf16",
         "no-norm", "sigmoid-all-groups-no-norm", "top1", "k-equals-E",
         "f32-swiglu-shared"]


def forced_rows(T, E, k, seed):
    """k distinct experts per token drawn uniformly, with a few invalid
    rows planted: all -1 (an unrecorded route), a repeat, E, INT32_MIN and
    E + 100 (in the last row).  Returns (ids [T,k] int32, planted rows)."""
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    bad = {}
    if T > 3:
        bad[3] = np.full(k, -1, dtype=np.int32)
    if T > 10 and k >= 2:
        row = ids[10].copy()
        row[k - 1] = row[0]
        bad[10] = row
    if T > 17:
        row = ids[17].copy()
        row[k // 2] = E
        bad[17] = row
    if T > 25:
        row = ids[25].copy()
        row[0] = np.iinfo(np.int32).min
        bad[25] = row
    if T > 1:
        row = ids[T - 1].copy()
        row[k - 1] = E + 100
        bad[T - 1] = row
    for t, row in bad.items():
        ids[t] = row
    return ids, sorted(bad)


def route_both(cfg, inp, forced_h):
    spec = moe.spec_from_config(cfg)
    T, k, E = cfg.T, cfg.top_k, cfg.E
    dev = "cuda"
    ws = moe.workspace(spec, T)
    want_p = cfg.router == synth.SOFTMAX_TOPK
    a = {"ids": torch.full((T, k), -7, dtype=torch.int32, device=dev),
         "w": torch.full((T, k), float("nan"), dtype=torch.float32, device=dev),
         "logits": torch.zeros((T, E), dtype=torch.float32, device=dev),
         "prob": torch.zeros(E, dtype=torch.float32, device=dev) if want_p else None}
    moe.moe_route(spec, T, inp["x"], inp["w_router"], inp["expert_bias"], a["ids"],
                  a["w"], a["logits"], a["prob"], ws)
    forced = a["ids"].clone() if forced_h is None else torch.as_tensor(forced_h).to(dev)
    b = {"ids": torch.full((T, k), -7, dtype=torch.int32, device=dev),
         "w": torch.full((T, k), float("nan"), dtype=torch.float32, device=dev),
         "logits": torch.zeros((T, E), dtype=torch.float32, device=dev),
         "prob": torch.zeros(E, dtype=torch.float32, device=dev) if want_p else None,
         "rejected": torch.full((1,), 12345, dtype=torch.int32, device=dev)}
    moe.moe_route_forced(spec, T, inp["x"], inp["w_router"], forced, b["ids"], b["w"],
                         b["rejected"], b["logits"], b["prob"], ws)
    torch.cuda.synchronize()
    return a, b, forced


@pytest.mark.parametrize("name", CASES)
def test_forcing_own_ids_reproduces_route(name):
    """Replaying the ids moe_route chose gives its weights, logits and
    probability sums bit for bit, and rejects nothing."""
    cfg = MEDIUM[name]
    gu.log(f"[replay own ids] {name}: T={cfg.T} E={cfg.E} k={cfg.top_k}")
    inp = gu.make_inputs(cfg)
    a, b, _ = route_both(cfg, inp, None)
    assert int(b["rejected"].item()) == 0
    assert torch.equal(a["ids"], b["ids"])
    assert torch.equal(a["logits"], b["logits"])
    # the same arithmetic on the same values (a selection bias only steers
    # the choice, never the weights)
    assert torch.equal(a["w"], b["w"])
    if a["prob"] is not None:
        assert torch.equal(a["prob"], b["prob"])


@pytest.mark.parametrize("name", CASES)
def test_forced_ids_match_oracle(name):
    cfg = MEDIUM[name]
    T, k, E = cfg.T, cfg.top_k, cfg.E
    forced_h, planted = forced_rows(T, E, k, seed=9000 + cfg.cfg_id)
    gu.log(f"[replay forced] {name}: T={T} E={E} k={k}, planted rows {planted}")
    inp = gu.make_inputs(cfg)
    a, b, _ = route_both(cfg, inp, forced_h)
    # the logits and probability sums do not depend on the ids
    assert torch.equal(a["logits"], b["logits"])
    if a["prob"] is not None:
        assert torch.equal(a["prob"], b["prob"])
    L = b["logits"].cpu().numpy()
    ids_o, w_o, rej_o = oracle.route_forced(L, forced_h, gu.spec_dict(cfg))
    assert set(np.flatnonzero(rej_o).tolist()) == set(planted)
    assert int(b["rejected"].item()) == int(rej_o.sum())
    ids_g = b["ids"].cpu().numpy()
    w_g = b["w"].cpu().numpy().astype(np.float64)
    assert np.array_equal(ids_g, ids_o)
    err = np.abs(w_g - w_o)
    gu.log(f"  weights max|err| {err.max():.2e}, rejected {int(rej_o.sum())}")
    assert np.all(err <= 1e-6)
    assert np.all(w_g[rej_o] == 0.0)


@pytest.mark.parametrize("name", ["swiglu-bf16-zipf-capacity", "sigmoid-group-shared"])
def test_replayed_route_through_the_layer(name):
    """moe_route_forced -> moe_dispatch -> moe_grouped_ffn -> moe_combine on
    planted and random ids equals the oracle's dispatch and layer output for
    the replayed ids and weights; a rejected token adds nothing beyond its
    shared experts."""
    cfg = MEDIUM[name]
    T, k, E, d = cfg.T, cfg.top_k, cfg.E, cfg.d
    forced_h, planted = forced_rows(T, E, k, seed=9100 + cfg.cfg_id)
    gu.log(f"[replay layer] {name}: T={T} E={E} k={k}, planted rows {planted}")
    inp = gu.make_inputs(cfg)
    spec = moe.spec_from_config(cfg)
    dev = "cuda"
    ws = moe.workspace(spec, T)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    rejected = torch.empty(1, dtype=torch.int32, device=dev)
    moe.moe_route_forced(spec, T, inp["x"], inp["w_router"],
                         torch.as_tensor(forced_h).to(dev), ids, tw, rejected, logits,
                         None, ws)
    r = {"counts_pre": torch.empty(E, dtype=torch.int32, device=dev),
         "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
         "sorted_token": torch.full((T * k,), -7, dtype=torch.int32, device=dev),
         "slot_row": torch.empty((T, k), dtype=torch.int32, device=dev),
         "dropped": torch.empty(1, dtype=torch.int32, device=dev)}
    sw = torch.empty(T * k, dtype=torch.float32, device=dev)
    moe.moe_dispatch(spec, T, ids, tw, r["counts_pre"], r["offsets"], r["sorted_token"],
                     sw, r["slot_row"], r["dropped"], workspace=ws)
    y = torch.zeros((T * k, d), dtype=torch.float32, device=dev)
    ysh = torch.zeros((max(1, cfg.shared_experts) * T, d), dtype=torch.float32, device=dev)
    moe.moe_grouped_ffn(spec, T, r["offsets"], r["sorted_token"], inp["x"], inp, y,
                        ysh if cfg.shared_experts else None, ws)
    r["out"] = torch.empty((T, d), dtype=torch.float32, device=dev)
    moe.moe_combine(spec, T, y, r["slot_row"], tw, ysh if cfg.shared_experts else None,
                    r["out"])
    torch.cuda.synchronize()
    ids_o, w_o, rej_o = oracle.route_forced(logits.cpu().numpy(), forced_h,
                                            gu.spec_dict(cfg))
    ids_g = ids.cpu().numpy()
    assert np.array_equal(ids_g, ids_o) and int(rejected.item()) == int(rej_o.sum())
    assert np.all(np.abs(tw.cpu().numpy().astype(np.float64) - w_o) <= 1e-6)
    disp = gu.check_dispatch(cfg, ids_g, r)
    gu.check_output(cfg, inp, r, ids_g, w_o, disp)
    if cfg.shared_experts == 0:
        out = r["out"].cpu().numpy()
        assert np.all(out[np.flatnonzero(rej_o)] == 0.0)
