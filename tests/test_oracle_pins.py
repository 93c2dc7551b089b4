"""Pins for the CPU oracle: closed forms, invariants, brute force on tiny
inputs and independent formulations, so that a dropped term, a wrong sign
or index, or a transposed operand in the oracle fails one of them.  CPU
only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "closed_forms.json")))


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- capacity
@pytest.mark.parametrize("case", GOLDEN["capacity"])
def test_capacity_closed_forms(case):
    assert oracle.capacity_for(case["T"], case["k"], case["E"], case["cf"]) == case["cap"]


def test_capacity_unlimited_never_drops():
    ids = np.zeros((100, 1), dtype=np.int32)  # everyone on expert 0
    d = oracle.dispatch(ids, 4, oracle.capacity_for(100, 1, 4, 0.0))
    assert d["dropped"] == 0 and d["kept"][0] == 100


# ---------------------------------------------------------------- softmax top-k
def test_softmax_topk_matches_subset_bruteforce():
    """P1: the chosen set is the k-subset of largest total probability."""
    E, k = 8, 2
    L = rng(1).normal(size=(300, E)) * 2.0
    ids, w, p = oracle.select_from_logits(L, k)
    for t in range(L.shape[0]):
        best = max(itertools.combinations(range(E), k),
                   key=lambda S: sum(p[t, e] for e in S))
        assert set(ids[t].tolist()) == set(best)
        assert p[t, ids[t, 0]] >= p[t, ids[t, 1]]
    assert np.all(np.abs(w.sum(axis=1) - 1.0) < 1e-15)
    # probabilities are a distribution, computed from exp directly
    ref = np.exp(L) / np.exp(L).sum(axis=1, keepdims=True)
    assert np.allclose(p, ref, rtol=1e-13, atol=0)


def test_softmax_topk_k1_and_kE():
    L = rng(2).normal(size=(50, 6))
    ids, w, p = oracle.select_from_logits(L, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(L, axis=1))
    ids, w, p = oracle.select_from_logits(L, 6)
    assert np.allclose(w, np.take_along_axis(p, ids, 1), rtol=1e-14, atol=0)
    assert np.array_equal(np.sort(ids, axis=1), np.tile(np.arange(6), (50, 1)))


def test_softmax_topk_no_norm_keeps_probabilities():
    L = rng(3).normal(size=(20, 8))
    ids, w, p = oracle.select_from_logits(L, 3, norm=False)
    assert np.array_equal(w, np.take_along_axis(p, ids, 1))
    assert np.all(w.sum(1) < 1.0)


def test_tie_rule_uniform_logits():
    """P2: zero router -> p = 1/E, ids = 0..k-1, w = 1/k."""
    g = GOLDEN["softmax_uniform"]
    L = np.zeros((5, g["E"]))
    ids, w, p = oracle.select_from_logits(L, g["k"])
    assert np.all(ids == np.array(g["ids"]))
    assert np.all(w == g["w"])
    assert np.all(p == 1.0 / g["E"])


def test_softmax_shift_invariance_and_large_logits():
    L = rng(4).normal(size=(10, 16)) * 5
    a = oracle.select_from_logits(L, 4)
    b = oracle.select_from_logits(L + 700.0, 4)  # exp would overflow unshifted
    assert np.array_equal(a[0], b[0])
    assert np.allclose(a[1], b[1], rtol=1e-12)


# ---------------------------------------------------------------- sigmoid group
def _group_bruteforce(L, k, n_group, topk_group, bias):
    """Independent formulation: the surviving groups are the topk_group-subset
    of largest total group score, and the experts the k-subset of largest
    total selection score inside them (distinct scores assumed)."""
    T, E = L.shape
    G = E // n_group
    s = (1.0 / (1.0 + np.exp(-L.astype(np.float32).astype(np.float64)))).astype(np.float32)
    sel = s + bias.astype(np.float32) if bias is not None else s
    out = []
    for t in range(T):
        gsc = []
        for j in range(n_group):
            top = sorted(sel[t, j * G:(j + 1) * G].tolist(), reverse=True)[:2]
            gsc.append(float(np.float32(top[0]) + np.float32(top[1])))
        groups = max(itertools.combinations(range(n_group), topk_group),
                     key=lambda S: sum(gsc[j] for j in S))
        cand = [e for j in groups for e in range(j * G, (j + 1) * G)]
        best = max(itertools.combinations(cand, k),
                   key=lambda S: sum(float(sel[t, e]) for e in S))
        out.append(set(best))
    return out, s


def test_sigmoid_group_bruteforce():
    E, n_group, topk_group, k = 12, 4, 2, 3
    r = rng(5)
    L = r.normal(size=(120, E)).astype(np.float32)
    bias = r.uniform(-0.05, 0.05, size=E).astype(np.float32)
    ids, w, s = oracle.group_select_from_logits(L, k, n_group, topk_group, 2.5,
                                                True, bias)
    sets, s_ref = _group_bruteforce(L, k, n_group, topk_group, bias)
    for t in range(L.shape[0]):
        assert set(ids[t].tolist()) == sets[t]
    # weights: raw sigmoid of the chosen, normalised, times the scaling
    raw = np.take_along_axis(s_ref.astype(np.float64), ids, 1)
    assert np.allclose(w, raw / raw.sum(1, keepdims=True) * 2.5, rtol=1e-15)


def test_sigmoid_group_all_groups_is_plain_topk():
    """P3: topk_group == n_group drops no group: plain top-k of s + b."""
    E, k = 16, 4
    r = rng(6)
    L = r.normal(size=(80, E)).astype(np.float32)
    bias = r.uniform(-0.05, 0.05, size=E).astype(np.float32)
    ids, _, s = oracle.group_select_from_logits(L, k, 4, 4, 1.0, True, bias)
    for t in range(80):
        sel = [float(np.float32(s[t, e]) + np.float32(bias[e])) for e in range(E)]
        best = max(itertools.combinations(range(E), k), key=lambda S: sum(sel[e] for e in S))
        assert set(ids[t].tolist()) == set(best)


def test_sigmoid_group_uniform_closed_form():
    g = GOLDEN["sigmoid_uniform"]
    L = np.zeros((3, g["E"]), dtype=np.float32)
    ids, w, _ = oracle.group_select_from_logits(L, g["k"], g["n_group"],
                                                g["topk_group"], g["scaling"])
    assert np.all(ids == np.array(g["ids"]))
    assert np.allclose(w, g["w"], rtol=1e-15, atol=0)


def test_sigmoid_group_bias_shift_and_raw_weights():
    E = 16
    r = rng(7)
    L = r.normal(size=(60, E)).astype(np.float32)
    bias = r.uniform(-0.05, 0.05, size=E).astype(np.float32)
    a = oracle.group_select_from_logits(L, 4, 4, 2, 2.5, True, bias)
    # a constant added to every bias changes neither ids nor weights
    b = oracle.group_select_from_logits(L, 4, 4, 2, 2.5, True, bias + np.float32(0.25))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # a large bias on one expert forces it in, yet weights stay raw sigmoid
    big = bias.copy()
    big[5] = 10.0
    ids, w, s = oracle.group_select_from_logits(L, 4, 4, 2, 1.0, False, big)
    assert np.all(np.any(ids == 5, axis=1))
    sig = 1.0 / (1.0 + np.exp(-L.astype(np.float64)))
    assert np.allclose(w, np.take_along_axis(sig, ids, 1), rtol=1e-7, atol=0)


def test_sigmoid_group_norm_off_keeps_scaled_sigmoid():
    L = rng(8).normal(size=(20, 8)).astype(np.float32)
    ids, w, s = oracle.group_select_from_logits(L, 2, 2, 1, 2.5, norm=False)
    assert np.array_equal(w, np.take_along_axis(s.astype(np.float64), ids, 1) * 2.5)


def test_near_tie_flags():
    spec = {"router": "softmax_topk", "top_k": 2}
    L = np.array([[3.0, 1.0, 1.0, 0.0],      # tie at the k boundary
                  [3.0, 2.0, 0.0, -1.0]])    # clear margin
    f = oracle.near_tie_flags(L, spec)
    assert f.tolist() == [True, False]
    spec_g = {"router": "sigmoid_group", "top_k": 2, "n_group": 2, "topk_group": 1}
    L = np.array([[2.0, 1.0, 2.0, 1.0],      # group tie
                  [4.0, 3.0, -2.0, -3.0]], dtype=np.float32)
    assert oracle.near_tie_flags(L, spec_g).tolist() == [True, False]



def _sel_flag(bias_units, tie=0.0):
    """near_tie_flags of one token with zero logits (every sigmoid score is
    exactly 0.5) under SIGMOID_GROUP with E = 8, groups of 2, topk_group 2,
    k = 2 (k < topk_group * G, so the expert margin inside the kept groups
    is examined).  The selection scores are 0.5 + bias; ``bias_units`` are
    multiples of 1/64 (exact in fp32) and ``tie`` an extra offset added to
    expert 2's bias."""
    b = np.array(bias_units, dtype=np.float64) / 64.0
    b[2] += tie
    spec = {"router": "sigmoid_group", "top_k": 2, "n_group": 4, "topk_group": 2}
    L = np.zeros((1, 8), dtype=np.float32)
    return bool(oracle.near_tie_flags(L, spec, b.astype(np.float32))[0])


def test_near_tie_flags_sigmoid_expert_margin():
    """The expert-level margin of SIGMOID_GROUP, hand-built.  Selection
    scores (0.5 + bias) per group of two: group 0 {0.9375, 0.875}, group 1
    {0.8125 + tie, 0.625}, group 2 / group 3 below; group sums keep groups 0
    and 1 by a wide margin.  The kept scores ranked: 0.9375, 0.875,
    0.8125 + tie, 0.625, so the k = 2 margin is 0.875 - (0.8125 + tie)."""
    base = [28, 24, 20, 8, 0, 0, -8, -8]  # /64: 0.4375, 0.375, 0.3125, 0.125, ...
    # margin 1/16: clear
    assert not _sel_flag(base)
    # margin 2^-21 (4.8e-7) < 1e-6: flagged; margin 2^-19 (1.9e-6): not
    assert _sel_flag(base, tie=1 / 16 - 2.0 ** -21)
    assert not _sel_flag(base, tie=1 / 16 - 2.0 ** -19)
    # an exact tie at the k boundary
    assert _sel_flag(base, tie=1 / 16)
    # a tie between the first and second choice is not a boundary: the k-th
    # and (k+1)-th scores (0.875 + 1/16 and 0.8125) stay 1/16 apart
    top_tie = [28, 28, 20, 8, 0, 0, -8, -8]
    assert not _sel_flag(top_tie)
    # the (k+1)-th best score overall sits in a dropped group (group 2:
    # {0.875 + 2^-22, 0.0625}, group sum 0.9375 < group 1's 1.4375) and
    # ties the k-th; inside the kept groups the margin is 1/16, so the token
    # is not flagged
    dropped_tie = [28, 24, 20, 8, 24, -28, -8, -8]
    b = np.array(dropped_tie, dtype=np.float64) / 64.0
    b[4] += 2.0 ** -22
    spec = {"router": "sigmoid_group", "top_k": 2, "n_group": 4, "topk_group": 2}
    L = np.zeros((1, 8), dtype=np.float32)
    assert not oracle.near_tie_flags(L, spec, b.astype(np.float32))[0]
    # the same scores with every group kept: now that tie is the boundary
    spec_all = dict(spec, topk_group=4)
    assert oracle.near_tie_flags(L, spec_all, b.astype(np.float32))[0]

# ---------------------------------------------------------------- dispatch
def _dispatch_sorted(ids, E, cap):
    """The sort-based formulation of the third blog program: flatten slots,
    stable argsort by expert, bincount, keep-mask per expert, offsets from
    kept counts.  Independent of the oracle's queue loop."""
    T, k = ids.shape
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    keep = np.ones(order.size, dtype=bool)
    cur = 0
    for e in range(E):
        c = int(counts[e])
        if cap is not None and c > cap:
            keep[cur + cap:cur + c] = False
        cur += c
    kept_slots = order[keep]
    kept_counts = np.bincount(flat[kept_slots], minlength=E)
    offsets = np.concatenate([[0], np.cumsum(kept_counts)])
    return counts, kept_counts, offsets, kept_slots


@pytest.mark.parametrize("seed", range(6))
def test_dispatch_invariants_and_sorted_formulation(seed):
    r = rng(10 + seed)
    T, E, k = 97, 6, 2
    L = r.normal(size=(T, E)) + np.linspace(0, 2, E)  # skewed: drops
    ids, _, _ = oracle.select_from_logits(L, k)
    cap = oracle.capacity_for(T, k, E, 1.0)
    d = oracle.dispatch(ids, E, cap)
    assert d["count_pre"].sum() == T * k
    assert d["kept"].sum() == T * k - d["dropped"]
    assert np.array_equal(d["kept"], np.minimum(d["count_pre"], cap))
    for e in range(E):
        seg = d["sorted_token"][d["offsets"][e]:d["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(np.any(ids[seg] == e, axis=1))
    # slot_row is the inverse of the permutation
    sr = d["slot_row"].reshape(-1)
    kept_rows = sr[sr >= 0]
    assert np.array_equal(np.sort(kept_rows), np.arange(T * k - d["dropped"]))
    assert np.array_equal(d["sorted_slot"][kept_rows], np.nonzero(sr >= 0)[0])
    # equals the stable-argsort + bincount formulation
    counts, kept_counts, offsets, kept_slots = _dispatch_sorted(ids, E, cap)
    assert np.array_equal(counts, d["count_pre"])
    assert np.array_equal(kept_counts, d["kept"])
    assert np.array_equal(offsets, d["offsets"])
    assert np.array_equal(kept_slots, d["sorted_slot"])
    assert d["dropped"] > 0 or seed > 3


def test_dispatch_zero_router_closed_form():
    """P5: Wr = 0 -> every token picks experts 0..k-1; with capacity c the
    tokens t >= c are dropped from those experts."""
    T, E, k, cf = 40, 8, 2, 1.25
    cap = oracle.capacity_for(T, k, E, cf)  # 40*2/8*1.25 = 12.5 -> 12
    assert cap == 12
    ids, _, _ = oracle.select_from_logits(np.zeros((T, E)), k)
    d = oracle.dispatch(ids, E, cap)
    assert d["kept"].tolist() == [12, 12, 0, 0, 0, 0, 0, 0]
    assert d["sorted_token"].tolist() == list(range(12)) * 2
    assert d["dropped"] == 2 * (T - 12)
    assert np.all(d["slot_row"][12:] == -1)


# ---------------------------------------------------------------- experts / combine
def _tiny_layer(seed, T=48, d=8, E=4, k=2, F=10, act="relu", cf=1.0, shared=0):
    r = rng(100 + seed)
    x = r.normal(size=(T, d))
    wr = r.normal(size=(E, d)) / math.sqrt(d)
    wr[:, 0] += np.linspace(0, 1.5, E)
    x[:, 0] = np.abs(x[:, 0])
    arrays = {"w_gate": r.normal(size=(E, F, d)) / math.sqrt(d),
              "w_up": r.normal(size=(E, F, d)) / math.sqrt(d),
              "w_down": r.normal(size=(E, d, F)) / math.sqrt(F)}
    if shared:
        arrays.update({"sh_gate": r.normal(size=(shared, F, d)),
                       "sh_up": r.normal(size=(shared, F, d)),
                       "sh_down": r.normal(size=(shared, d, F))})
    spec = {"router": "softmax_topk", "E": E, "top_k": k, "act": act,
            "capacity_factor": cf, "shared_experts": shared, "norm_topk_prob": True}
    bank = oracle.ExpertBank.from_arrays(arrays, act)
    return x, wr, arrays, spec, bank


def _ffn(X, act, a, b, o):
    if act == "relu":
        return np.maximum(X @ a.T, 0.0) @ o.T
    z = X @ a.T
    return (z / (1 + np.exp(-z)) * (X @ b.T)) @ o.T


@pytest.mark.parametrize("act", ["relu", "swiglu"])
@pytest.mark.parametrize("seed", range(4))
def test_three_formulations_agree(act, seed):
    """P13: the per-token queue loop (oracle), the per-expert nonzero/truncate
    loop of the second blog program and the sorted-block form of the third
    give the same drops and outputs."""
    x, wr, arrays, spec, bank = _tiny_layer(seed, act=act)
    res = oracle.layer(x, wr, bank, spec)
    T, d = x.shape
    E, k = spec["E"], spec["top_k"]
    ids, w = res["ids"], res["w"]
    cap = res["capacity"]
    # second program: per-expert loop
    out2 = np.zeros((T, d))
    dropped2 = 0
    for e in range(E):
        pos, rank = np.nonzero(ids == e)
        if pos.size > cap:
            dropped2 += pos.size - cap
            pos, rank = pos[:cap], rank[:cap]
        y = _ffn(x[pos], act, arrays["w_gate"][e], arrays["w_up"][e], arrays["w_down"][e])
        out2[pos] += w[pos, rank][:, None] * y
    # third program: sorted blocks + scatter-add
    counts, kept_counts, offsets, kept_slots = _dispatch_sorted(ids, E, cap)
    order = kept_slots // k
    perm_out = np.zeros((order.size, d))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        perm_out[lo:hi] = _ffn(x[order[lo:hi]], act, arrays["w_gate"][e],
                               arrays["w_up"][e], arrays["w_down"][e])
    perm_out *= w.reshape(-1)[kept_slots][:, None]
    out3 = np.zeros((T, d))
    np.add.at(out3, order, perm_out)
    assert res["dispatch"]["dropped"] == dropped2 == T * k - offsets[E]
    assert np.allclose(res["out"], out2, rtol=1e-12, atol=1e-12)
    assert np.allclose(res["out"], out3, rtol=1e-12, atol=1e-12)
    assert dropped2 > 0


def test_dense_mask_formulation_no_drops():
    """P9: every expert on every token, masked by the routing, equals the
    dispatched computation when nothing is dropped."""
    x, wr, arrays, spec, bank = _tiny_layer(7, act="swiglu", cf=0.0)
    res = oracle.layer(x, wr, bank, spec)
    dense = np.zeros_like(res["out"])
    for e in range(spec["E"]):
        y = _ffn(x, "swiglu", arrays["w_gate"][e], arrays["w_up"][e], arrays["w_down"][e])
        mask_w = np.where(res["ids"] == e, res["w"], 0.0).sum(1)
        dense += mask_w[:, None] * y
    assert np.allclose(res["out"], dense, rtol=1e-12, atol=1e-12)


def test_single_expert_is_plain_gemm():
    """P9: one expert that takes every token is two plain matrix products."""
    r = rng(9)
    X = r.normal(size=(30, 6))
    a, o = r.normal(size=(5, 6)), r.normal(size=(6, 5))
    y = oracle.expert_forward(X, "relu", a, None, o)
    h = np.einsum("td,fd->tf", X, a)
    h[h < 0] = 0
    assert np.allclose(y, np.einsum("tf,df->td", h, o), rtol=1e-13)


def test_identical_experts_give_dense_ffn_and_mixture():
    """P10: identical experts with renormalised weights reduce to the dense
    FFN; k = E without capacity is the softmax mixture."""
    x, wr, arrays, spec, bank = _tiny_layer(11, act="swiglu", cf=0.0)
    E = spec["E"]
    for n in ("w_gate", "w_up", "w_down"):
        arrays[n] = np.repeat(arrays[n][:1], E, axis=0)
    res = oracle.layer(x, wr, bank, spec)
    dense = _ffn(x, "swiglu", arrays["w_gate"][0], arrays["w_up"][0], arrays["w_down"][0])
    assert np.allclose(res["out"], dense, rtol=1e-12, atol=1e-12)
    x, wr, arrays, spec, bank = _tiny_layer(12, act="relu", cf=0.0)
    spec["top_k"] = E
    res = oracle.layer(x, wr, bank, spec)
    p = res["p"]
    mix = sum(p[:, e:e + 1] * _ffn(x, "relu", arrays["w_gate"][e], None, arrays["w_down"][e])
              for e in range(E))
    assert np.allclose(res["out"], mix, rtol=1e-12, atol=1e-12)


def test_fully_dropped_token_is_exact_zero():
    """P6: a token whose slots were all dropped gets exactly 0 output."""
    T, E, k, d = 20, 4, 1, 5
    r = rng(13)
    x = r.normal(size=(T, d))
    wr = np.zeros((E, d))
    arrays = {"w_gate": r.normal(size=(E, 7, d)), "w_down": r.normal(size=(E, d, 7))}
    spec = {"router": "softmax_topk", "E": E, "top_k": k, "act": "relu",
            "capacity_factor": 1.0, "shared_experts": 0}
    res = oracle.layer(x, wr, oracle.ExpertBank.from_arrays(arrays, "relu"), spec)
    cap = res["capacity"]  # 20/4 = 5, everyone on expert 0
    assert cap == 5
    assert np.all(res["out"][cap:] == 0.0)
    assert np.all(np.any(res["out"][:cap] != 0.0, axis=1))


def test_shared_expert_added_unweighted():
    x, wr, arrays, spec, bank = _tiny_layer(14, act="swiglu", cf=1.0, shared=1)
    res = oracle.layer(x, wr, bank, spec)
    spec0 = dict(spec, shared_experts=0)
    res0 = oracle.layer(x, wr, bank, spec0)
    sh = _ffn(x, "swiglu", arrays["sh_gate"][0], arrays["sh_up"][0], arrays["sh_down"][0])
    assert np.allclose(res["out"] - res0["out"], sh, rtol=1e-11, atol=1e-11)


def test_silu_relu_closed_forms():
    """P14: hand-built 2x2 closed forms."""
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    X = np.array([[1.0, 2.0]])
    a = np.array([[1.0, 0.0], [0.0, -1.0]])   # pre-activation (1, -2)
    o = np.array([[2.0, 3.0], [0.0, 1.0]])
    assert np.array_equal(oracle.expert_forward(X, "relu", a, None, o), [[2.0, 0.0]])
    b = np.array([[0.0, 1.0], [1.0, 0.0]])    # up = (2, 1)
    s1, s2 = 1.0 / (1.0 + math.exp(-1.0)), -2.0 / (1.0 + math.exp(2.0))
    h = np.array([s1 * 2.0, s2 * 1.0])
    y = oracle.expert_forward(X, "swiglu", a, b, o)
    assert np.allclose(y, [[2 * h[0] + 3 * h[1], h[1]]], rtol=1e-15)


# ---------------------------------------------------------------- stats / bias
def test_aux_loss_uniform_cyclic():
    """P7: cyclic routing with T = m*E gives every expert T*k/E slots and
    P_e = 1/E exactly in expectation over the cycle: aux = 1, aux3 = k."""
    E, k, m = 8, 2, 5
    T = m * E
    L = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            L[t, (t + j) % E] = 3.0
    x = np.eye(T)                     # logits = Wr^T rows via identity input
    res_ids, w, p = oracle.select_from_logits(L, k)
    d = oracle.dispatch(res_ids, E, None)
    st = oracle.layer_stats(d["count_pre"], d["kept"], d["dropped"], p.mean(0), T, k, E)
    g = GOLDEN["aux_uniform"]
    assert np.all(d["kept"] == T * k // E)
    assert abs(st["aux"] - g["aux"]) < 1e-14
    assert abs(st["aux3"] / k - g["aux3_over_k"]) < 1e-14
    assert abs(st["entropy_ratio"] - 1.0) < 1e-14 and not st["collapsed"]
    del x


def test_health_collapse_and_drop_fraction():
    E, T, k = 4, 10, 1
    st = oracle.layer_stats([10, 0, 0, 0], [10, 0, 0, 0], 0, None, T, k, E)
    assert st["entropy"] == 0.0 and st["collapsed"] and st["max_share"] == 1.0
    st = oracle.layer_stats([7, 3, 0, 0], [5, 3, 0, 0], 2, None, T, k, E)
    assert st["dropped_fraction"] == 0.2
    assert abs(st["load_peak_over_mean"] - 7 / 2.5) < 1e-15


def test_bias_update_direction():
    """P8: over-used experts move down, under-used up, equal loads stay."""
    b = np.zeros(4)
    nb = oracle.bias_update(b, np.array([10, 2, 5, 3]), 0.01)  # mean load 5
    assert nb.tolist() == [-0.01, 0.01, 0.0, 0.01]
    assert np.array_equal(oracle.bias_update(b, np.array([1, 2, 3, 4]), None), b)


# ---------------------------------------------------------------- 4-bit weights
def test_u4_golden_pack_and_group():
    gp, gg = GOLDEN["u4_pack"], GOLDEN["u4_group"]
    packed = np.array([[gp["word"]] * 8], dtype=np.uint32)   # one row, K = 64
    scale = np.array([[gg["scale_bits"]]], dtype=np.uint16)
    bias = np.array([[gg["bias_bits"]]], dtype=np.uint16)
    W = oracle.dequant_u4_affine(packed, scale, bias, 64)
    assert W.shape == (1, 64)
    expect = [gg["bias"] + gg["scale"] * q for q in gp["codes"]] * 8
    assert W[0].tolist() == expect
    packed = np.zeros((1, 8), dtype=np.uint32)
    packed[0, 0] = 0xF10                       # codes 0, 1, 15 in nibbles 0..2
    W = oracle.dequant_u4_affine(packed, scale, bias, 64)
    assert W[0, :3].tolist() == gg["w"]


def test_u4_quantiser_roundtrip_and_error_bound():
    """P12: values on the quantisation grid round-trip exactly; arbitrary
    values stay within scale/2 plus the bf16 rounding of scale and bias."""
    g = torch.Generator().manual_seed(0)
    N, K = 16, 128
    q0 = torch.randint(0, 16, (N, K), generator=g).double()
    s0 = torch.full((N, K // 64), 0.0625, dtype=torch.float64)
    b0 = (-1.0 + 0.125 * torch.arange(N, dtype=torch.float64))[:, None].repeat(1, K // 64)  # bf16-exact
    q0[:, ::64] = 0
    q0[:, 1::64] = 15                           # pin min and max of each group
    w_grid = (q0 * s0.repeat_interleave(64, 1) + b0.repeat_interleave(64, 1)).float()
    words, sc, bi = synth.quantize_u4_affine(w_grid, 64)
    W = oracle.dequant_u4_affine(synth.host_array(words), synth.host_array(sc),
                                 synth.host_array(bi), 64)
    assert np.array_equal(W, w_grid.double().numpy())
    w = torch.randn((N, K), generator=g)
    words, sc, bi = synth.quantize_u4_affine(w, 64)
    W = oracle.dequant_u4_affine(synth.host_array(words), synth.host_array(sc),
                                 synth.host_array(bi), 64)
    s = oracle.bf16_to_f64(synth.host_array(sc)).repeat(64, axis=1)
    err = np.abs(W - w.double().numpy())
    # half a step, plus the scale's bf16 rounding over 15 steps and the
    # bias's bf16 rounding (2^-8 relative each)
    bound = 0.5 * s + 15 * s * 2.0 ** -8 + np.abs(w.double().numpy()).max() * 2.0 ** -8
    assert np.all(err <= bound)


# ---------------------------------------------------------------- synth inputs
def test_synth_seeded_and_per_expert():
    cfg = synth.CONFIGS[1]
    a = synth.make_layer_inputs(cfg, "cpu")
    b = synth.make_layer_inputs(cfg, "cpu")
    for kname in ("x", "w_router", "w_gate", "w_down"):
        assert torch.equal(a[kname], b[kname])
    assert a["w_up"] is None and a["x"].dtype == torch.float32
    # one expert regenerates on its own
    e3 = synth.gaussian((cfg.F, cfg.d), 1 / math.sqrt(cfg.d),
                        synth.seed_for(1, synth.TID_GATE, 3), "cpu")
    assert torch.equal(a["w_gate"][3], e3)


def test_cfg1_seeds_include_drops():
    """The tiny fp32 config (capacity 20, mean load 16) drops for at least
    one of the seeds 1234..1241."""
    cfg = synth.CONFIGS[1]
    spec = {"router": "softmax_topk", "top_k": 2}
    drops = []
    for base in range(1234, 1242):
        inp = synth.make_layer_inputs(cfg, "cpu", base=base, with_weights=False)
        L = oracle.router_logits(synth.host_array(inp["x"]), synth.host_array(inp["w_router"]))
        ids, _, _ = oracle.route_from_logits(L, spec)
        drops.append(oracle.dispatch(ids, cfg.E, 20)["dropped"])
    assert max(drops) > 0


def test_zipf_skew_makes_hot_experts():
    cfg = synth.CONFIGS[4].replace(T=2048)
    inp = synth.make_layer_inputs(cfg, "cpu", with_weights=False)
    L = oracle.router_logits(synth.host_array(inp["x"]), synth.host_array(inp["w_router"]))
    ids, _, _ = oracle.select_from_logits(L, cfg.top_k)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    assert counts[0] > 5 * counts.mean()
    assert counts[:8].mean() > counts[-32:].mean() * 4


# ---------------------------------------------------------------- P15 replay
@pytest.mark.parametrize("router", ["softmax", "sigmoid"])
@pytest.mark.parametrize("norm", [True, False])
def test_route_forced_replays_the_routers_own_choice(router, norm):
    """Replaying the ids the router itself chose gives back its weights:
    the forced path and the selection path share only the softmax/sigmoid,
    not the ranking or the renormalisation code."""
    rng = np.random.default_rng(17)
    T, E, k = 40, 16, 4
    L = rng.normal(size=(T, E)).astype(np.float32).astype(np.float64)
    if router == "softmax":
        spec = {"router": oracle.SOFTMAX_TOPK, "top_k": k, "norm_topk_prob": norm}
        ids, w, _ = oracle.route_from_logits(L, spec)
    else:
        spec = {"router": oracle.SIGMOID_GROUP, "top_k": k, "norm_topk_prob": norm,
                "n_group": 4, "topk_group": 2, "routed_scaling": 2.5}
        bias = rng.uniform(-0.05, 0.05, size=E)
        ids, w, _ = oracle.route_from_logits(L, spec, bias)
    ids_f, w_f, rej = oracle.route_forced(L, ids, spec)
    assert not rej.any()
    assert np.array_equal(ids_f, ids)
    np.testing.assert_allclose(w_f, w, rtol=1e-12, atol=0)


def test_route_forced_weights_are_the_gate_at_the_given_ids():
    """Any distinct ids, in any order: weights are p[id] renormalised over
    the given set (softmax), or sigmoid(L)[id] (sigmoid, norm off) -- order
    preserved, worked by hand on one row."""
    L = np.array([[0.0, np.log(2.0), np.log(3.0), np.log(4.0)]])
    spec = {"router": oracle.SOFTMAX_TOPK, "top_k": 2, "norm_topk_prob": True}
    ids, w, rej = oracle.route_forced(L, np.array([[3, 0]]), spec)
    assert ids.tolist() == [[3, 0]] and not rej[0]
    np.testing.assert_allclose(w, [[4.0 / 5.0, 1.0 / 5.0]], rtol=1e-15)
    spec["norm_topk_prob"] = False
    _, w, _ = oracle.route_forced(L, np.array([[1, 2]]), spec)
    np.testing.assert_allclose(w, [[2.0 / 10.0, 3.0 / 10.0]], rtol=1e-15)
    sspec = {"router": oracle.SIGMOID_GROUP, "top_k": 2, "norm_topk_prob": False,
             "n_group": 2, "topk_group": 1, "routed_scaling": 3.0}
    _, w, _ = oracle.route_forced(np.zeros((1, 4)), np.array([[2, 1]]), sspec)
    np.testing.assert_allclose(w, [[1.5, 1.5]], rtol=1e-15)  # 3 * sigmoid(0)


@pytest.mark.parametrize("row", [[-1, 2], [2, 2], [0, 4], [7, -7]])
def test_route_forced_rejects_sentinels_and_duplicates(row):
    """A missing-route sentinel, a repeated id or an id outside [0, E) is
    rejected: identity route, zero weights, reported."""
    L = np.zeros((2, 4))
    spec = {"router": oracle.SOFTMAX_TOPK, "top_k": 2, "norm_topk_prob": True}
    ids, w, rej = oracle.route_forced(L, np.array([[1, 3], row]), spec)
    assert rej.tolist() == [False, True]
    assert ids[1].tolist() == [0, 1] and np.all(w[1] == 0.0)
    np.testing.assert_allclose(w[0], [0.5, 0.5])


# ---------------------------------------------------------------- P16 fused gate/up
def test_fused_gate_up_split_gives_gate_then_up():
    """[edge0] "Weight layout" and "Bundle layout": in the fused tensor each
    expert's gate rows sit above its up rows, so one product with the fused
    matrix, split in two halves along the output, is (gate, up); the slices
    are interleaved expert by expert, and a wholesale concatenation of the
    two stacks would pair the wrong rows."""
    r = rng(71)
    E, F, d = 3, 5, 4
    g = r.normal(size=(E, F, d))
    u = r.normal(size=(E, F, d))
    fused = np.concatenate([g, u], axis=1)          # [E, 2F, d], per expert
    x = r.normal(size=(6, d))
    for e in range(E):
        xg, xu = np.split(x @ fused[e].T, 2, axis=-1)
        assert np.allclose(xg, x @ g[e].T, rtol=1e-13, atol=1e-13)
        assert np.allclose(xu, x @ u[e].T, rtol=1e-13, atol=1e-13)
        a, b = oracle.ExpertBank.split_gate_up(fused[e])
        assert np.array_equal(a, g[e]) and np.array_equal(b, u[e])
    wholesale = np.concatenate([g.reshape(E * F, d), u.reshape(E * F, d)]).reshape(E, 2 * F, d)
    a, b = oracle.ExpertBank.split_gate_up(wholesale[1])
    assert not np.array_equal(a, g[1]) and not np.array_equal(b, u[1])


@pytest.mark.parametrize("seed", range(2))
def test_fused_bank_layer_equals_separate(seed):
    """The layer over a fused gate/up bank (routed and shared experts) is the
    layer over the separate bank, bit for bit; a wholesale-concatenated
    tensor changes the output."""
    x, wr, arrays, spec, bank = _tiny_layer(seed, act="swiglu", shared=1)
    fused = {"w_gate_up": np.concatenate([arrays["w_gate"], arrays["w_up"]], axis=1),
             "w_down": arrays["w_down"],
             "sh_gate_up": np.concatenate([arrays["sh_gate"], arrays["sh_up"]], axis=1),
             "sh_down": arrays["sh_down"]}
    a = oracle.layer(x, wr, bank, spec)
    b = oracle.layer(x, wr, oracle.ExpertBank.from_arrays(fused, "swiglu", fused=True), spec)
    assert np.array_equal(a["out"], b["out"])
    E, F, d = arrays["w_gate"].shape
    bad = dict(fused)
    bad["w_gate_up"] = np.concatenate([arrays["w_gate"].reshape(E * F, d),
                                       arrays["w_up"].reshape(E * F, d)]).reshape(E, 2 * F, d)
    c = oracle.layer(x, wr, oracle.ExpertBank.from_arrays(bad, "swiglu", fused=True), spec)
    assert not np.allclose(a["out"], c["out"])


def test_fused_u4_inputs_decode_to_the_separate_experts():
    """4-bit codes, scales and biases in the fused storage (synth's fusing of
    the seeded separate tensors) decode, through the fused bank, to exactly
    the separate bank's gate and up matrices."""
    base = synth.LayerConfig("u4-fused-pin", 77, T=4, d=128, E=3, top_k=2, F=64,
                             weight_dtype=synth.U4, shared_experts=1, shared_F=64)
    sep = synth.make_layer_inputs(base)
    fus = synth.make_layer_inputs(base.replace(layout=synth.FUSED_GATE_UP))
    assert fus["q_gate_up"].shape == (3, 128, 16) and fus["s_gate_up"].shape == (3, 128, 2)
    assert "q_up" not in fus and "sh_up" not in fus

    def bank(inp, fused):
        arrays = {k: synth.host_array(v) for k, v in inp.items()
                  if v is not None and k not in ("x", "w_router", "expert_bias")}
        return oracle.ExpertBank.from_arrays(arrays, "swiglu", u4=True, fused=fused)

    bs, bf = bank(sep, False), bank(fus, True)
    for e in range(3):
        for m1, m2 in zip(bs.routed(e), bf.routed(e)):
            assert np.array_equal(m1, m2)
    for m1, m2 in zip(bs.shared(0), bf.shared(0)):
        assert np.array_equal(m1, m2)
