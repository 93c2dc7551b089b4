"""CPU oracle for the sparse MoE layer forward: route -> dispatch -> expert
FFN -> combine.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module.  The product path (the HIP
library and its Python binding) never does, and the two share no code: this
file uses NumPy only.

Arithmetic is fp64 throughout, on inputs decoded exactly (bf16 bit patterns
and 4-bit affine codes are decoded to fp64 without rounding), except where a
page fixes the precision: the sigmoid-group selection of the Edge0 page
("MoE Spec and Routing", ``group_select_from_logits``) casts logits to fp32
and scores in fp32, so its *selection* values (sigmoid, sigmoid + bias, group
sums) are held in fp32 here too.  Sorting and matrix products are NumPy
library routines; everything else is written out step by step.

Pages cited (by title):
  [dockyard]  "Mixture-of-Experts" (dockyard_rl design doc)
  [compdocs]  "Mixture-of-Experts Documentation" (moe-competition docs)
  [blog]      "Mixture of Experts" blog page -- three programs: the first
              pure-Python one, the second with RoutingHealth, the third
              with tokens sorted into contiguous expert blocks
  [skill]     "moe-architecture" skill page
  [edge0]     "MoE Spec and Routing (MoESpec / Routing)" (Edge0 docs)

Every function below is pinned by a CPU test in ``tests/`` (closed forms,
invariants, brute force, or an independent formulation); none is "parity
unpinned".
"""
from __future__ import annotations

import math
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

SOFTMAX_TOPK = "softmax_topk"
SIGMOID_GROUP = "sigmoid_group"
SWIGLU = "swiglu"
RELU = "relu"

# [blog] second program: below half of the uniform entropy the router has
# collapsed.
COLLAPSE_ENTROPY_RATIO = 0.5


# --------------------------------------------------------------------------
# exact decoding of stored inputs
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def as_f64(a: np.ndarray) -> np.ndarray:
    """Exact fp64 view of a stored tensor: uint16 is bf16, floats widen."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64, copy=False)


def dequant_u4_affine(packed: np.ndarray, scale: np.ndarray, bias: np.ndarray,
                      group: int = 64) -> np.ndarray:
    """4-bit affine weights -> fp64, [edge0] ``QuantSpec`` (bits 4, group 64,
    mode affine): w = scale * q + bias, one (scale, bias) per ``group``
    consecutive elements along K of one output row; q in 0..15.

    Storage: ``packed`` [N, K/8] uint32, element 8j+i of a row in nibble i
    (low nibble first) of word j; ``scale``/``bias`` [N, K/group] bf16.
    """
    packed = np.asarray(packed, dtype=np.uint32)
    N, W = packed.shape
    K = W * 8
    shifts = (4 * np.arange(8, dtype=np.uint32))
    q = ((packed[:, :, None] >> shifts[None, None, :]) & np.uint32(0xF))
    q = q.reshape(N, K).astype(np.float64)
    s = np.repeat(bf16_to_f64(scale), group, axis=1)
    b = np.repeat(bf16_to_f64(bias), group, axis=1)
    return s * q + b


# --------------------------------------------------------------------------
# capacity
# --------------------------------------------------------------------------
def capacity_for(T: int, top_k: int, E: int, capacity_factor: float) -> Optional[int]:
    """Per-expert buffer size, [blog] first program ``moe_layer`` and second
    program ``MoEConfig.capacity_for``: max(1, int(T*k/E*cf)), evaluated
    left to right in double precision and truncated.  ``capacity_factor``
    0 means no capacity limit (returns None): the Mixtral-shaped workload
    has none.
    """
    if capacity_factor == 0:
        return None
    exact = T * top_k / E * capacity_factor
    return max(1, int(exact))


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """Bias-free linear gate, [skill] "Design the router"; [blog] second
    program ``Router.route`` (fp64 logits): L = x @ Wr^T."""
    return as_f64(x) @ as_f64(w_router).T


def softmax(L: np.ndarray) -> np.ndarray:
    """Max-shifted softmax over the last axis ([blog] first program
    ``softmax``; [edge0] ``precise=True``)."""
    L = np.asarray(L, dtype=np.float64)
    shifted = L - L.max(axis=-1, keepdims=True)
    ex = np.exp(shifted)
    return ex / ex.sum(axis=-1, keepdims=True)


def rank_descending(scores: np.ndarray) -> np.ndarray:
    """Indices ordered by score, highest first; equal scores keep index
    order (a stable sort on the negated score, as the first [blog] program's
    ``route`` sorts).  This fixes the one case -- exact ties -- where
    several top-k answers would otherwise be correct."""
    return np.argsort(-scores, axis=-1, kind="stable")


def select_from_logits(L: np.ndarray, top_k: int, norm: bool = True):
    """SOFTMAX_TOPK, [edge0] ``select_from_logits`` and [blog] ``route``:
    p = softmax(L); keep the k most probable experts; weights are p over
    the kept mass when ``norm`` (renormalisation), else p itself.

    Returns (ids [T,k] int32, highest first; weights [T,k] fp64;
    probabilities [T,E] fp64).
    """
    p = softmax(L)
    ids = rank_descending(p)[:, :top_k]
    pk = np.take_along_axis(p, ids, axis=-1)
    w = pk / pk.sum(axis=-1, keepdims=True) if norm else pk
    return ids.astype(np.int32), w, p


def sigmoid_f32(L: np.ndarray) -> np.ndarray:
    """Sigmoid of fp32 logits held in fp32: evaluated in fp64 and rounded
    once, i.e. the correctly rounded fp32 sigmoid ([edge0]
    ``group_select_from_logits`` scores fp32 logits)."""
    L32 = np.asarray(L, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-L32))
    return s.astype(np.float32)


def group_selection_scores(L: np.ndarray, n_group: int,
                           expert_bias: Optional[np.ndarray]):
    """Selection scores of SIGMOID_GROUP in fp32: s = sigmoid(L), sel = s +
    bias, and per group the sum of its two largest sel.  Groups are
    contiguous blocks of E/n_group experts."""
    s = sigmoid_f32(L)
    sel = s + np.asarray(expert_bias, dtype=np.float32)[None, :] \
        if expert_bias is not None else s.copy()
    T, E = sel.shape
    G = E // n_group
    grouped = sel.reshape(T, n_group, G)
    two = -np.sort(-grouped, axis=-1)[..., :2]
    gscore = (two[..., 0] + two[..., 1]).astype(np.float32)
    return s, sel, gscore


def group_select_from_logits(L: np.ndarray, top_k: int, n_group: int,
                             topk_group: int, routed_scaling: float,
                             norm: bool = True,
                             expert_bias: Optional[np.ndarray] = None):
    """SIGMOID_GROUP, [edge0] ``group_select_from_logits`` (DeepSeek-V3
    rules):

      1. s = sigmoid(L) (fp32); selection score sel = s + bias (bias steers
         selection only);
      2. each group scores the sum of its top-two sel; the best
         ``topk_group`` groups survive (ties to the lower group index) and
         the other groups' sel become -inf -- nothing is dropped when
         ``topk_group == n_group``;
      3. the k largest sel are chosen (ties to the lower index);
      4. weights are the chosen experts' raw s (bias excluded), divided by
         (their sum + 1e-20) when ``norm``, then times ``routed_scaling``.

    Returns (ids [T,k] int32, weights [T,k] fp64, s [T,E] fp32).
    """
    s, sel, gscore = group_selection_scores(L, n_group, expert_bias)
    T, E = sel.shape
    G = E // n_group
    masked = sel.astype(np.float64)
    if topk_group < n_group:
        drop = rank_descending(gscore.astype(np.float64))[:, topk_group:]
        m = masked.reshape(T, n_group, G)
        rows = np.arange(T)[:, None]
        m[rows, drop, :] = -np.inf
        masked = m.reshape(T, E)
    ids = rank_descending(masked)[:, :top_k]
    w = np.take_along_axis(s.astype(np.float64), ids, axis=-1)
    if norm:
        w = w / (w.sum(axis=-1, keepdims=True) + 1e-20)
    w = w * routed_scaling
    return ids.astype(np.int32), w, s


def route_from_logits(L: np.ndarray, spec: Dict, expert_bias=None):
    """Steps after the logits, for either router kind.  Returns (ids,
    weights, probabilities or None); probabilities only for SOFTMAX_TOPK."""
    if spec["router"] == SOFTMAX_TOPK:
        if expert_bias is not None:
            raise ValueError("a selection bias belongs to sigmoid-group routing")
        return select_from_logits(L, spec["top_k"], spec.get("norm_topk_prob", True))
    ids, w, _ = group_select_from_logits(
        L, spec["top_k"], spec["n_group"], spec["topk_group"],
        spec.get("routed_scaling", 1.0), spec.get("norm_topk_prob", True),
        expert_bias)
    return ids, w, None


def route_forced(L: np.ndarray, forced_ids: np.ndarray, spec: Dict):
    """Router replay, [dockyard] "Router replay (R3)": the expert ids of
    every token are given (recorded at generation), and the gating weights
    still come from the model's own gate on these logits:

      * SOFTMAX_TOPK: p = softmax(L); w_i = p[id_i], divided by the given
        ids' total probability when ``norm_topk_prob``;
      * SIGMOID_GROUP: w_i = sigmoid(L)[id_i] (fp32 scores, no bias: the
        bias only steers selection), divided by (their sum + 1e-20) when
        ``norm_topk_prob``, then times ``routed_scaling``.

    A row whose ids are not k distinct experts in [0, E) -- e.g. the
    sentinel of a missing route -- is rejected instead of replayed: it gets
    the identity route 0..k-1 with zero weights and is reported.

    Returns (ids [T,k] int32, weights [T,k] fp64, rejected [T] bool).
    """
    T, E = L.shape
    k = spec["top_k"]
    f = np.asarray(forced_ids, dtype=np.int64).reshape(T, k)
    in_range = np.all((f >= 0) & (f < E), axis=1)
    distinct = np.array([len(set(row.tolist())) == k for row in f])
    rejected = ~(in_range & distinct)
    ids = np.where(rejected[:, None], np.arange(k)[None, :], f)
    if spec["router"] == SOFTMAX_TOPK:
        score = softmax(L)
    else:
        score = sigmoid_f32(L).astype(np.float64)
    w = np.take_along_axis(score, ids, axis=-1)
    if spec["router"] == SOFTMAX_TOPK:
        if spec.get("norm_topk_prob", True):
            w = w / w.sum(axis=-1, keepdims=True)
    else:
        if spec.get("norm_topk_prob", True):
            w = w / (w.sum(axis=-1, keepdims=True) + 1e-20)
        w = w * spec.get("routed_scaling", 1.0)
    w[rejected] = 0.0
    return ids.astype(np.int32), w, rejected


def route(x, w_router, spec: Dict, expert_bias=None):
    """Router: fp64 logits, then ``route_from_logits``.  Returns (L, ids,
    weights, probabilities or None)."""
    L = router_logits(x, w_router)
    ids, w, p = route_from_logits(L, spec, expert_bias)
    return L, ids, w, p


def near_tie_flags(L: np.ndarray, spec: Dict, expert_bias=None,
                   eps: float = 1e-6) -> np.ndarray:
    """Tokens whose top-k decision has a margin below ``eps``: the gap
    between the k-th and (k+1)-th selection score (p for SOFTMAX_TOPK, sel
    for SIGMOID_GROUP, among the surviving groups), and for SIGMOID_GROUP
    also the gap between the ``topk_group``-th and next group score.  There
    is no margin when everything is kept."""
    T = L.shape[0]
    k = spec["top_k"]
    flags = np.zeros(T, dtype=bool)
    if spec["router"] == SOFTMAX_TOPK:
        p = softmax(L)
        E = p.shape[1]
        if k < E:
            srt = -np.sort(-p, axis=-1)
            flags |= (srt[:, k - 1] - srt[:, k]) < eps
        return flags
    n_group, topk_group = spec["n_group"], spec["topk_group"]
    _, sel, gscore = group_selection_scores(L, n_group, expert_bias)
    E = sel.shape[1]
    G = E // n_group
    sel = sel.astype(np.float64)
    if topk_group < n_group:
        gs = -np.sort(-gscore.astype(np.float64), axis=-1)
        flags |= (gs[:, topk_group - 1] - gs[:, topk_group]) < eps
        drop = rank_descending(gscore.astype(np.float64))[:, topk_group:]
        m = sel.reshape(T, n_group, G).copy()
        m[np.arange(T)[:, None], drop, :] = -np.inf
        sel = m.reshape(T, E)
    if k < topk_group * G:
        srt = -np.sort(-sel, axis=-1)
        flags |= (srt[:, k - 1] - srt[:, k]) < eps
    return flags


# --------------------------------------------------------------------------
# dispatch
# --------------------------------------------------------------------------
def dispatch(ids: np.ndarray, E: int, capacity: Optional[int]) -> Dict[str, np.ndarray]:
    """Capacity-limited assignment in arrival order, [blog] first program
    ``moe_layer``: visit tokens in order and, inside a token, its k choices;
    each expert takes slots until its capacity is full and every later slot
    for it is dropped (no expert applied, nothing added).

    Returns, as arrays:
      count_pre [E]     slots that chose e (before capacity)
      kept [E]          slots kept by e = min(count_pre, capacity)
      offsets [E+1]     exclusive prefix of ``kept``: e owns rows
                        offsets[e]:offsets[e+1]
      sorted_token [N]  token of each kept row (expert-major, token order
                        inside an expert)
      sorted_slot [N]   flat slot t*k+i of each kept row
      slot_row [T,k]    row of slot (t,i), -1 if dropped
      dropped           T*k - N
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    count_pre = np.zeros(E, dtype=np.int64)
    queues: List[List[int]] = [[] for _ in range(E)]
    for t in range(T):
        for i in range(k):
            e = int(ids[t, i])
            count_pre[e] += 1
            if capacity is None or len(queues[e]) < capacity:
                queues[e].append(t * k + i)
    kept = np.array([len(q) for q in queues], dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    sorted_slot = np.array([s for q in queues for s in q], dtype=np.int64)
    sorted_token = sorted_slot // k
    slot_row = np.full(T * k, -1, dtype=np.int64)
    slot_row[sorted_slot] = np.arange(sorted_slot.size)
    return {
        "count_pre": count_pre,
        "kept": kept,
        "offsets": offsets,
        "sorted_token": sorted_token,
        "sorted_slot": sorted_slot,
        "slot_row": slot_row.reshape(T, k),
        "dropped": int(T * k - offsets[E]),
    }


# --------------------------------------------------------------------------
# experts
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_forward(X: np.ndarray, act: str, w_a: np.ndarray,
                   w_b: Optional[np.ndarray], w_out: np.ndarray) -> np.ndarray:
    """One expert on rows X [n, d] (fp64).

    ReLU ([blog] ``expert_forward``): y = W_out relu(W_in x).
    SwiGLU ([edge0] ``_swiglu``: silu(gate) * up; [skill] Mixtral expert
    with SiLU): y = W_down (silu(W_gate x) * (W_up x)).
    Weights are [out, in] row-major, applied as X @ W^T ([blog] second
    program).
    """
    if act == RELU:
        h = X @ w_a.T
        h = np.where(h > 0.0, h, 0.0)
    else:
        h = silu(X @ w_a.T) * (X @ w_b.T)
    return h @ w_out.T


class ExpertBank:
    """fp64 expert matrices decoded on demand from stored tensors.

    ``fetch(name, index)`` returns the raw stored slice: for name in
    w_gate/w_up/w_down/sh_gate/sh_up/sh_down a [N, K] array (float32, or
    uint16 bf16 bits), and for 4-bit weights q_* (uint32 packed), s_*, b_*
    (uint16 bf16 bits).

    ``fused``: the gate and up projections are stored together, [edge0]
    "Weight layout" (FUSED_GATE_UP) and "Bundle layout and the up-first
    order": one [2F, K] slice per expert under w_gate_up
    (q_/s_/b_gate_up for 4-bit, sh_gate_up for shared experts) whose first F
    rows are the gate and the last F the up projection, so that splitting
    x @ W^T in two halves gives (gate, up).
    """

    def __init__(self, fetch: Callable[[str, int], np.ndarray], act: str,
                 u4: bool = False, group: int = 64, fused: bool = False):
        self.fetch = fetch
        self.act = act
        self.u4 = u4
        self.group = group
        self.fused = fused

    @classmethod
    def from_arrays(cls, arrays: Dict[str, np.ndarray], act: str,
                    u4: bool = False, group: int = 64,
                    fused: bool = False) -> "ExpertBank":
        return cls(lambda name, e: arrays[name][e], act, u4, group, fused)

    @staticmethod
    def split_gate_up(w: np.ndarray):
        """(gate, up) of one fused [2F, K] slice: gate rows on top."""
        F = w.shape[0] // 2
        return w[:F], w[F:]

    def _mat(self, name: str, e: int) -> np.ndarray:
        if self.u4 and not name.startswith("sh_"):
            part = name.split("_", 1)[1]
            return dequant_u4_affine(self.fetch("q_" + part, e),
                                     self.fetch("s_" + part, e),
                                     self.fetch("b_" + part, e), self.group)
        return as_f64(self.fetch(name, e))

    def routed(self, e: int):
        if self.fused:
            a, b = self.split_gate_up(self._mat("w_gate_up", e))
        else:
            a = self._mat("w_gate", e)
            b = self._mat("w_up", e) if self.act == SWIGLU else None
        return a, b, self._mat("w_down", e)

    def shared(self, s: int):
        if self.fused:
            a, b = self.split_gate_up(as_f64(self.fetch("sh_gate_up", s)))
        else:
            a = as_f64(self.fetch("sh_gate", s))
            b = as_f64(self.fetch("sh_up", s)) if self.act == SWIGLU else None
        return a, b, as_f64(self.fetch("sh_down", s))


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------
def combine(T: int, d: int, ids: np.ndarray, w: np.ndarray,
            slot_row: np.ndarray, expert_out: Dict[int, np.ndarray],
            shared_out: Optional[np.ndarray] = None,
            tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """Weighted sum back in token order ([dockyard] "The pipeline", combine;
    [blog] first program's accumulation; [skill] output = sum of weight_i *
    expert_i(input)).

    out[t] = sum over kept slots i of w[t,i] * y_{t,i}  (+ shared experts'
    outputs, unweighted).  A dropped slot adds nothing and the remaining
    weights are not renormalised; a token with every slot dropped and no
    shared expert gets exactly 0.

    ``expert_out`` maps a kept row (``slot_row`` value) to that slot's
    expert output (1-D, fp64).  ``tokens`` restricts the result to those
    tokens (rows of the returned array follow ``tokens``).
    """
    toks = list(range(T)) if tokens is None else list(tokens)
    out = np.zeros((len(toks), d), dtype=np.float64)
    k = ids.shape[1]
    for j, t in enumerate(toks):
        for i in range(k):
            r = int(slot_row[t, i])
            if r >= 0:
                out[j] += w[t, i] * expert_out[r]
        if shared_out is not None:
            out[j] += shared_out[j]
    return out


# --------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------
def ffn_and_combine(x: np.ndarray, ids: np.ndarray, w: np.ndarray,
                    disp: Dict[str, np.ndarray], bank: ExpertBank,
                    spec: Dict, tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """Expert FFN on every kept slot (of ``tokens``, or all tokens) plus the
    shared experts, then ``combine``.  Slots of one expert are evaluated
    together as one fp64 matrix product (a library matmul; the per-row
    result is the per-token definition)."""
    X = as_f64(x)
    T, d = X.shape
    k = ids.shape[1]
    toks = list(range(T)) if tokens is None else list(tokens)
    slot_row = disp["slot_row"]
    by_expert: Dict[int, List[int]] = {}
    for t in toks:
        for i in range(k):
            r = int(slot_row[t, i])
            if r >= 0:
                by_expert.setdefault(int(ids[t, i]), []).append(r)
    expert_out: Dict[int, np.ndarray] = {}
    sorted_token = disp["sorted_token"]
    for e in sorted(by_expert):
        rows = by_expert[e]
        wa, wb, wo = bank.routed(e)
        Y = expert_forward(X[sorted_token[rows]], spec["act"], wa, wb, wo)
        for r, y in zip(rows, Y):
            expert_out[r] = y
    shared_out = None
    S = spec.get("shared_experts", 0)
    if S:
        shared_out = np.zeros((len(toks), d))
        for s in range(S):
            wa, wb, wo = bank.shared(s)
            shared_out += expert_forward(X[toks], spec["act"], wa, wb, wo)
    return combine(T, d, ids, w, slot_row, expert_out, shared_out, toks)


def layer(x, w_router, bank: ExpertBank, spec: Dict, expert_bias=None,
          tokens: Optional[Sequence[int]] = None) -> Dict:
    """Whole forward: fp64 logits -> route -> capacity dispatch -> expert
    FFN -> combine, plus routing statistics.  Returns a dict with out
    ([T or len(tokens), d] fp64), the routing and dispatch arrays and
    ``stats``."""
    T = np.asarray(x).shape[0]
    L, ids, w, p = route(x, w_router, spec, expert_bias)
    cap = capacity_for(T, spec["top_k"], spec["E"], spec.get("capacity_factor", 0.0))
    disp = dispatch(ids, spec["E"], cap)
    out = ffn_and_combine(x, ids, w, disp, bank, spec, tokens)
    P = p.mean(axis=0) if p is not None else None
    st = layer_stats(disp["count_pre"], disp["kept"], disp["dropped"], P, T,
                     spec["top_k"], spec["E"])
    return {"out": out, "logits": L, "ids": ids, "w": w, "p": p,
            "capacity": cap, "dispatch": disp, "stats": st}


# --------------------------------------------------------------------------
# statistics and the load-balance bias
# --------------------------------------------------------------------------
def layer_stats(count_pre, kept, dropped: int, P: Optional[np.ndarray],
                T: int, top_k: int, E: int) -> Dict:
    """Routing statistics from the dispatch counts.

    * aux: E * sum_e f_e * P_e with f_e = kept_e / (T*k) (the fraction of
      routed slots; equals 1 under uniform routing) and P_e the mean router
      probability ([blog] ``load_balancing_loss``; [skill] step 4).  aux3 is
      the same sum with f_e = kept_e / T as the [blog] programs code it
      (= k * aux).  Softmax routing only (P is None otherwise).
    * health ([blog] second program ``RoutingHealth`` / third program
      ``routing_health``): shares = kept/T, entropy of the normalised
      shares, max entropy log E, their ratio, collapse below 0.5, dropped
      fraction = dropped/(T*k), max normalised share.
    * load peak/mean over the pre-capacity counts.
    """
    kept = np.asarray(kept, dtype=np.float64)
    count_pre = np.asarray(count_pre, dtype=np.float64)
    st: Dict = {"count_pre": count_pre.astype(np.int64),
                "kept": kept.astype(np.int64), "dropped": int(dropped)}
    if P is not None:
        st["aux"] = float(E * np.dot(kept / (T * top_k), P))
        st["aux3"] = float(E * np.dot(kept / T, P))
    shares = kept / T
    total = shares.sum()
    if total <= 0.0:
        entropy, ratio, max_share = 0.0, 0.0, 0.0
    else:
        nz = shares[shares > 0.0] / total
        entropy = float(-np.sum(nz * np.log(nz)))
        ratio = entropy / math.log(E)
        max_share = float((shares / total).max())
    st.update({"shares": shares, "entropy": entropy,
               "max_entropy": math.log(E), "entropy_ratio": ratio,
               "collapsed": ratio < COLLAPSE_ENTROPY_RATIO,
               "max_share": max_share,
               "dropped_fraction": dropped / (T * top_k),
               "load_peak_over_mean": float(count_pre.max() / count_pre.mean())
               if count_pre.sum() > 0 else 0.0})
    return st


def bias_update(bias: np.ndarray, load: np.ndarray, coeff: Optional[float]) -> np.ndarray:
    """Aux-loss-free balancing, [dockyard] "Aux-loss-free load balancing":
    each step every expert's selection bias moves by the step size --
    up when the expert's load is below the mean load, down when above,
    unchanged when equal.  ``coeff`` None switches it off."""
    b = np.asarray(bias, dtype=np.float64)
    if coeff is None:
        return b.copy()
    load = np.asarray(load, dtype=np.float64)
    return b + coeff * np.sign(load.mean() - load)
