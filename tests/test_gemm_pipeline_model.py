"""Host-side check of the load pipeline of the grouped GEMM
(grouped_gemm_kernel in csrc/gemm_bf16.hip), restated from the kernel for
every stage configuration it is built with and every K-step count from 1 to
12, as one wave's sequence of events:

  * the direct loads it issues, in order: the prologue's (activations, then
    weights, of steps 0, 1 and 2 where stages exist), then after the barrier
    that ends step kt the activations of step kt + NSA and the weights of
    step kt + NSW (while those steps exist);
  * the counted waits: before step 0 `vmcnt(loads of the later prologue
    steps)`, and before the barrier that publishes step kt + 1
    `vmcnt(loads issued after step kt + 1's)` while step kt + 2's loads are
    in flight, else `vmcnt(0)`.

Vector-memory loads retire in issue order, so a wait for "at most N pending"
leaves pending only the N loads issued last.  The model checks that every
step's activation and weight loads have all retired at the wait before the
step is read, that each step is loaded exactly once, and that a stage is
reloaded only after the barrier that ends the last step read from it.  The
GPU parity tests cover K = 64, 128, 192 and longer reductions; this pins
the bookkeeping for every count."""
import pytest

# (NSA, NSW, activation loads per step, weight loads per step) per wave:
# 256-row bf16 tiles (2 + 3 stages), 128-row bf16 tiles and the 4-bit tiles
# (3 + 3 stages; 4-bit weights: one code load and one scale/bias load)
CONFIGS = {
    "bf16-256": (2, 3, 4, 4),
    "bf16-128": (3, 3, 2, 4),
    "u4-256": (3, 3, 4, 2),
    "u4-128": (3, 3, 2, 2),
}


def schedule(NSA, NSW, LA, LW, KT):
    """Events of one wave: ("load", operand, step) per load instruction,
    ("wait", n, step) for a counted wait before `step` is read,
    ("barrier", step) for the barrier after which `step` is read."""
    ev = []

    def issue_a(j):
        ev.extend(("load", "A", j) for _ in range(LA))

    def issue_w(j):
        ev.extend(("load", "W", j) for _ in range(LW))

    step_loads = LA + LW
    # prologue
    issue_a(0)
    issue_w(0)
    if KT > 1:
        issue_a(1)
        issue_w(1)
    if KT > 2:
        if NSA > 2:
            issue_a(2)
        if NSW > 2:
            issue_w(2)
    pro2 = (LA if NSA > 2 else 0) + (LW if NSW > 2 else 0)
    if pro2 > 0 and KT > 2:
        ev.append(("wait", step_loads + pro2, 0))
    elif KT > 1:
        ev.append(("wait", step_loads, 0))
    else:
        ev.append(("wait", 0, 0))
    ev.append(("barrier", 0))
    later = (step_loads if NSA == 3 else LW) if NSW == 3 else 0
    for kt in range(KT):
        if kt + NSW < KT:
            kind = 0
        elif NSA < NSW and kt + NSA < KT:
            kind = 3
        elif kt + 1 < KT:
            kind = 1
        else:
            kind = 2
        ev.append(("reads", kt))
        if kind == 2:
            continue
        ev.append(("wait", later if (later > 0 and kt + 2 < KT) else 0, kt + 1))
        ev.append(("barrier", kt + 1))
        if kind == 0:
            issue_a(kt + NSA)
            issue_w(kt + NSW)
        elif kind == 3:
            issue_a(kt + NSA)
    return ev


@pytest.mark.parametrize("name", list(CONFIGS))
@pytest.mark.parametrize("KT", list(range(1, 13)))
def test_every_step_is_complete_when_read_and_stages_are_free_when_reloaded(name, KT):
    NSA, NSW, LA, LW = CONFIGS[name]
    ev = schedule(NSA, NSW, LA, LW, KT)
    issued = []          # (operand, step) per load, in issue order
    retired = 0          # loads known retired (a prefix of `issued`)
    last_read = {}       # (operand, stage) -> last step read from it
    published = -1       # last step published by a barrier
    for e in ev:
        if e[0] == "load":
            _, op, j = e
            ns = NSA if op == "A" else NSW
            stage = j % ns
            # the stage's previous step has been read to the end and a
            # barrier has passed since (its reads precede the barrier that
            # publishes the following step)
            prev = last_read.get((op, stage))
            assert prev is None or published > prev, (name, KT, op, j, prev, published)
            issued.append((op, j))
        elif e[0] == "wait":
            _, n, step = e
            retired = max(retired, len(issued) - n)
            pending = issued[retired:]
            assert ("A", step) not in pending and ("W", step) not in pending, (name, KT, step, n)
            assert ("A", step) in issued and ("W", step) in issued, (name, KT, step)
        elif e[0] == "barrier":
            published = e[1]
        elif e[0] == "reads":
            j = e[1]
            assert published == j
            last_read[("A", j % NSA)] = j
            last_read[("W", j % NSW)] = j
    # each step loaded exactly once, and nothing beyond the reduction
    for op, ns, per in (("A", NSA, LA), ("W", NSW, LW)):
        for j in range(KT):
            assert sum(1 for x in issued if x == (op, j)) == per, (name, KT, op, j)
        assert all(j < KT for o, j in issued if o == op)


def test_weights_run_ahead_of_activations_with_two_activation_stages():
    """With 2 activation and 3 weight stages, the weights of step t + 2 are
    in flight when step t + 1 is published (two steps ahead) and the
    activations of step t + 1 only since step t - 1 ended (one ahead)."""
    ev = schedule(2, 3, 4, 4, 10)
    pos = {}
    for i, e in enumerate(ev):
        if e[0] == "load":
            pos.setdefault((e[1], e[2]), i)
        if e[0] == "barrier":
            pos[("barrier", e[1])] = i
    for t in range(1, 8):
        # weights of step t + 2 were issued before the barrier publishing t + 1
        assert pos[("W", t + 2)] < pos[("barrier", t + 1)]
        # activations of step t + 1 were issued once step t - 1 had ended
        # (the barrier publishing t), before the barrier publishing t + 1
        assert pos[("barrier", t)] < pos[("A", t + 1)] < pos[("barrier", t + 1)]
        # and the weights of step t + 2 at the same point
        assert pos[("barrier", t)] < pos[("W", t + 2)]
