"""Host-side check of the index scheme of the 4-bit matrix-core kernels
(csrc/gemm_u4.hip), restated here from the kernel's formulas: the direct
loads of one item fill LDS with a permutation of the item's code bytes that
puts, for every lane and LDS read, the 16 bytes that lane needs; the 16
lanes one LDS read serves together hit distinct banks for K >= 512; and the
halving lane sum leaves every (unit, activation row) total in exactly one
writing lane, with gate and up of the same output pairable.  The GPU parity
tests check the kernels themselves; this pins the scheme they implement.
"""
import pytest

KS = (64, 128, 256, 512, 1024, 2048)


def kcfg(K):
    KB = min(K, 128)
    NKS = K // KB
    NUG = 16 // NKS
    UPI = 4 * NUG
    kCode = UPI * K // 2
    return dict(KB=KB, NKS=NKS, NUG=NUG, UPI=UPI, G=K // 64, WPL=KB // 8, GPL=KB // 64,
                kCode=kCode, kDma=kCode // 1024, kSB=UPI * (K // 64) * 2,
                kSeg=min(K // 2, 64), kPieces=min(K // 2, 64) // 16)


def dma_source(K, c, lane):
    """(LDS byte, item code byte fetched) of load c, lane `lane`."""
    C = kcfg(K)
    q = c * 1024 + 16 * lane
    u, o = divmod(q, K // 2)
    s, r = divmod(o, C["kSeg"])
    slot = r // 16
    return q, u * (K // 2) + s * C["kSeg"] + (slot ^ (u % C["kPieces"])) * 16


def reader(K, lane, c):
    """(LDS byte read, item code byte wanted) of read c of lane `lane`."""
    C = kcfg(K)
    i4, blk = lane & 3, lane >> 2
    ug, ks = divmod(blk, C["NKS"])
    u = 4 * ug + i4
    o = ks * (C["KB"] // 2) + 16 * c
    s, r = divmod(o, C["kSeg"])
    piece = r // 16
    return u * (K // 2) + s * C["kSeg"] + (piece ^ (u % C["kPieces"])) * 16, u * (K // 2) + o


@pytest.mark.parametrize("K", KS)
def test_loads_fill_a_permutation_read_back_correctly(K):
    C = kcfg(K)
    assert C["kCode"] == 32 * C["KB"] and C["kCode"] % 1024 == 0 and C["kSB"] == 2 * C["KB"]
    lds = {}
    for c in range(C["kDma"]):
        for lane in range(64):
            q, src = dma_source(K, c, lane)
            assert 0 <= q < C["kCode"] and q not in lds
            lds[q] = src
    assert sorted(lds.values()) == list(range(0, C["kCode"], 16))
    for lane in range(64):
        for c in range(C["WPL"] // 4):
            at, want = reader(K, lane, c)
            assert lds[at] == want, (K, lane, c)


@pytest.mark.parametrize("K", [k for k in KS if k >= 512])
def test_lds_reads_are_conflict_free(K):
    C = kcfg(K)
    for c in range(C["WPL"] // 4):
        for q0 in range(0, 64, 16):
            slots = [(reader(K, lane, c)[0] % 256) // 16 for lane in range(q0, q0 + 16)]
            assert len(set(slots)) == 16, (K, c, q0, slots)


def kred_index(V, DTOP, lane, j):
    idx, c, d = j, V, DTOP
    while d >= 4 and c > 1:
        c //= 2
        if lane & d:
            idx += c
        d //= 2
    return idx


def kred_last(V, DTOP):
    c, last, d = V, 2 * DTOP, DTOP
    while d >= 4 and c > 1:
        c //= 2
        last = d
        d //= 2
    return max(last, 4)


@pytest.mark.parametrize("K", KS)
@pytest.mark.parametrize("pair", [True, False])
def test_lane_sum_leaves_each_total_in_one_writer(K, pair):
    C = kcfg(K)
    M = 2 if pair else 1
    V, DTOP = 4 * M, 2 * C["NKS"]
    CNT = 1 if C["NKS"] >= V else V // C["NKS"]
    last = kred_last(V, DTOP)
    seen = {}
    for lane in range(64):
        writer = (lane & (last - 1) & ~3) == 0
        ug = (lane >> 2) // C["NKS"]
        for j in range(CNT):
            idx = kred_index(V, DTOP, lane, j)
            if pair:
                if CNT > 1:
                    if j % 2:
                        continue
                    # the up total of the same output sits next to the gate
                    assert kred_index(V, DTOP, lane, j + 1) == idx + 1
                else:
                    partner = kred_index(V, DTOP, lane ^ last, 0)
                    assert partner == idx ^ 1
                    if idx % 2:
                        continue
            if writer:
                key = (4 * ug + idx // M, lane & 3)
                seen[key] = seen.get(key, 0) + 1
    assert seen == {(u, r): 1 for u in range(C["UPI"]) for r in range(4)}


def load_rows_range(K, row0, rows, lane, sorted_token):
    """(kept row, first element, end element) that `load_rows` of the 4-bit
    stream kernel reads for lane `lane` of a chunk starting at kept row
    row0 with `rows` rows, restated from the kernel: the lane's row i4 =
    lane % 4 (a lane past the chunk reads the chunk's first row and discards
    it), its K slice ks = (lane / 4) % NKS, and the 8-element words
    8w .. 8w+7 of that slice for w < KB / 8 -- one contiguous range."""
    C = kcfg(K)
    i4 = lane & 3
    ks = (lane >> 2) % C["NKS"]
    live = i4 < rows
    kr = row0 + (i4 if live else 0)
    src = sorted_token[kr] if sorted_token is not None else kr
    first = src * K + ks * C["KB"]
    return kr, ks, first, first + 8 * (C["KB"] // 8)


@pytest.mark.parametrize("K", KS)
@pytest.mark.parametrize("gather", [True, False])
def test_activation_rows_stay_in_their_buffer(K, gather):
    """Over random dispatch outcomes (offsets, sorted tokens), every chunk
    of every expert -- the chunks the kernel's items visit, row0 = offs[e] +
    4k < offs[e+1] -- reads only kept rows and, through them, only elements
    of x (T rows) or of H (the kept rows), and every K slice stays inside
    its row."""
    import random
    rnd = random.Random(K * 2 + gather)
    C = kcfg(K)
    for _ in range(10):
        E, T = rnd.randint(2, 40), rnd.randint(1, 300)
        counts = [rnd.randint(0, 12) for _ in range(E)]
        offs = [0]
        for c in counts:
            offs.append(offs[-1] + c)
        kept = offs[-1]
        st = [rnd.randrange(T) for _ in range(kept)] if gather else None
        nrows = T if gather else kept
        for e in range(E):
            for row0 in range(offs[e], offs[e + 1], 4):
                rows = min(4, offs[e + 1] - row0)
                for lane in range(64):
                    kr, ks, a, b = load_rows_range(K, row0, rows, lane, st)
                    assert offs[e] <= kr < offs[e + 1]
                    assert 0 <= a and b <= nrows * K
                    assert a // K == (b - 1) // K  # inside one row
                    assert a % K == ks * C["KB"] and b - a == C["KB"]


def stream_split(counts, NBW, W, item_cost=12, rows_max=4):
    """The 4-bit stream kernel's split of its items over W waves, restated
    from the kernel: the active experts (count > 0) in expert order with
    their first chunk p[a] and cost prefix c[a] (NBW * (chunks * item_cost +
    rows) per expert), and each wave's first item -- the first item whose
    cost prefix reaches wv * TC / W.  Returns the start items of waves
    0..W, and for every expert start_item lands in, the row count read from
    the offsets against the one its cost implies."""
    act = [(e, c) for e, c in enumerate(counts) if c > 0]
    p, cst = [0], [0]
    for _, c in act:
        ch = -(-c // rows_max)
        p.append(p[-1] + ch)
        cst.append(cst[-1] + NBW * (ch * item_cost + c))
    A, C, TC = len(act), p[-1], cst[-1]
    derived = {}

    def start(wv):
        x = wv * TC // W
        if x >= TC:
            return C * NBW
        lo, hi = 0, A - 1
        while lo < hi:
            mid = (lo + hi + 1) >> 1
            if cst[mid] <= x:
                lo = mid
            else:
                hi = mid - 1
        ch = p[lo + 1] - p[lo]
        cnt = act[lo][1]  # offsets[e + 1] - offsets[e]
        derived[lo] = (cst[lo + 1] - cst[lo]) // NBW - ch * item_cost
        full = NBW * (item_cost + rows_max)
        y = x - cst[lo]
        k = min(y // full, ch - 1)
        rows = min(rows_max, cnt - k * rows_max)
        rem = y - k * full
        b = (rem + item_cost + rows - 1) // (item_cost + rows)
        return (p[lo] + k) * NBW + b

    return [start(w) for w in range(W + 1)], derived, act, C


@pytest.mark.parametrize("NBW", [1, 4, 128])
def test_stream_split_partitions_the_items(NBW):
    """Over random routing outcomes, the waves' ranges are consecutive and
    cover every item (chunk, unit block) exactly once, and an expert's cost
    prefix difference is NBW * (chunks * item_cost + rows)."""
    import random
    rnd = random.Random(NBW)
    for _ in range(40):
        E = rnd.randint(1, 300)
        counts = [rnd.choice([0, 0, 1, 1, 2, 3, 4, 5, 9, 30]) for _ in range(E)]
        if sum(counts) == 0:
            counts[0] = 1
        W = rnd.choice([8, 64, 2048])
        starts, derived, act, C = stream_split(counts, NBW, W)
        assert starts[0] == 0 and starts[-1] == C * NBW
        assert all(a <= b for a, b in zip(starts, starts[1:]))
        for a, cnt in derived.items():
            assert cnt == act[a][1]
