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
