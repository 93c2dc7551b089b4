"""Host-side check of the index scheme of the tiled 4-bit grouped GEMM
(the U4 variant of grouped_gemm_kernel in csrc/gemm_bf16.hip), restated from
the kernel's formulas for one 256 x 256 tile and every K step:

  * every direct load (codes: 16 bytes per lane; scale and bias: one dword
    per lane) stays inside the byte range its buffer descriptor carries;
  * the LDS bytes the fragment readers use are exactly those the loads
    wrote, so no reader sees a stale or foreign byte;
  * the weight a lane dequantises for (sub-step, element) is the element of
    its output row at the same K index as the activation element the lane
    pairs it with, so the permuted order of K chunks is the same
    permutation on both operands and the MFMA sums every K index once;
  * the dword that holds a row's scale for a K step holds that row's
    scale (the bf16 half selected by the step's parity), with an even
    number of groups per row.
The GPU parity tests check the kernel itself; this pins the scheme."""
import pytest

BN, BK, WAVES = 256, 64, 8
Q_CODE = BN * 32  # code bytes per stage


def tile_rows(mode, nt, N):
    """Output row n (of the expert's weight matrix) and matrix (0 gate /
    in / down, 1 up) of each of the 256 tile rows, clamped like the kernel."""
    out = []
    for r in range(BN):
        if mode == "swiglu":
            n, m = nt * (BN // 2) + (r & 127), 1 if r >= 128 else 0
        else:
            n, m = nt * BN + r, 0
        out.append((min(n, N - 1), m))
    return out


def code_loads(mode, nt, N, K, step):
    """(LDS byte, matrix, global byte in that matrix) of every code byte
    the 8 waves load for K step `step`."""
    rows = tile_rows(mode, nt, N)
    res = []
    for w in range(WAVES):
        for lane in range(64):
            rq = w * 32 + (lane >> 1)
            n, m = rows[rq]
            voff = n * (K // 2) + (lane & 1) * 16
            g = voff + step * 32
            for b in range(16):
                res.append((w * 1024 + lane * 16 + b, m, g + b))
    return res


def sb_loads(mode, nt, N, K, step):
    """(LDS byte, matrix, scale-or-bias, global byte) of the scale/bias
    dwords loaded for K step `step`."""
    G = K // 64
    rows = tile_rows(mode, nt, N)
    res = []
    for w in range(WAVES):
        for lane in range(64):
            rs = (w & 3) * 64 + lane
            n, m = rows[rs]
            kind = "s" if w < 4 else "b"
            voff = n * G * 2
            g = voff + (step >> 1) * 4
            lds = Q_CODE + (w >> 2) * (BN * 4) + (w & 3) * 256 + lane * 4
            for b in range(4):
                res.append((lds + b, m, kind, g + b))
    return res


def wrow(mode, wn, nb, fr):
    return ((128 if nb else 0) + wn * 32 + fr) if mode == "swiglu" else wn * 64 + nb * 32 + fr


CASES = [("swiglu", 0, 512, 256), ("swiglu", 3, 448, 640), ("down", 1, 700, 384),
         ("relu", 0, 200, 128), ("down", 0, 2048, 2048)]


@pytest.mark.parametrize("mode,nt,N,K", CASES)
def test_loads_in_range_and_cover_the_readers(mode, nt, N, K):
    G = K // 64
    assert G % 2 == 0
    code_bytes, sb_bytes = N * (K // 2), N * G * 2
    for step in range(K // BK):
        lds_code = {}
        for lds, m, gb in code_loads(mode, nt, N, K, step):
            assert 0 <= gb < code_bytes
            assert lds not in lds_code
            lds_code[lds] = (m, gb)
        lds_sb = {}
        for lds, m, kind, gb in sb_loads(mode, nt, N, K, step):
            assert 0 <= gb < sb_bytes
            assert lds not in lds_sb
            lds_sb[lds] = (m, kind, gb)
        rows = tile_rows(mode, nt, N)
        for wn in range(4):
            for nb in range(2):
                for lane in range(64):
                    fr, fh = lane & 31, lane >> 5
                    r = wrow(mode, wn, nb, fr)
                    n, m = rows[r]
                    for ks in range(4):
                        # the reader's 4-byte code word of sub-step ks
                        for b in range(4):
                            lds = r * 32 + fh * 16 + ks * 4 + b
                            assert lds_code[lds][0] == m
                            gb = lds_code[lds][1]
                            # byte b of word ks holds elements 2b, 2b+1 of the
                            # reader's K chunk 4*fh + ks of this step
                            elem = (gb - n * (K // 2)) * 2
                            assert gb // (K // 2) == n
                            chunk = fh * 4 + ks
                            assert elem == step * BK + chunk * 8 + 2 * b
                    # scale and bias dwords: the row's element n*G + step
                    for kind, base in (("s", Q_CODE), ("b", Q_CODE + BN * 4)):
                        gbs = [lds_sb[base + r * 4 + b] for b in range(4)]
                        assert all(x[0] == m and x[1] == kind for x in gbs)
                        first = gbs[0][2]
                        assert first % 4 == 0
                        half = step & 1
                        assert first // 2 + half == n * G + step


@pytest.mark.parametrize("fh", [0, 1])
def test_activation_chunks_pair_with_weight_chunks(fh):
    """The activation fragment of sub-step ks, lane half fh reads K chunk
    4*fh + ks (8 elements); the weight fragment of the same lane half and
    sub-step dequantises word ks of the lane's 16 code bytes, i.e. the same
    chunk.  Over the 4 sub-steps and both halves each chunk is used once."""
    seen = []
    for ks in range(4):
        a_chunk = fh * 4 + ks
        w_chunk = fh * 4 + ks  # word ks of piece fh
        assert a_chunk == w_chunk
        seen.append(a_chunk)
    other = [(1 - fh) * 4 + ks for ks in range(4)]
    assert sorted(seen + other) == list(range(8))
