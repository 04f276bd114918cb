"""Every global-memory access of the bf16 Newton-Schulz tile routine, checked
on the host (no GPU): the direct-to-LDS operand loads of every stage (the
clamped tail re-loads included) and the epilogue's combine-term loads and
predicated stores, for every tile of every product, in both operand layouts
(row-wise and k-major), at the five workloads' canonical shapes, ragged
shapes and the largest accepted dimension (65536).

The index arithmetic below restates the tile routine's, element for element:
the tile order (lower-triangle groups for the Gram and the square, row groups
for the apply), each lane's source row, chunk and swizzle, the stage offset,
and the epilogue's row/column mapping with its clamps. A load must lie inside
its operand buffer; a store that executes (its predicate holds) must lie
inside its output buffer, and every output element of the padded matrix must
be stored exactly once per tile grid (the mirrored tile included). The LDS
destinations of the loads must fill each stage buffer exactly.
"""

import numpy as np
import pytest

BM = BN = 256
BK = 32
NTHR = 512
RB = BK * 2          # bytes per LDS row of a contraction-contiguous operand
XR = BN * 2          # bytes per LDS row of a k-major operand
OPB = BM * RB        # bytes per operand per stage
NSTAGE = 4
TRI_GROUP = 4
APPLY_GROUP = 8

tid = np.arange(NTHR)
lane = tid & 63
w = tid >> 6


def swz(row):
    return (row >> 2) & 3


def xswz(k):
    return (k & 3) << 2


def tri_decode(k):
    i = int((np.sqrt(np.float32(8.0 * k + 1.0)) - np.float32(1.0)) * np.float32(0.5))
    while (i + 1) * (i + 2) // 2 <= k:
        i += 1
    while i * (i + 1) // 2 > k:
        i -= 1
    return i, k - i * (i + 1) // 2


def tri_decode_grouped(t, ntr):
    i, _ = tri_decode(t)
    r0 = (i // TRI_GROUP) * TRI_GROUP
    gsz = min(TRI_GROUP, ntr - r0)
    u = t - r0 * (r0 + 1) // 2
    if u < r0 * gsz:
        return r0 + u % gsz, u // gsz
    u -= r0 * gsz
    c = 0
    while u >= gsz - c:
        u -= gsz - c
        c += 1
    return r0 + c + u, r0 + c


def apply_decode(t, ntr, ntc):
    r0 = (t // (APPLY_GROUP * ntc)) * APPLY_GROUP
    gsz = min(APPLY_GROUP, ntr - r0)
    u = t - r0 * ntc
    return r0 + u % gsz, u // gsz


def operand_geometry(op, rp, cp):
    """(A buffer, B buffer, lda, ldb, K, limA, limB) in elements."""
    if op == "gram":
        return "X", "X", cp, cp, cp, rp, rp
    if op == "square":
        return "A", "A", rp, rp, rp, rp, rp
    return "B", "X", rp, cp, rp, rp, cp


def load_offsets(op, km, ti, tj, lda, ldb, limA, limB):
    """Element offsets of the four direct loads of stage 0 per thread, and the
    per-stage step of each (k-major operands advance by whole k-rows)."""
    if not km:
        d0 = 32 * w + (lane >> 2)
        d1 = d0 + 16
        c0, c1 = (lane & 3) ^ swz(d0), (lane & 3) ^ swz(d1)
        a0 = np.minimum(ti * BM + d0, limA - 1) * lda + c0 * 8
        a1 = np.minimum(ti * BM + d1, limA - 1) * lda + c1 * 8
        steps_a = (BK, BK)
        if op != "apply":
            b0 = np.minimum(tj * BN + d0, limB - 1) * ldb + c0 * 8
            b1 = np.minimum(tj * BN + d1, limB - 1) * ldb + c1 * 8
            steps_b = (BK, BK)
        else:
            x0 = 4 * w + (lane >> 5)
            x1 = x0 + 2
            xc0, xc1 = (lane & 31) ^ xswz(x0), (lane & 31) ^ xswz(x1)
            b0 = x0 * ldb + np.minimum(tj * BN + xc0 * 8, limB - 8)
            b1 = x1 * ldb + np.minimum(tj * BN + xc1 * 8, limB - 8)
            steps_b = (BK * ldb, BK * ldb)
    else:
        x0 = 4 * w + (lane >> 5)
        x1 = x0 + 2
        xc0, xc1 = (lane & 31) ^ xswz(x0), (lane & 31) ^ xswz(x1)
        a0 = x0 * lda + np.minimum(ti * BM + xc0 * 8, limA - 8)
        a1 = x1 * lda + np.minimum(ti * BM + xc1 * 8, limA - 8)
        b0 = x0 * ldb + np.minimum(tj * BN + xc0 * 8, limB - 8)
        b1 = x1 * ldb + np.minimum(tj * BN + xc1 * 8, limB - 8)
        steps_a = (BK * lda, BK * lda)
        steps_b = (BK * ldb, BK * ldb)
    return (a0, a1, b0, b1), steps_a + steps_b


def lds_destinations(km, op):
    """LDS byte offsets (within one stage's operand buffer) that the two load
    instructions of each operand write, per thread (16 bytes each)."""
    dlds = w * 32 * RB
    first = dlds + 16 * lane
    second_a = first + (16 * RB if not km else 2 * XR)
    second_b = first + (2 * XR if (km or op == "apply") else 16 * RB)
    return first, second_a, second_b


def epilogue_accesses(op, ti, tj, rp, cp):
    """(element offset, executes) of every 4-element store of the tile, and
    the offsets of the combine-term loads (always executed, clamped)."""
    if op == "apply":
        ldo, limR, limC = cp, rp, cp
    else:
        ldo, limR, limC = rp, rp, rp
    wr, wc = w >> 2, w & 3
    stores, loads = [], []
    if op != "apply" and ti != tj:
        for i in range(4):
            for j in range(2):
                for g in range(4):
                    gr = tj * BN + wc * 64 + j * 32 + (lane & 31)
                    gc = ti * BM + wr * 128 + i * 32 + 8 * g + 4 * (lane >> 5)
                    ok = (gr < limR) & (gc < limC)
                    go = np.minimum(gr, limR - 1) * ldo + np.minimum(gc, limC - 4)
                    stores.append((go, ok, gr, gc))
                    if op == "square":
                        loads.append(go)
    per = (64 * BN // 4) // NTHR
    for p in range(4):
        for it in range(per):
            q = tid + NTHR * it
            sr = q >> 6
            cc = (q & 63) * 4
            gr = ti * BM + (sr >> 5) * 128 + p * 32 + (sr & 31)
            gc = tj * BN + cc
            ok = (gr < limR) & (gc < limC)
            go = np.minimum(gr, limR - 1) * ldo + np.minimum(gc, limC - 4)
            stores.append((go, ok, gr, gc))
            if op != "gram":
                loads.append(go)
    return stores, loads, ldo, limR, limC


def check_shape(r, c, layouts=(False, True)):
    rp, cp = -(-r // 128) * 128, -(-c // 128) * 128
    sizes = {"X": rp * cp, "A": rp * rp, "B": rp * rp}
    ntr, ntc = -(-rp // BM), -(-cp // BN)
    for op in ("gram", "square", "apply"):
        Ab, Bb, lda, ldb, K, limA, limB = operand_geometry(op, rp, cp)
        assert K % (BK * NSTAGE) == 0         # the main loop is unrolled by four stages
        nk = K // BK
        ntile = ntr * (ntr + 1) // 2 if op != "apply" else ntr * ntc
        seen = set()
        out_cover = np.zeros((rp, rp if op != "apply" else cp), dtype=np.int32)
        for km in ((False,) if op == "gram" else layouts):
            for t in range(ntile):
                ti, tj = apply_decode(t, ntr, ntc) if op == "apply" else tri_decode_grouped(t, ntr)
                assert 0 <= tj < (ntc if op == "apply" else ti + 1) and 0 <= ti < ntr
                if not km:
                    seen.add((ti, tj))
                offs, steps = load_offsets(op, km, ti, tj, lda, ldb, limA, limB)
                for o, st, buf in zip(offs, steps, (Ab, Ab, Bb, Bb)):
                    # stages 0 .. nk + 2 read stage min(s, nk - 1): the extremes
                    # are stage 0 and stage nk - 1
                    lo, hi = o.min(), o.max() + (nk - 1) * st
                    assert lo >= 0 and hi + 8 <= sizes[buf], (op, km, rp, cp, t)
                stores, loads, ldo, limR, limC = epilogue_accesses(op, ti, tj, rp, cp)
                obuf = {"gram": "A", "square": "B", "apply": "X"}[op]
                for go in loads:
                    assert go.min() >= 0 and go.max() + 4 <= sizes["A" if op == "square" else "X"]
                if not km:
                    for go, ok, gr, gc in stores:
                        g = go[ok]
                        assert g.size == 0 or (g.min() >= 0 and g.max() + 4 <= sizes[obuf])
                        for u in range(4):
                            np.add.at(out_cover, (gr[ok], gc[ok] + u), 1)
        expect = ({(i, j) for i in range(ntr) for j in range(i + 1)} if op != "apply"
                  else {(i, j) for i in range(ntr) for j in range(ntc)})
        assert seen == expect, (op, rp, cp)
        # every element of the padded output is stored by exactly one tile
        assert (out_cover == 1).all(), (op, rp, cp, int(out_cover.min()), int(out_cover.max()))


def test_lds_destinations_fill_each_stage_buffer():
    for km in (False, True):
        for op in ("gram", "square", "apply"):
            if op == "gram" and km:
                continue
            first, second_a, second_b = lds_destinations(km, op)
            for second in (second_a, second_b):
                bytes_ = np.concatenate([(first[:, None] + np.arange(16)).ravel(),
                                         (second[:, None] + np.arange(16)).ravel()])
                assert sorted(bytes_.tolist()) == list(range(OPB)), (km, op)


SHAPES = [(1, 1), (7, 3), (200, 300), (129, 1000), (384, 128), (768, 768), (768, 3072), (1408, 2048),
          (2304, 2560), (1024, 4096)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_tile_accesses_in_bounds(shape):
    check_shape(min(shape), max(shape))


@pytest.mark.parametrize("shape", [(4096, 4096), (4096, 14336), (8192, 8192), (8192, 28672), (129, 65536),
                                   (1000, 65536)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_tile_accesses_in_bounds_large(shape):
    """The large workload shapes and the 65536 edge: loads and store
    predicates (the coverage count is skipped above 64 M elements)."""
    r, c = shape
    rp, cp = -(-r // 128) * 128, -(-c // 128) * 128
    sizes = {"X": rp * cp, "A": rp * rp, "B": rp * rp}
    ntr, ntc = -(-rp // BM), -(-cp // BN)
    for op in ("gram", "square", "apply"):
        Ab, Bb, lda, ldb, K, limA, limB = operand_geometry(op, rp, cp)
        nk = K // BK
        ntile = ntr * (ntr + 1) // 2 if op != "apply" else ntr * ntc
        # the extreme tiles of each block row and column bound every access
        tiles = range(ntile) if ntile <= 600 else sorted({0, ntile - 1, *range(0, ntile, max(1, ntile // 300))})
        for km in ((False,) if op == "gram" else (False, True)):
            for t in tiles:
                ti, tj = apply_decode(t, ntr, ntc) if op == "apply" else tri_decode_grouped(t, ntr)
                offs, steps = load_offsets(op, km, ti, tj, lda, ldb, limA, limB)
                for o, st, buf in zip(offs, steps, (Ab, Ab, Bb, Bb)):
                    assert o.min() >= 0 and o.max() + (nk - 1) * st + 8 <= sizes[buf]
                stores, loads, _, _, _ = epilogue_accesses(op, ti, tj, rp, cp)
                obuf = {"gram": "A", "square": "B", "apply": "X"}[op]
                for go in loads:
                    assert go.min() >= 0 and go.max() + 4 <= sizes["A" if op == "square" else "X"]
                for go, ok, _, _ in stores:
                    g = go[ok]
                    assert g.size == 0 or (g.min() >= 0 and g.max() + 4 <= sizes[obuf])
        # the last tile's corner: the largest offsets of the tile grid
        assert max(rp, cp) <= 65536 and rp * cp < 2 ** 31
