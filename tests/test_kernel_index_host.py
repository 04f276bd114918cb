"""Index schemes of the elementwise reduction kernels, checked on the host.

The canonical row sum (the NorMuon and Muon+ reductions) reads a row of c
elements as whole 16-byte vectors of V elements (V = 8 for bf16, 4 for fp32),
four per lane and round, then a scalar tail. This enumerates what every lane
of the wave reads, for ragged and workload row lengths: each element of the
row exactly once, nothing at or past c, and the weights (one per element) from
the same indices.

It also restates the arithmetic of the normalisation pass's overflow guard.
"""
import numpy as np
import pytest


def rowsum_reads(c, V, R=4, lanes=64):
    nv = c // V
    seen = []
    for lane in range(lanes):
        for v0 in range(lane, nv, R * lanes):
            for u in range(R):
                v = v0 + lanes * u
                if v < nv:
                    seen.extend(range(v * V, v * V + V))
        seen.extend(range(nv * V + lane, c, lanes))
    return seen


@pytest.mark.parametrize("V", [4, 8])
@pytest.mark.parametrize("c", [1, 3, 7, 8, 9, 100, 129, 255, 256, 257, 768, 1000, 1408, 2048, 3072, 4096,
                               14336, 28672, 65536])
def test_rowsum_reads_each_element_once(c, V):
    seen = rowsum_reads(c, V)
    assert sorted(seen) == list(range(c))



# ---------------------------------------------------------------------------
# The first-Gram overflow guard of the normalisation pass. With n = ||Q||_F
# (summed in fp64) at or above 2^60, X0 is scaled by 2^-k with
# k = ilogb(n) - 30 and sigma = 2^k / (n * s + eps) is stored instead of
# 1 / (n * s + eps). Restated here in fp64/fp32 numpy: for every finite Q the
# scaled norm lies in [2^30, 2^31), so the fp32 sums of the first Gram (at most
# the squared norm) stay below 2^62; 2^-k is a normal float; and sigma times
# the scaled X0 is the same normalised X as before.
# ---------------------------------------------------------------------------
def guard(norm, scale=1.0, eps=1e-7):
    k = 0
    if np.isfinite(norm) and norm >= 2.0 ** 60:
        k = int(np.frexp(norm)[1] - 1) - 30          # ilogb
    sigma = np.float32(np.ldexp(1.0 / (norm * scale + eps), k))
    return k, sigma, np.float32(np.ldexp(1.0, -k))


def test_guard_keeps_the_first_gram_in_range():
    fmax = float(np.finfo(np.float32).max)
    # the largest norm of a finite fp32 matrix the planner accepts (2^31 elements)
    top = fmax * np.sqrt(2.0 ** 31)
    for norm in np.geomspace(2.0 ** 60, top, 2000).tolist() + [2.0 ** 60, top]:
        k, sigma, f = guard(norm)
        assert k > 0
        scaled = norm * 2.0 ** -k
        assert 2.0 ** 30 <= scaled < 2.0 ** 31
        assert scaled ** 2 < 2.0 ** 127
        assert f == np.float32(2.0 ** -k) and f >= np.finfo(np.float32).tiny
        assert np.isfinite(sigma) and sigma > 0
        # the normalised X is unchanged: sigma * (2^-k Q) = Q / (n + eps)
        assert abs(float(sigma) * scaled - norm / (norm + 1e-7)) < 2 ** -23


def test_guard_is_idle_below_its_threshold():
    for norm in (0.0, 1e-30, 1e-3, 1.0, 1e10, 2.0 ** 60 * (1 - 2 ** -52)):
        k, sigma, f = guard(norm)
        assert k == 0 and f == 1.0
        assert sigma == np.float32(1.0 / (norm + 1e-7))
    # below the threshold the unscaled Gram is in range: sums at most 2^120
    assert (2.0 ** 60) ** 2 < 2.0 ** 127

