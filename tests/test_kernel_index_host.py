"""Index schemes of the elementwise reduction kernels, checked on the host.

The canonical row sum (the NorMuon and Muon+ reductions) reads a row of c
elements as whole 16-byte vectors of V elements (V = 8 for bf16, 4 for fp32),
four per lane and round, then a scalar tail. This enumerates what every lane
of the wave reads, for ragged and workload row lengths: each element of the
row exactly once, nothing at or past c, and the weights (one per element) from
the same indices.
"""
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

