"""The GPU parity bars, checked on the host against an emulation of the bf16
Newton-Schulz chain and against planted mistakes.

The emulation stores X, A and B in bf16 (round to nearest even) and sums
their products in fp32 (numpy's float32 matrix product), as the matrix-core
path does; it is test scaffolding for the bars, not a reference for any
expected value. The localized bars of ``check_local`` must admit it with
margin at ragged and workload shapes, and must reject a wrong row, a wrong
tile and a single wrong element that the Frobenius bar alone lets through.
"""
import numpy as np
import pytest

from oracle import muon as omuon
from tests.gpu_helpers import bf16_ulps, check_local


def bf16(x):
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)


def ns_bf16_chain(Q, steps=5, coeffs=(3.4445, -4.7750, 2.0315), eps=1e-7):
    tall = Q.shape[0] > Q.shape[1]
    X = bf16((Q.T if tall else Q).astype(np.float32))
    sig = np.float32(1.0 / (np.sqrt(np.sum(X.astype(np.float64) ** 2)) + eps))
    a, b, c = (np.float32(v) for v in coeffs)
    for it in range(steps):
        s2, s1 = (sig * sig, sig) if it == 0 else (np.float32(1), np.float32(1))
        A = bf16(s2 * (X @ X.T))
        B = bf16(b * A + c * (A @ A))
        X = bf16(s1 * (a * X + B @ X))
    return (X.T if tall else X).astype(np.float64)


CASES = [(7, 3), (300, 200), (129, 1000), (768, 768), (3072, 768), (1408, 2048)]


@pytest.fixture(scope="module")
def chains():
    r = np.random.default_rng(5)
    out = {}
    for shape in CASES:
        Q = bf16(r.standard_normal(shape).astype(np.float32)).astype(np.float64)
        out[shape] = (ns_bf16_chain(Q), omuon.newton_schulz(Q))
    return out


@pytest.mark.parametrize("shape", CASES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_bars_admit_a_bf16_chain_with_margin(chains, shape):
    got, want = chains[shape]
    check_local(got, want, 2e-2, shape)
    # and with room: the localized bars hold at half their width (the
    # Frobenius bar is the brief's and is kept as it is)
    d = got - want
    fro = np.linalg.norm(want)
    m, n = want.shape
    rms = fro / np.sqrt(want.size)
    assert np.linalg.norm(d, axis=1).max() / (fro / np.sqrt(m)) < 0.5 * 3 * 2e-2
    assert np.linalg.norm(d, axis=0).max() / (fro / np.sqrt(n)) < 0.5 * 3 * 2e-2
    assert (np.abs(d) / (rms + np.abs(want))).max() < 0.5 * 6 * 2e-2


def test_bars_admit_gradient_outliers():
    """1% of the input x100 (the Llama workload's gradients): the update has
    spikes of tens of RMS there, and the element bar scales with them."""
    r = np.random.default_rng(6)
    Q = r.standard_normal((1024, 4096))
    Q[r.random(Q.shape) < 0.01] *= 100
    Q = bf16(Q.astype(np.float32)).astype(np.float64)
    check_local(ns_bf16_chain(Q), omuon.newton_schulz(Q), 2e-2)


def test_bars_reject_localized_mistakes(chains):
    got, want = chains[(768, 768)]
    bad_row = got.copy()
    bad_row[100] *= 0.6                         # one row 40% short
    assert np.linalg.norm(bad_row - want) / np.linalg.norm(want) < 2e-2   # the Frobenius bar alone passes
    with pytest.raises(AssertionError):
        check_local(bad_row, want, 2e-2)
    mild_row = got.copy()
    mild_row[100] *= 1.08                       # 8% off: within the element bar, not the row bar
    with pytest.raises(AssertionError, match="'row'"):
        check_local(mild_row, want, 2e-2)
    got, want = chains[(1408, 2048)]
    bad_tile = got.copy()
    bad_tile[256:512, 512:768] *= 1.10          # one 256x256 tile 10% off
    assert np.linalg.norm(bad_tile - want) / np.linalg.norm(want) < 2e-2
    with pytest.raises(AssertionError):
        check_local(bad_tile, want, 2e-2)
    bad_elem = got.copy()
    bad_elem[7, 9] = -want[7, 9]                # one element with its sign flipped
    with pytest.raises(AssertionError, match="element"):
        check_local(bad_elem, want, 2e-2)


def test_ulp_distance():
    assert bf16_ulps([0x3F80], [0x3F81]).tolist() == [1]
    assert bf16_ulps([0x0000], [0x8000]).tolist() == [0]          # +0 and -0
    assert bf16_ulps([0x0001], [0x8001]).tolist() == [2]          # across zero
    assert bf16_ulps([0xBF80], [0xBF82]).tolist() == [2]
