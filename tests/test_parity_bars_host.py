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


# ---------------------------------------------------------------------------
# check_update: the cautious masks
# ---------------------------------------------------------------------------
def _update_case(cautious, param_dtype="f32", seed=12):
    """A 300 x 200 step: the oracle's result, the same step taken with the
    bf16 chain's U and with U to fp32 precision (relative noise 1e-7)."""
    from oracle import storage
    r = np.random.default_rng(seed)
    m, n, lr, wd = 300, 200, 0.02, 0.1
    W0 = storage.decode(storage.round_to(r.standard_normal((m, n)) * 0.02, param_dtype), param_dtype)
    G = r.standard_normal((m, n)) * 1e-3
    Q = bf16(G.astype(np.float32)).astype(np.float64)
    U, U_chain = omuon.newton_schulz(Q), ns_bf16_chain(Q)
    U_f32 = U * (1.0 + 1e-7 * r.standard_normal(U.shape))
    s = omuon.shape_scale(m, n)

    def step(Ud):
        if cautious == "wd_mask":
            return omuon.apply_cautious_wd(W0, Ud, lr, wd, s)
        return omuon.apply_cautious_wrapper(W0, Ud, G, lr, wd, s)[0]

    rnd = lambda x: storage.decode(storage.round_to(x, param_dtype), param_dtype)
    return dict(W0=W0, G=G, U=U, h={"cautious": cautious}, lr=lr, wd=wd, s=s, want=step(U), chain=rnd(step(U_chain)),
                near_exact=rnd(step(U_f32)), rnd=rnd)


@pytest.mark.parametrize("cautious,pd", [("wd_mask", "f32"), ("wd_mask", "bf16"), ("wrapper", "f32"),
                                         ("wrapper", "bf16")])
def test_update_check_admits_the_bf16_chain_and_rejects_mask_mistakes(cautious, pd):
    """At the bf16 Newton-Schulz bars the step taken with the bf16 chain's
    update passes. At the fp32 bars (1e-5) the step taken with U to fp32
    precision passes, and the same step with the mask inverted, with no mask,
    or with 5% of the decisions turned over fails. (At the bf16 bars the
    weight-decay mask is not visible: it moves an element by lr wd W, about
    3% of the update's RMS here, as much as a 2e-2 error of U moves it.)"""
    from tests.gpu_helpers import check_update
    c = _update_case(cautious, pd)
    W0, U, G, lr, wd, s = c["W0"], c["U"], c["G"], c["lr"], c["wd"], c["s"]
    common = (W0, c["want"], G, U, c["h"], lr, wd, s, pd)
    check_update(c["chain"], *common, 6e-2 if pd == "bf16" else 4e-2, 2e-2)
    check_update(c["near_exact"], *common, 1e-5, 1e-5)
    # the other branch everywhere: decay where U W < 0 (the mask keeps it where
    # U W >= 0); the update where it opposes the gradient (the wrapper keeps
    # it where (W - W_new) G > 0)
    if cautious == "wd_mask":
        inverted = W0 - lr * s * U - lr * wd * np.where((U * W0) >= 0.0, 0.0, W0)
    else:
        delta = lr * wd * W0 + lr * s * U
        inverted = np.where((delta * G) > 0.0, W0, W0 - delta)
    plain = omuon.apply_decoupled(W0, U, lr, wd, s)
    turned = c["want"].copy()
    pick = np.random.default_rng(3).random(turned.shape) < 0.05
    turned[pick] = inverted[pick]
    for name, bad in (("inverted", inverted), ("no mask", plain), ("5% turned", turned)):
        with pytest.raises(AssertionError):
            check_update(c["rnd"](bad), *common, 1e-5, 1e-5)
            pytest.fail(f"{name} passed")
