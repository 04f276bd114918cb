"""Pins of the fp64 oracle against what the pages and the mathematics fix.

CPU only. Each check is written so that a plausible slip in the oracle (a
dropped term, a wrong sign or index, a transposed operand) fails at least one of
them; ``test_oracle_mutations.py`` plants such slips and asserts they are
caught. Expected values come from closed forms derived here, the SVD reduction
of the Newton-Schulz iteration (a textbook identity computed with
numpy.linalg.svd), invariants the pages state, and brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import adamw as oadamw
from oracle import muon as omuon
from oracle import storage

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")
with open(GOLDEN) as f:
    PAGE = json.load(f)
A, B, C = PAGE["ns_coeffs"]["value"]
STEPS = PAGE["ns_steps"]["value"]
EPS = PAGE["ns_eps"]["value"]


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Newton-Schulz through the SVD: X = U S V^T  =>  X X^T = U S^2 U^T, and each
# iteration maps every singular value x to phi(x) = a x + b x^3 + c x^5 while
# keeping the singular vectors. This route shares nothing with the oracle's
# matrix iteration.
# ---------------------------------------------------------------------------
def phi_iter(x, steps=STEPS, coeffs=(A, B, C)):
    a, b, c = coeffs
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def ns_by_svd(X, steps=STEPS, eps=EPS):
    U, S, Vt = np.linalg.svd(np.asarray(X, dtype=np.float64), full_matrices=False)
    fro = math.sqrt(float(np.sum(S * S)))
    return (U * phi_iter(S / (fro + eps), steps)) @ Vt


def check_ns_svd(ns=None):
    ns = ns or omuon.newton_schulz
    r = rng(11)
    for shape in [(4, 3), (3, 4), (5, 5), (6, 2), (2, 7), (1, 5), (8, 8)]:
        X = r.standard_normal(shape)
        got = ns(X)
        want = ns_by_svd(X)
        err = np.linalg.norm(got - want) / np.linalg.norm(want)
        assert err < 1e-11, (shape, err)
    # a small-norm input makes the eps term visible
    X = 1e-4 * r.standard_normal((4, 3))
    got, want = ns(X), ns_by_svd(X)
    assert np.linalg.norm(got - want) / np.linalg.norm(want) < 1e-11


def test_ns_matches_svd_reduction():
    check_ns_svd()


def test_ns_scalar_constants():
    # rank-1 input: the single normalised singular value is 1/(1+eps/||X||) ~ 1
    assert abs(phi_iter(1.0) - 0.6964364094697522) < 1e-15
    u = rng(1).standard_normal(6)
    v = rng(2).standard_normal(4)
    X = np.outer(u, v)
    got = omuon.newton_schulz(X)
    nrm = np.linalg.norm(X)
    want = phi_iter(nrm / (nrm + EPS)) * X / nrm
    assert np.abs(got - want).max() < 1e-13
    # 4x3 with orthonormal columns: every normalised singular value is 1/sqrt(3)
    Q, _ = np.linalg.qr(rng(3).standard_normal((4, 3)))
    got = omuon.newton_schulz(Q)
    f = phi_iter((1 / math.sqrt(3)) * math.sqrt(3) / (math.sqrt(3) + EPS))
    assert abs(f - 0.6857849207555402) < 1e-6
    assert np.abs(got - f * Q).max() < 1e-13
    # 5x2 with orthonormal columns (tall, transposed inside): both normalised
    # singular values are 1/sqrt(2)
    Q, _ = np.linalg.qr(rng(4).standard_normal((5, 2)))
    f = phi_iter(math.sqrt(2) / (math.sqrt(2) + EPS) / math.sqrt(2))
    assert abs(f - 1.1081111156829304) < 1e-6
    assert np.abs(omuon.newton_schulz(Q) - f * Q).max() < 1e-13
    # 4x4 orthogonal (square, not transposed): every normalised singular value
    # is 1/2
    Q, _ = np.linalg.qr(rng(6).standard_normal((4, 4)))
    f = phi_iter(2.0 / (2.0 + EPS) / 2.0)
    assert abs(f - 0.7654385304543396) < 1e-6
    assert np.abs(omuon.newton_schulz(Q) - f * Q).max() < 1e-13


def check_ns_equivariance(ns=None, trials=60):
    """NS(P X Q) = P NS(X) Q for orthogonal P and Q: the iteration is a
    polynomial in X X^T applied to X, so it commutes with rotations on both
    sides (the Frobenius norm is rotation-invariant too). Random shapes from
    1 x 1 to 12 x 12, square, wide and tall."""
    ns = ns or omuon.newton_schulz
    r = rng(41)
    for _ in range(trials):
        m, n = int(r.integers(1, 13)), int(r.integers(1, 13))
        X = r.standard_normal((m, n))
        P, _ = np.linalg.qr(r.standard_normal((m, m)))
        Q, _ = np.linalg.qr(r.standard_normal((n, n)))
        want = P @ ns(X) @ Q
        got = ns(P @ X @ Q)
        assert np.abs(got - want).max() < 1e-12 * max(1.0, np.abs(want).max()), (m, n)


def test_ns_orthogonal_equivariance():
    check_ns_equivariance()


def test_ns_scale_invariance():
    """NS(c X) = NS(X) up to the eps term: with ||X||_F ~ 10 and c from 1e-2 to
    1e6, the normalised inputs differ by at most eps / (c ||X||) relative."""
    r = rng(42)
    for shape in [(5, 3), (3, 5), (6, 6), (1, 7)]:
        X = r.standard_normal(shape) * 4
        base = omuon.newton_schulz(X * 1e6)        # eps negligible
        for c in [1e-2, 1.0, 1e3]:
            got = omuon.newton_schulz(X * c)
            bound = 50 * EPS / (c * np.linalg.norm(X))   # the eps term, amplified by at most ~phi'(x)^5
            assert np.abs(got - base).max() <= bound + 1e-13, (shape, c)


def test_ns_transpose_symmetry():
    r = rng(5)
    for shape in [(7, 3), (3, 7), (16, 48)]:
        X = r.standard_normal(shape)
        assert np.array_equal(omuon.newton_schulz(X.T), omuon.newton_schulz(X).T)
    X = r.standard_normal((9, 9))
    d = np.abs(omuon.newton_schulz(X.T) - omuon.newton_schulz(X).T).max()
    assert d < 1e-13


def test_ns_zero_stays_finite():
    for shape in [(4, 3), (3, 4), (16, 16)]:
        out = omuon.newton_schulz(np.zeros(shape))
        assert np.all(np.isfinite(out)) and np.all(out == 0.0)


def test_ns_output_band():
    # well-conditioned inputs: normalised singular values >= 1.5e-3 land in
    # phi^5's band; the band's ends are checked on a dense grid first
    grid = np.linspace(1.5e-3, 1.0, 200001)
    y = phi_iter(grid)
    assert y.min() > 0.679 and y.max() < 1.2025
    r = rng(7)
    U, _ = np.linalg.qr(r.standard_normal((256, 128)))
    V, _ = np.linalg.qr(r.standard_normal((128, 128)))
    S = np.geomspace(1.0, 0.1, 128)          # condition number 10
    X = (U * S) @ V.T
    sv = np.linalg.svd(omuon.newton_schulz(X), compute_uv=False)
    assert sv.min() > 0.679 and sv.max() < 1.2025
    G = r.standard_normal((96, 384))           # Gaussian, aspect 4: well conditioned
    sv = np.linalg.svd(omuon.newton_schulz(G), compute_uv=False)
    assert sv.min() > 0.679 and sv.max() < 1.2025


# ---------------------------------------------------------------------------
# Whole-matrix closed forms from zero momentum (beta 0.95, lr 0.02, wd 0.1)
# ---------------------------------------------------------------------------
HP = {"beta": 0.95, "nesterov": True}


def check_first_step(step_fn=None):
    step_fn = step_fn or omuon.muon_tensor_step
    r = rng(0)
    for (m, n, s) in [(256, 128, math.sqrt(2.0)), (64, 96, 1.0), (96, 64, math.sqrt(1.5)),
                      (40, 40, 1.0)]:
        G = r.standard_normal((1, m, n))
        W = 0.02 * r.standard_normal((1, m, n))
        Bm = np.zeros((1, m, n))
        W1, B1, _, _ = step_fn(W, G, Bm, None, 1, HP, 0.02, 0.1)
        assert np.abs(B1 - 0.05 * G).max() <= 1e-16 * np.abs(G).max() * 4
        U = ns_by_svd(0.0975 * G[0])
        want = 0.998 * W[0] - 0.02 * s * U
        err = np.abs(W1[0] - want).max()
        assert err < 1e-14, (m, n, err)


def test_first_step_closed_form():
    check_first_step()


def check_second_step(step_fn=None):
    step_fn = step_fn or omuon.muon_tensor_step
    r = rng(1)
    m, n = 48, 80
    G1 = r.standard_normal((1, m, n))
    G2 = r.standard_normal((1, m, n))
    W0 = 0.02 * r.standard_normal((1, m, n))
    W1, B1, _, _ = step_fn(W0, G1, np.zeros((1, m, n)), None, 1, HP, 0.02, 0.1)
    W2, B2, _, _ = step_fn(W1, G2, B1, None, 1, HP, 0.02, 0.1)
    assert np.abs(B2 - (0.0475 * G1 + 0.05 * G2)).max() < 1e-15
    Q2 = 0.045125 * G1[0] + 0.0975 * G2[0]
    want = 0.998 * W1[0] - 0.02 * ns_by_svd(Q2)
    assert np.abs(W2[0] - want).max() < 1e-14


def test_second_step_closed_form():
    check_second_step()


def test_muon_steps_match_torch_optim_muon():
    """Three steps of the oracle's plain Muon on a wide and a tall matrix against
    torch.optim.Muon in float64, with torch's Newton-Schulz call (bf16, and a
    clamped norm instead of norm + eps) swapped for the SVD closed form of the
    quintic iteration: the momentum, the Nesterov lerp, the shape scale and the
    decoupled decay then come from the library."""
    import torch.optim._muon as tmuon
    r = rng(23)
    shapes = [(48, 80), (96, 32)]
    lr, wd = 0.02, 0.1
    Ws = [0.02 * r.standard_normal(s) for s in shapes]
    Bs = [np.zeros((1,) + s) for s in shapes]
    tps = [torch.nn.Parameter(torch.from_numpy(W.copy())) for W in Ws]
    orig = tmuon._zeropower_via_newtonschulz
    tmuon._zeropower_via_newtonschulz = lambda g, coeffs, steps, eps: torch.from_numpy(
        ns_by_svd(g.numpy(), steps, eps))
    try:
        opt = torch.optim.Muon(tps, lr=lr, weight_decay=wd, momentum=0.95, nesterov=True, ns_steps=STEPS,
                               eps=EPS)
        for _ in range(3):
            Gs = [r.standard_normal(s) for s in shapes]
            for tp, G in zip(tps, Gs):
                tp.grad = torch.from_numpy(G.copy())
            opt.step()
            for k, G in enumerate(Gs):
                W1, B1, _, _ = omuon.muon_tensor_step(Ws[k][None], G[None], Bs[k], None, 1, HP, lr, wd)
                Ws[k], Bs[k] = W1[0], B1
                assert np.abs(Ws[k] - tps[k].detach().numpy()).max() < 1e-13
                assert np.abs(Bs[k][0] - opt.state[tps[k]]["momentum_buffer"].numpy()).max() < 1e-15
    finally:
        tmuon._zeropower_via_newtonschulz = orig


def test_nesterov_off_uses_momentum():
    r = rng(2)
    G = r.standard_normal((1, 8, 12))
    B0 = r.standard_normal((1, 8, 12))
    W = np.zeros((1, 8, 12))
    hp = {"beta": 0.9, "nesterov": False}
    W1, B1, _, _ = omuon.muon_tensor_step(W, G, B0, None, 1, hp, 0.5, 0.0)
    assert np.allclose(B1, 0.9 * B0 + 0.1 * G, rtol=0, atol=1e-15)
    assert np.abs(W1[0] + 0.5 * ns_by_svd(B1[0])).max() < 1e-14


def check_views(step_fn=None):
    """A (2, m, n) view: each half is its own matrix with its own scale."""
    step_fn = step_fn or omuon.muon_tensor_step
    r = rng(3)
    m, n = 8, 4                       # each view is tall 8x4 -> scale sqrt(2)
    G = r.standard_normal((1, 2 * m, n))
    W = 0.02 * r.standard_normal((1, 2 * m, n))
    W1, _, _, _ = step_fn(W, G, np.zeros_like(G), None, 2, HP, 0.02, 0.1)
    for v in range(2):
        sl = slice(v * m, (v + 1) * m)
        want = 0.998 * W[0, sl] - 0.02 * math.sqrt(2.0) * ns_by_svd(0.0975 * G[0, sl])
        assert np.abs(W1[0, sl] - want).max() < 1e-14


def test_views_are_independent_matrices():
    check_views()


def test_batch_entries_are_independent():
    r = rng(4)
    G = r.standard_normal((3, 6, 10))
    W = r.standard_normal((3, 6, 10))
    W1, _, _, _ = omuon.muon_tensor_step(W, G, np.zeros_like(G), None, 1, HP, 0.02, 0.1)
    for b in range(3):
        Wb, _, _, _ = omuon.muon_tensor_step(W[b:b + 1], G[b:b + 1], np.zeros_like(G[b:b + 1]),
                                             None, 1, HP, 0.02, 0.1)
        assert np.array_equal(Wb[0], W1[b])


def test_absent_gradient_leaves_everything():
    W = rng(5).standard_normal((2, 4, 4))
    Bm = rng(6).standard_normal((2, 4, 4))
    V = np.abs(rng(7).standard_normal((2, 4)))
    W1, B1, V1, U = omuon.muon_tensor_step(W, None, Bm, V, 1, {"normuon": True}, 0.02, 0.1)
    assert np.array_equal(W1, W) and np.array_equal(B1, Bm) and np.array_equal(V1, V)
    assert U is None


def test_zero_gradient_only_decays():
    W = rng(8).standard_normal((1, 5, 7))
    W1, B1, _, _ = omuon.muon_tensor_step(W, np.zeros_like(W), np.zeros_like(W), None, 1,
                                          HP, 0.02, 0.1)
    assert np.all(np.isfinite(W1)) and np.all(B1 == 0.0)
    assert np.array_equal(W1, 0.998 * W)


def test_shape_scale_values():
    assert omuon.shape_scale(256, 128) == math.sqrt(2.0)
    assert omuon.shape_scale(3072, 768) == 2.0
    assert abs(omuon.shape_scale(14336, 4096) - 1.8708286933869707) < 1e-15
    assert abs(omuon.shape_scale(28672, 8192) - 1.8708286933869707) < 1e-15
    assert omuon.shape_scale(768, 3072) == 1.0
    assert omuon.shape_scale(768, 768) == 1.0


# ---------------------------------------------------------------------------
# NorMuon, Muon+ and the cautious masks
# ---------------------------------------------------------------------------
def check_normuon(fn=None):
    fn = fn or omuon.normuon
    r = rng(9)
    m, n = 12, 20
    U = r.standard_normal((m, n)) * np.linspace(0.2, 3.0, m)[:, None]
    out, V1 = fn(U, np.zeros(m), 0.95)
    # step 1 from zero state: V = 0.05 * row mean of U^2 and every output row
    # has the same norm, ||U||_F / sqrt(m); directions are kept row by row
    assert np.abs(V1 - 0.05 * (U * U).sum(axis=1) / n).max() < 1e-15
    rn = np.linalg.norm(out, axis=1)
    assert np.abs(rn - np.linalg.norm(U) / math.sqrt(m)).max() < 1e-12
    assert abs(np.linalg.norm(out) - np.linalg.norm(U)) < 1e-12
    cos = (out * U).sum(axis=1) / (rn * np.linalg.norm(U, axis=1))
    assert np.abs(cos - 1.0).max() < 1e-14
    # step 2: V2 = 0.95 V1 + 0.05 rho2
    U2 = r.standard_normal((m, n))
    _, V2 = fn(U2, V1, 0.95)
    assert np.abs(V2 - (0.95 * V1 + 0.05 * (U2 * U2).sum(axis=1) / n)).max() < 1e-15


def test_normuon_rows():
    check_normuon()


def check_muon_plus(fn=None):
    fn = fn or omuon.muon_plus_row_col
    r = rng(10)
    U = r.standard_normal((9, 14)) * np.linspace(0.1, 2.0, 14)[None, :]
    out = fn(U, 0.0)
    # rows are normalised first, columns last: with eps 0 the columns are unit
    assert np.abs(np.linalg.norm(out, axis=0) - 1.0).max() < 1e-14
    # the row stage leaves each column's entries in the ratio U_ij / ||U_i||
    R = U / np.linalg.norm(U, axis=1, keepdims=True)
    assert np.abs(out - R / np.linalg.norm(R, axis=0, keepdims=True)).max() < 1e-14
    # scaled orthogonal matrix: every row and column has norm t
    Q, _ = np.linalg.qr(r.standard_normal((6, 6)))
    t, eps = 0.3, 1e-8
    out = fn(t * Q, eps)
    k = 1.0 / (math.sqrt(t * t + eps) * math.sqrt(t * t / (t * t + eps) + eps))
    assert np.abs(out - k * t * Q).max() < 1e-15


def test_muon_plus_row_col():
    check_muon_plus()


def check_cautious(wrapper=None, wdmask=None):
    wrapper = wrapper or omuon.apply_cautious_wrapper
    wdmask = wdmask or omuon.apply_cautious_wd
    r = rng(12)
    W = r.standard_normal((6, 8))
    U = r.standard_normal((6, 8))
    G = r.standard_normal((6, 8))
    lr, wd, s = 0.02, 0.1, 1.5
    # ties: a zero gradient entry and a zero update entry keep the old value
    G[0, 0] = 0.0
    W[1, 1] = 0.0
    U[1, 1] = 0.0
    out, mask = wrapper(W, U, G, lr, wd, s)
    delta = lr * wd * W + lr * s * U
    keep = ~((delta * G) > 0)
    assert keep[0, 0] and keep[1, 1]
    assert np.array_equal(out[keep], W[keep])
    assert np.array_equal(out[~keep], (W - delta)[~keep])
    assert np.array_equal(mask, ~keep)
    # weight-decay mask: no decay where U*W < 0; a zero product still decays
    out = wdmask(W, U, lr, wd, s)
    neg = (U * W) < 0
    assert np.array_equal(out[neg], (W - lr * s * U)[neg])
    assert np.array_equal(out[~neg], (W - lr * s * U - lr * wd * W)[~neg])
    W2 = W.copy()
    W2[2, 2] = 0.0
    U2 = U.copy()
    U2[3, 3] = 0.0
    o2 = wdmask(W2, U2, lr, wd, s)
    assert o2[3, 3] == W2[3, 3] - lr * wd * W2[3, 3]


def test_cautious_masks():
    check_cautious()


def test_step_with_normuon_and_cautious_wd():
    """Config-4-like tensor (2 views, batch 2): the full step equals NS by SVD,
    then NorMuon's closed form, then the masked apply, matrix by matrix."""
    r = rng(13)
    batch, views, m, n = 2, 2, 6, 10
    G = r.standard_normal((batch, views * m, n))
    W = 0.02 * r.standard_normal((batch, views * m, n))
    V = np.zeros((batch, views * m))
    hp = dict(HP, normuon=True, normuon_beta2=0.95, cautious="wd_mask")
    W1, _, V1, _ = omuon.muon_tensor_step(W, G, np.zeros_like(G), V, views, hp, 0.02, 0.1)
    for b in range(batch):
        for v in range(views):
            sl = slice(v * m, (v + 1) * m)
            U = ns_by_svd(0.0975 * G[b, sl])
            Vv = 0.05 * (U * U).mean(axis=1)
            assert np.abs(V1[b, sl] - Vv).max() < 1e-15
            Un = U / np.sqrt(Vv)[:, None]
            Un *= np.linalg.norm(U) / np.linalg.norm(Un)
            Wv = W[b, sl]
            decay = np.where(Un * Wv >= 0, Wv, 0.0)
            want = Wv - 0.02 * Un - 0.02 * 0.1 * decay
            assert np.abs(W1[b, sl] - want).max() < 1e-14


def _row_col_by_diagonals(U, eps):
    """Muon+ row_col written as two diagonal scalings, D_r^-1 U D_c^-1: D_r
    from the rows of U, D_c from the columns of the row-normalised matrix
    (speedtronic "v2 optimizers", "Muon+": rows first, then columns, eps
    inside each square root)."""
    d_r = np.array([math.sqrt(float(U[i] @ U[i]) + eps) for i in range(U.shape[0])])
    R = np.diag(1.0 / d_r) @ U
    d_c = np.array([math.sqrt(float(R[:, j] @ R[:, j]) + eps) for j in range(U.shape[1])])
    return R @ np.diag(1.0 / d_c)


def check_muon_plus_wrapper_step(step_fn=None):
    """The wide-model workload's whole composition over two steps: Newton-Schulz
    (by SVD), then Muon+ row_col, then the shape scale, then
    delta = lr*wd*W + lr*s*U, kept only where delta * G > 0 with G this step's
    raw gradient (speedtronic "v2 optimizers": "Muon update", "Muon+",
    "Cautious updates"). A packed tensor of two tall 12x5 views (scale
    sqrt(12/5)) and a wide 5x12 tensor (scale 1). The second gradient is drawn
    so that at some entries its sign differs from the Nesterov Q's, which a
    mask taken from Q instead of G would get wrong."""
    step_fn = step_fn or omuon.muon_tensor_step
    r = rng(31)
    lr, wd, eps = 0.02, 0.1, 1e-8
    hp = dict(HP, muon_plus=True, muon_plus_eps=eps, cautious="wrapper")
    for views, m, n in [(2, 12, 5), (1, 5, 12)]:
        s = math.sqrt(max(1.0, m / n))
        shape = (1, views * m, n)
        G1 = r.standard_normal(shape)
        # G2 opposes 3*G1 in a quarter of the entries: there Q2 = 0.045125 G1 +
        # 0.0975 G2 takes G1's sign, against G2's
        G2 = r.standard_normal(shape)
        flip = r.random(shape) < 0.25
        G2[flip] = -0.3 * G1[flip]
        W0 = 0.02 * r.standard_normal(shape)
        Q1 = 0.0975 * G1
        Q2 = 0.045125 * G1 + 0.0975 * G2
        assert np.any(np.sign(Q2) != np.sign(G2))
        W1, B1, _, _ = step_fn(W0, G1, np.zeros(shape), None, views, hp, lr, wd)
        W2, B2, _, _ = step_fn(W1, G2, B1, None, views, hp, lr, wd)
        assert np.abs(B2 - (0.0475 * G1 + 0.05 * G2)).max() < 1e-15
        masks_differ = 0
        for (Wprev, Wgot, Q, G) in [(W0, W1, Q1, G1), (W1, W2, Q2, G2)]:
            for v in range(views):
                sl = slice(v * m, (v + 1) * m)
                U = _row_col_by_diagonals(ns_by_svd(Q[0, sl]), eps)
                delta = lr * wd * Wprev[0, sl] + lr * s * U
                prod = delta * G[0, sl]
                assert np.abs(prod).min() > 1e-12          # no tie near the decision
                want = np.where(prod > 0, Wprev[0, sl] - delta, Wprev[0, sl])
                assert np.abs(Wgot[0, sl] - want).max() < 1e-14, (views, m, n, v)
                masks_differ += int(np.sum((prod > 0) != (delta * Q[0, sl] > 0)))
        assert masks_differ > 0


def test_muon_plus_and_wrapper_two_steps():
    check_muon_plus_wrapper_step()


def check_normuon_wdmask_two_steps(step_fn=None):
    """The MoE workload's composition over two steps, the second moment carried
    from the first: Newton-Schulz (by SVD), NorMuon over each stored row, the
    shape scale, then decay only where U*W >= 0 (flaxchat "Muon Algorithm",
    steps 1 to 4; the shape scale from speedtronic "Muon update"). Batch 2 of a
    packed tensor of two tall 12x5 views: the stored rows (12 per view) are not
    the canonical rows (5), and sqrt(12/5) multiplies the update but not the
    decay. The second gradient's rows are scaled unevenly so that its row means
    differ from the first step's and the carried V matters."""
    step_fn = step_fn or omuon.muon_tensor_step
    r = rng(32)
    lr, wd, b2 = 0.02, 0.1, 0.95
    hp = dict(HP, normuon=True, normuon_beta2=b2, cautious="wd_mask")
    batch, views, m, n = 2, 2, 12, 5
    s = math.sqrt(m / n)
    shape = (batch, views * m, n)
    G1 = r.standard_normal(shape)
    G2 = r.standard_normal(shape) * np.linspace(3.0, 0.2, views * m)[None, :, None]
    W0 = 0.02 * r.standard_normal(shape)
    V0 = np.zeros((batch, views * m))
    W1, B1, V1, _ = step_fn(W0, G1, np.zeros(shape), V0, views, hp, lr, wd)
    W2, _, V2, _ = step_fn(W1, G2, B1, V1, views, hp, lr, wd)
    Q1 = 0.0975 * G1
    Q2 = 0.045125 * G1 + 0.0975 * G2
    carried = 0.0
    for (Wprev, Wgot, Vprev, Vgot, Q) in [(W0, W1, V0, V1, Q1), (W1, W2, V1, V2, Q2)]:
        masked = 0
        for b in range(batch):
            for v in range(views):
                sl = slice(v * m, (v + 1) * m)
                U = ns_by_svd(Q[b, sl])
                rho = np.array([float(U[i] @ U[i]) / n for i in range(m)])
                Vw = b2 * Vprev[b, sl] + (1.0 - b2) * rho
                assert np.abs(Vgot[b, sl] - Vw).max() < 1e-15
                carried = max(carried, float(np.abs(Vw - (1.0 - b2) * rho).max()))
                Un = U / np.sqrt(Vw)[:, None]
                Un *= np.linalg.norm(U) / np.linalg.norm(Un)
                Wv = Wprev[b, sl]
                prod = Un * Wv
                assert np.abs(prod).min() > 1e-12          # no tie near the decision
                keep = prod >= 0
                masked += int(np.sum(~keep))
                want = Wv - lr * s * Un - lr * wd * np.where(keep, Wv, 0.0)
                assert np.abs(Wgot[b, sl] - want).max() < 1e-14, (b, v)
        assert masked > 0
    assert carried > 1e-3


def test_normuon_wdmask_two_steps_tall_views():
    check_normuon_wdmask_two_steps()


# ---------------------------------------------------------------------------
# AdamW closed forms
# ---------------------------------------------------------------------------
def check_adamw(fn=None):
    fn = fn or oadamw.adamw_update
    r = rng(14)
    p0 = 0.02 * r.standard_normal(1000)
    g1 = 1e-3 * r.standard_normal(1000)
    g2 = 1e-3 * r.standard_normal(1000)
    lr, wd, eps = 3e-4, 0.1, 1e-8
    p1, m1, v1 = fn(p0, g1, np.zeros(1000), np.zeros(1000), lr, wd, 0.9, 0.95, eps, 1)
    def rel(x, y):
        return np.abs(x - y).max() / np.abs(y).max()
    assert rel(m1, 0.1 * g1) < 1e-15
    assert rel(v1, 0.05 * g1 * g1) < 1e-15
    want1 = p0 - lr * (g1 / (np.abs(g1) + eps) + wd * p0)
    assert rel(p1, want1) < 1e-15
    p2, m2, v2 = fn(p1, g2, m1, v1, lr, wd, 0.9, 0.95, eps, 2)
    mm = 0.09 * g1 + 0.1 * g2
    vv = 0.0475 * g1 * g1 + 0.05 * g2 * g2
    want2 = p1 - lr * ((mm / 0.19) / (np.sqrt(vv / 0.0975) + eps) + wd * p1)
    assert rel(m2, mm) < 1e-15
    assert rel(v2, vv) < 1e-15
    assert rel(p2, want2) < 1e-15


def test_adamw_closed_forms():
    check_adamw()


def test_adamw_zero_grad_is_pure_decay():
    p = np.linspace(-1, 1, 11)
    p1, m1, v1 = oadamw.adamw_update(p, np.zeros(11), np.zeros(11), np.zeros(11),
                                     1e-3, 0.1, 0.9, 0.95, 1e-8, 1)
    assert np.array_equal(m1, np.zeros(11)) and np.array_equal(v1, np.zeros(11))
    assert np.allclose(p1, p * (1 - 1e-4), rtol=0, atol=1e-18)


def test_adamw_matches_torch_optim_adamw():
    """Four steps of the oracle against torch.optim.AdamW in float64 on the CPU
    (decoupled decay, bias-corrected moments, eps outside the square root), a
    library routine the oracle shares no code with."""
    r = np.random.default_rng(21)
    p = r.standard_normal(257)
    lr, wd, b1, b2, eps = 3e-3, 0.1, 0.9, 0.95, 1e-8
    tp = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    for step in range(1, 5):
        g = r.standard_normal(257) * 10.0 ** r.integers(-3, 3)
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        p, m, v = oadamw.adamw_update(p, g, m, v, lr, wd, b1, b2, eps, step)
        st = opt.state[tp]
        assert np.abs(m - st["exp_avg"].numpy()).max() <= 1e-15 * np.abs(m).max()
        assert np.abs(v - st["exp_avg_sq"].numpy()).max() <= 1e-15 * np.abs(v).max()
        assert np.abs(p - tp.detach().numpy()).max() <= 1e-14 * np.abs(p).max()


# ---------------------------------------------------------------------------
# Storage formats
# ---------------------------------------------------------------------------
def check_bf16_rounding(fn=None):
    fn = fn or storage.round_bf16_bits
    cases = {1.0: 0x3F80, -2.5: 0xC020, 1.0 + 2 ** -8: 0x3F80, 1.0 + 3 * 2 ** -8: 0x3F82,
             1.0 + 2 ** -8 + 2 ** -30: 0x3F81, 0.0: 0x0000, 2 ** -133: 0x0001,
             3.0e38: 0x7F62}
    for x, bits in cases.items():
        assert int(fn(np.array([x]))[0]) == bits, (x, hex(int(fn(np.array([x]))[0])))
    assert int(fn(np.array([np.nan]))[0]) & 0x7F80 == 0x7F80
    # values exact in binary32 round the same as torch's float32 -> bfloat16
    x = (np.random.default_rng(15).standard_normal(100000) * 10.0 ** np.random.default_rng(16)
         .integers(-20, 20, 100000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fn(x.astype(np.float64)), ref)


def test_bf16_rounding():
    check_bf16_rounding()


def test_decode():
    bits = np.array([0x3F80, 0xC020, 0x0001, 0x7F80], dtype=np.uint16)
    v = storage.decode(bits, "bf16")
    assert v[0] == 1.0 and v[1] == -2.5 and v[2] == 2.0 ** -133 and np.isinf(v[3])
    f = np.array([1.5, -3.25], dtype=np.float32)
    assert np.array_equal(storage.decode(f, "f32"), np.array([1.5, -3.25]))


def test_round_trip_f32_state():
    x = np.random.default_rng(17).standard_normal(1000)
    assert np.array_equal(storage.round_f32(x), x.astype(np.float32))


def test_muon_step_dict_api_bf16():
    """The list-of-tensors entry with bf16 storage: outputs round once from fp64."""
    r = rng(18)
    W = (0.02 * r.standard_normal((1, 16, 8))).astype(np.float32)
    G = r.standard_normal((1, 16, 8)).astype(np.float32)
    Wb = torch.from_numpy(W).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    Gb = torch.from_numpy(G).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    t = {"param": Wb, "param_dtype": "bf16", "grad": Gb, "grad_dtype": "bf16",
         "momentum": np.zeros((1, 16, 8), np.float32), "row_v": None, "views": 1,
         "lr": 0.02, "wd": 0.1, "shape": (1, 16, 8)}
    out = omuon.muon_step([t], HP)[0]
    W64 = storage.decode(Wb, "bf16")
    G64 = storage.decode(Gb, "bf16")
    want = 0.998 * W64[0] - 0.02 * math.sqrt(2.0) * ns_by_svd(0.0975 * G64[0])
    assert np.abs(out["W64"][0] - want).max() < 1e-14
    assert np.array_equal(out["param"], storage.round_bf16_bits(out["W64"]))
    assert np.array_equal(out["momentum"], (0.05 * G64).astype(np.float32))


# ---------------------------------------------------------------------------
# Next rows: stochastic rounding, bf16 moments, global-norm clip, cautious
# AdamW, per-iteration coefficients
# ---------------------------------------------------------------------------
from oracle import gradnorm as ognorm  # noqa: E402


def test_splitmix64_reference_outputs():
    """SplitMix64 (Steele, Lea and Flood 2014) seeded with 0 yields
    0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F: the published
    generator's first outputs, state advanced by the golden-ratio gamma."""
    g = storage.SPLITMIX_GAMMA
    got = [int(storage.splitmix64_mix(np.uint64((k * g) % 2**64))) for k in (1, 2, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_stochastic_rounding_keeps_exact_values_and_specials():
    """A value already in bf16 has zero discarded bits: no noise can carry, so
    it is kept for every key; infinities stay infinite; NaN stays NaN
    (dew.training.optim "stochastic_round_bf16")."""
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 0x7F7F, size=5000).astype(np.uint16)
    bits[::2] |= 0x8000
    x = storage.decode(bits, "bf16").astype(np.float32)
    for key in (0, 1, 0xDEADBEEFCAFEF00D):
        assert np.array_equal(storage.stochastic_round_bf16_bits(x, key), bits)
    sp = np.array([np.inf, -np.inf, np.nan, -np.nan], dtype=np.float32)
    # NaNs whose payload sits only in the discarded low bits must not truncate to inf
    sp = np.concatenate([sp, np.array([0x7F800001, 0xFF80FFFF], dtype=np.uint32).view(np.float32)])
    out = storage.stochastic_round_bf16_bits(sp, 7)
    assert out[0] == 0x7F80 and out[1] == 0xFF80
    back = storage.decode(out, "bf16")
    assert np.isnan(back[2:]).all()


@pytest.mark.parametrize("frac", [0.1, 0.25, 0.5, 0.9])
def test_stochastic_rounding_probability_is_distance(frac):
    """x between two bf16 neighbours rounds up with probability equal to its
    fractional distance from the lower one (the page: "rounded ... up or down
    with the probability of its distance to each"), over 40000 flat indices."""
    lo = np.float32(1.5)
    ulp = np.float32(2.0 ** -7)          # bf16 spacing in [1, 2)
    x = np.full(40000, lo + np.float32(frac) * ulp, dtype=np.float32)
    out = storage.decode(storage.stochastic_round_bf16_bits(x, 12345), "bf16")
    assert set(np.unique(out)) <= {float(lo), float(lo + ulp)}
    p_up = np.mean(out > lo)
    sigma = math.sqrt(frac * (1 - frac) / x.size)
    assert abs(p_up - frac) < 5 * sigma + 1e-4, (p_up, frac)


def test_bf16_second_moment_increments_kept_in_expectation():
    """The page's reason for stochastic rounding: with beta2 = 0.999 most
    increments of the second moment are below half its bf16 spacing, so
    round-to-nearest loses them all, while the stochastic rounding keeps each
    one in expectation. v = 1 (exact in bf16), g^2 = 1.5: the increment is
    0.0005, about a sixteenth of the spacing 2^-7."""
    v0, g2, b2 = 1.0, 1.5, 0.999
    v1 = b2 * v0 + (1 - b2) * g2
    rne = storage.decode(storage.round_bf16_bits(np.array([v1])), "bf16")[0]
    assert rne == v0                                  # nearest rounding loses it
    x = np.full(200000, np.float32(v1), dtype=np.float32)
    sr = storage.decode(storage.stochastic_round_bf16_bits(x, 99), "bf16")
    mean_inc = float(np.mean(sr) - v0)
    assert abs(mean_inc - (v1 - v0)) < 5 * math.sqrt((v1 - v0) * 2 ** -7 / x.size) + 1e-7


def test_adamw_bf16_moments_use_the_step_tensor_and_moment_keys():
    """bf16 moments: the update runs on the widened moments; each new moment is
    the fp32 value stochastically rounded with the key of (seed, step, tensor,
    moment); different tensors, moments or steps draw different bits."""
    rng = np.random.default_rng(8)
    n = 5000
    t = lambda: {"param": rng.normal(0, 0.02, n).astype(np.float32), "param_dtype": "f32",
                 "grad": rng.normal(0, 1e-3, n).astype(np.float32), "grad_dtype": "f32",
                 "m": storage.round_bf16_bits(rng.normal(0, 1e-4, n)),
                 "v": storage.round_bf16_bits(rng.uniform(1e-8, 1e-6, n)), "moment_dtype": "bf16",
                 "lr": 1e-3, "wd": 0.1}
    t0 = t()
    ts = [t0, {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in t0.items()}]   # identical inputs
    hp = {"beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "step": 3, "seed": 42}
    out = oadamw.adamw_step(ts, hp)
    # the same values in two tensors draw different noise (the tensor index is in the key)
    assert np.array_equal(out[0]["param"], out[1]["param"])
    assert not np.array_equal(out[0]["m"], out[1]["m"]) and not np.array_equal(out[0]["v"], out[1]["v"])
    for k, (ti, o) in enumerate(zip(ts, out)):
        p64, m64, v64 = oadamw.adamw_update(storage.decode(ti["param"], "f32"), storage.decode(ti["grad"], "f32"),
                                            storage.decode(ti["m"], "bf16"), storage.decode(ti["v"], "bf16"),
                                            1e-3, 0.1, 0.9, 0.999, 1e-8, 3)
        assert np.array_equal(o["param"], storage.round_f32(p64))
        # each stored moment is one of the two bf16 neighbours of its fp32 value
        for nm, x64 in (("m", m64), ("v", v64)):
            x32 = storage.round_f32(x64).astype(np.float64)
            got = storage.decode(o[nm], "bf16")
            lo = storage.decode((np.asarray(storage.round_f32(x64)).view(np.uint32) >> 16).astype(np.uint16), "bf16")
            assert np.all((got == lo) | (np.abs(got) > np.abs(lo))) and np.all(np.abs(got - x32) <= np.abs(x32) * 2 ** -7)
    assert not np.array_equal(out[0]["m"], oadamw.adamw_step([ts[0]], dict(hp, step=4))[0]["m"])


def test_global_norm_and_clip_closed_forms():
    """||g|| over every element of every gradient; the clip factor is
    max_norm/||g|| above max_norm, 1 below it or with max_norm <= 0 (clipping
    off, the norm still observed); a norm that is not finite skips the step."""
    a = np.ones(300, dtype=np.float32)
    b = storage.round_bf16_bits(np.full((10, 10), 2.0))
    nrm = ognorm.global_norm([(a, "f32"), None, (b, "bf16")])
    assert nrm == math.sqrt(300 + 400)
    assert ognorm.clip_state(nrm, 10.0) == (10.0 / math.sqrt(700), False)
    assert ognorm.clip_state(nrm, 100.0) == (1.0, False)
    assert ognorm.clip_state(nrm, 0.0) == (1.0, False)
    big = np.array([1e30, 1e30], dtype=np.float32)
    assert ognorm.clip_state(ognorm.global_norm([(big, "f32")]), 1.0)[1] is False   # finite in fp64
    inf = np.array([np.inf], dtype=np.float32)
    nan = np.array([np.nan], dtype=np.float32)
    assert ognorm.clip_state(ognorm.global_norm([(inf, "f32")]), 1.0)[1] is True
    assert ognorm.clip_state(ognorm.global_norm([(nan, "f32")]), 0.0)[1] is True


def test_global_norm_matches_torch_clip_grad_norm():
    """The norm over several fp32 and bf16 gradients against
    torch.nn.utils.clip_grad_norm_ in float64 on the decoded values, and the
    scaled gradients against torch's (whose factor has 1e-6 added to the norm)."""
    r = np.random.default_rng(22)
    stored = [(r.standard_normal(1000).astype(np.float32), "f32"),
              (storage.round_bf16_bits(r.standard_normal((33, 7)) * 3.0), "bf16"),
              (r.standard_normal(5).astype(np.float32) * 100.0, "f32")]
    nrm = ognorm.global_norm(stored + [None])
    ts = [torch.nn.Parameter(torch.zeros(storage.decode(x, dt).size, dtype=torch.float64)) for x, dt in stored]
    for t, (x, dt) in zip(ts, stored):
        t.grad = torch.from_numpy(storage.decode(x, dt).reshape(-1).astype(np.float64))
    ref = float(torch.nn.utils.clip_grad_norm_(ts, max_norm=50.0))
    assert abs(nrm - ref) <= 1e-15 * ref
    factor, skip = ognorm.clip_state(nrm, 50.0)
    assert not skip and factor < 1.0
    for t, (x, dt) in zip(ts, stored):
        want = storage.decode(x, dt).reshape(-1) * factor
        assert np.abs(t.grad.numpy() - want).max() <= 1e-7 * np.abs(want).max()


def test_clip_skip_leaves_every_buffer_and_scales_the_gradient():
    """A skipped step returns every stored input unchanged (both halves); a
    clip factor enters as a scaled gradient: from zero momentum the new
    momentum is (1 - beta) * factor * G."""
    rng = np.random.default_rng(5)
    W = rng.normal(0, 0.02, (1, 40, 60)).astype(np.float32)
    G = rng.normal(0, 1e-3, (1, 40, 60)).astype(np.float32)
    t = {"param": W, "param_dtype": "f32", "grad": G, "grad_dtype": "f32",
         "momentum": np.zeros_like(W), "row_v": None, "views": 1, "lr": 0.02, "wd": 0.1, "shape": (1, 40, 60)}
    out = omuon.muon_step([t], {"ns_steps": 5}, clip=(0.25, True))[0]
    assert np.array_equal(out["param"], W) and np.array_equal(out["momentum"], t["momentum"])
    out = omuon.muon_step([t], {"ns_steps": 5, "beta": 0.95}, clip=(0.25, False))[0]
    assert np.allclose(out["B64"], 0.05 * 0.25 * G.astype(np.float64), rtol=1e-14, atol=0)
    a = {"param": W.ravel(), "param_dtype": "f32", "grad": G.ravel(), "grad_dtype": "f32",
         "m": np.zeros(W.size, np.float32), "v": np.zeros(W.size, np.float32), "lr": 1e-3, "wd": 0.1}
    o = oadamw.adamw_step([a], {"beta1": 0.9, "beta2": 0.95, "eps": 1e-8, "step": 1}, clip=(1.0, True))[0]
    assert np.array_equal(o["param"], a["param"]) and np.array_equal(o["m"], a["m"])


def test_cautious_adamw_masks_against_the_gradient():
    """speedtronic "Cautious updates" over AdamW. At step 1 with zero state,
    m_hat = g and v_hat = g^2, so the update is lr (g/(|g|+eps) + wd p): with
    wd = 0 it always points along g (nothing masked); with a large decay on a
    parameter of opposite sign to g it points against g, and that parameter
    is left bit for bit; the moments are updated everywhere."""
    g = np.array([1e-3, -2e-3, 1e-3, -1e-3, 0.0])
    p = np.array([0.5, 0.5, -100.0, 100.0, 0.5])
    z = np.zeros(5)
    p0, m0, v0 = oadamw.adamw_update(p, g, z, z, 1e-2, 0.0, 0.9, 0.999, 1e-8, 1)
    p1, m1, v1 = oadamw.adamw_update(p, g, z, z, 1e-2, 0.0, 0.9, 0.999, 1e-8, 1, cautious=True)
    assert np.array_equal(p0, p1)
    # a zero gradient: the update is pure decay, not > 0 against g = 0: kept as is
    pz, _, _ = oadamw.adamw_update(p, g, z, z, 1e-2, 0.1, 0.9, 0.999, 1e-8, 1, cautious=True)
    assert pz[4] == p[4]
    p2, m2, v2 = oadamw.adamw_update(p, g, z, z, 1e-2, 0.1, 0.9, 0.999, 1e-8, 1, cautious=True)
    # entries 2, 3: 1 + 0.1 * p has the opposite sign of g -> masked
    assert p2[2] == p[2] and p2[3] == p[3]
    assert p2[0] < p[0] and p2[1] < p[1] + 1.0
    assert np.array_equal(m2, m0) and np.array_equal(v2, v0)


def test_ns_table_closed_forms_and_order():
    """Per-iteration coefficients, against the SVD X0 = U S V^T of the
    normalised input: a row (s, 0, 0) scales X by s; (0, 1, 0) maps S to S^3;
    (0, 0, 1) maps S to S^5. So [(2,0,0), (0,1,0), (0,0,1)] gives
    U (2S)^15 V^T... i.e. singular values (8 S^3)^5, and the reversed table
    gives 2 S^15: each row is used at its own iteration."""
    rng = np.random.default_rng(11)
    M = rng.normal(size=(20, 30))
    X0 = M / np.linalg.norm(M)
    U, S, Vt = np.linalg.svd(X0, full_matrices=False)
    fwd = omuon.newton_schulz(M, steps=3, eps=0.0, table=[(2, 0, 0), (0, 1, 0), (0, 0, 1)])
    rev = omuon.newton_schulz(M, steps=3, eps=0.0, table=[(0, 0, 1), (0, 1, 0), (2, 0, 0)])
    assert np.allclose(fwd, (U * (8 * S ** 3) ** 5) @ Vt, rtol=1e-10, atol=1e-300)
    assert np.allclose(rev, (U * (2 * S ** 15)) @ Vt, rtol=1e-10, atol=1e-300)
    # a constant table is the plain iteration
    plain = omuon.newton_schulz(M)
    assert np.array_equal(omuon.newton_schulz(M, table=[omuon.NS_COEFFS] * 5), plain)


def test_ns_norm_scale_is_flaxchat_safety_factor():
    """flaxchat "Muon Algorithm" step 2 starts from g / (||g|| * 1.01): with one
    identity iteration (1, 0, 0) the output is exactly that, plus eps."""
    rng = np.random.default_rng(12)
    M = rng.normal(size=(16, 24))
    out = omuon.newton_schulz(M, steps=1, eps=1e-7, table=[(1, 0, 0)], norm_scale=1.01)
    assert np.allclose(out, M / (np.linalg.norm(M) * 1.01 + 1e-7), rtol=1e-14, atol=0)
