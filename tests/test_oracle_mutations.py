"""Plant plausible slips in the oracle (on the CPU) and check that a pin fails.

Each mutant replaces one oracle function with a copy carrying a single slip
(a dropped term, a flipped sign, a transposed operand, a wrong axis or
comparison). The pins in ``test_oracle_pins.py`` must reject every mutant;
that is what makes them pins rather than retypings of the oracle.
"""
import math

import numpy as np
import pytest

import oracle.adamw as oadamw
import oracle.muon as omuon
import oracle.storage as ostorage
from tests import test_oracle_pins as pins

A, B, C = pins.A, pins.B, pins.C


def _ns_template(M, steps=5, eps=1e-7, coeffs=(A, B, C), *, wrong_side=False,
                 spectral=False, drop_eps=False, steps_delta=0, norm_power=1):
    X = np.array(M, dtype=np.float64)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    nrm = np.linalg.norm(X, 2) if spectral else np.linalg.norm(X)
    X = X / (nrm ** norm_power + (0.0 if drop_eps else eps))
    a, b, c = coeffs
    for _ in range(steps + steps_delta):
        Am = X @ X.T
        Bm = b * Am + c * (Am @ Am)
        X = a * X + (X.T @ Bm.T).T if wrong_side else a * X + Bm @ X
    return X.T if tall else X


def ns_flip_b(M, steps=5, eps=1e-7, coeffs=(A, B, C), table=None, norm_scale=1.0):
    return _ns_template(M, steps, eps, (A, -B, C))


def ns_drop_c(M, steps=5, eps=1e-7, coeffs=(A, B, C), table=None, norm_scale=1.0):
    return _ns_template(M, steps, eps, (A, B, 0.0))


def ns_spectral(M, steps=5, eps=1e-7, coeffs=(A, B, C), table=None, norm_scale=1.0):
    return _ns_template(M, steps, eps, coeffs, spectral=True)


def ns_no_eps(M, steps=5, eps=1e-7, coeffs=(A, B, C), table=None, norm_scale=1.0):
    return _ns_template(M, steps, eps, coeffs, drop_eps=True)


def ns_four_steps(M, steps=5, eps=1e-7, coeffs=(A, B, C), table=None, norm_scale=1.0):
    return _ns_template(M, steps, eps, coeffs, steps_delta=-1)


def ns_norm_squared(M, steps=5, eps=1e-7, coeffs=(A, B, C), table=None, norm_scale=1.0):
    """Normalised by the squared Frobenius norm (the sum of squares, no root)."""
    return _ns_template(M, steps, eps, coeffs, norm_power=2)


def ns_xa_order(M, steps=5, eps=1e-7, coeffs=(A, B, C), table=None, norm_scale=1.0):
    """X (bA + cA^2) instead of (bA + cA^2) X: the operands swap places, which
    only type-checks (and only differs) for a square matrix."""
    X = np.array(M, dtype=np.float64)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = X / (np.linalg.norm(X) + eps)
    a, b, c = coeffs
    for _ in range(steps):
        Am = X @ X.T
        Bm = b * Am + c * (Am @ Am)
        X = a * X + (X @ Bm if X.shape[0] == X.shape[1] else Bm @ X)
    return X.T if tall else X


NS_MUTANTS = [ns_flip_b, ns_drop_c, ns_spectral, ns_no_eps, ns_four_steps, ns_xa_order, ns_norm_squared]


# a mutant may diverge and overflow; that is part of how it fails
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("mutant", NS_MUTANTS, ids=lambda f: f.__name__)
def test_ns_mutants_caught(mutant, monkeypatch):
    with pytest.raises(AssertionError):
        pins.check_ns_svd(mutant)
    monkeypatch.setattr(omuon, "newton_schulz", mutant)
    with pytest.raises(AssertionError):
        pins.check_first_step()


def momentum_no_dampening(Bm, G, beta):
    return beta * Bm + G


def momentum_swapped(Bm, G, beta):
    return (1.0 - beta) * Bm + beta * G


def nesterov_old_sign(G, Bm, beta):
    return G - beta * (Bm - G)


def scale_swapped(m, n):
    return max(1.0, n / m) ** 0.5


def scale_no_sqrt(m, n):
    return max(1.0, m / n)


def decay_not_lr_scaled(W, U, lr, wd, s):
    return (1.0 - wd) * W - lr * s * U


def decay_dropped(W, U, lr, wd, s):
    return W - lr * s * U


def decay_after_update(W, U, lr, wd, s):
    """The decay factor applied to the already updated weight."""
    return (1.0 - lr * wd) * (W - lr * s * U)


@pytest.mark.parametrize("name,mutant", [
    ("momentum_ema", momentum_no_dampening),
    ("momentum_ema", momentum_swapped),
    ("nesterov_lerp", nesterov_old_sign),
    ("shape_scale", scale_swapped),
    ("shape_scale", scale_no_sqrt),
    ("apply_decoupled", decay_not_lr_scaled),
    ("apply_decoupled", decay_dropped),
    ("apply_decoupled", decay_after_update),
], ids=lambda x: x if isinstance(x, str) else x.__name__)
def test_step_mutants_caught(name, mutant, monkeypatch):
    monkeypatch.setattr(omuon, name, mutant)
    failures = 0
    for check in (pins.check_first_step, pins.check_second_step, pins.check_views):
        try:
            check()
        except AssertionError:
            failures += 1
    assert failures >= 1


def test_nesterov_using_old_momentum_caught(monkeypatch):
    """Nesterov from the momentum before this step's update."""
    real = omuon.muon_tensor_step

    def stale(W, G, Bm, V, views, hp, lr, wd):
        beta = hp.get("beta", 0.95)
        Q = G + beta * (Bm - G)
        B_new = omuon.momentum_ema(Bm, G, beta)
        Wn = np.empty_like(W)
        m = W.shape[1] // views
        for b in range(W.shape[0]):
            for v in range(views):
                sl = slice(v * m, (v + 1) * m)
                Wn[b, sl], _, _ = omuon.matrix_update(Q[b, sl], W[b, sl], G[b, sl], None, hp, lr, wd)
        return Wn, B_new, None, None

    with pytest.raises(AssertionError):
        pins.check_second_step(stale)
    pins.check_second_step(real)


def view_scale_from_parent(W, G, Bm, V, views, hp, lr, wd):
    """Scale taken from the packed parent's rows instead of the view's."""
    beta = hp.get("beta", 0.95)
    B_new = omuon.momentum_ema(Bm, G, beta)
    Q = omuon.nesterov_lerp(G, B_new, beta)
    batch, rows, cols = W.shape
    m = rows // views
    Wn = np.empty_like(W)
    for b in range(batch):
        for v in range(views):
            sl = slice(v * m, (v + 1) * m)
            U = omuon.newton_schulz(Q[b, sl])
            Wn[b, sl] = omuon.apply_decoupled(W[b, sl], U, lr, wd, omuon.shape_scale(rows, cols))
    return Wn, B_new, None, None


def whole_parent_ns(W, G, Bm, V, views, hp, lr, wd):
    """The packed parent orthogonalised as one matrix (views ignored)."""
    return omuon.muon_tensor_step(W, G, Bm, V, 1, hp, lr, wd)


def batch_norm_shared(W, G, Bm, V, views, hp, lr, wd):
    """Every batch entry normalised by the Frobenius norm of the whole batch
    before its own iteration, instead of by its own norm."""
    beta = hp.get("beta", 0.95)
    B_new = omuon.momentum_ema(Bm, G, beta)
    Q = omuon.nesterov_lerp(G, B_new, beta)
    batch, rows, cols = W.shape
    total = np.linalg.norm(Q)
    Wn = np.empty_like(W)
    for b in range(batch):
        X = Q[b].T if rows > cols else Q[b]
        X = X / (total + 1e-7)
        for _ in range(5):
            Am = X @ X.T
            X = A * X + (B * Am + C * (Am @ Am)) @ X
        U = X.T if rows > cols else X
        Wn[b] = omuon.apply_decoupled(W[b], U, lr, wd, omuon.shape_scale(rows, cols))
    return Wn, B_new, None, None


def test_batch_norm_shared_caught(monkeypatch):
    monkeypatch.setattr(omuon, "muon_tensor_step", batch_norm_shared)
    with pytest.raises(AssertionError):
        pins.test_batch_entries_are_independent()


@pytest.mark.parametrize("mutant", [view_scale_from_parent, whole_parent_ns],
                         ids=lambda f: f.__name__)
def test_view_mutants_caught(mutant):
    with pytest.raises(AssertionError):
        pins.check_views(mutant)


def normuon_column_axis(U, V, beta2):
    v_mean = np.mean(U * U, axis=0)
    V_new = V + (1.0 - beta2) * (v_mean[: V.shape[0]] - V)
    U_hat = U * (np.maximum(V_new, 1e-30) ** -0.5)[:, None]
    return U_hat * (np.linalg.norm(U) / np.linalg.norm(U_hat)), V_new


def normuon_not_norm_preserving(U, V, beta2):
    v_mean = np.mean(U * U, axis=1)
    V_new = V + (1.0 - beta2) * (v_mean - V)
    return U * (np.maximum(V_new, 1e-30) ** -0.5)[:, None], V_new


def normuon_beta_swapped(U, V, beta2):
    v_mean = np.mean(U * U, axis=1)
    V_new = V + beta2 * (v_mean - V)
    U_hat = U * (np.maximum(V_new, 1e-30) ** -0.5)[:, None]
    return U_hat * (np.linalg.norm(U) / np.linalg.norm(U_hat)), V_new


def normuon_no_running_average(U, V, beta2):
    """V replaced by this step's row means instead of averaged into them."""
    v_mean = np.mean(U * U, axis=1)
    U_hat = U * (np.maximum(v_mean, 1e-30) ** -0.5)[:, None]
    return U_hat * (np.linalg.norm(U) / np.linalg.norm(U_hat)), v_mean


@pytest.mark.parametrize("mutant", [normuon_column_axis, normuon_not_norm_preserving,
                                    normuon_beta_swapped, normuon_no_running_average], ids=lambda f: f.__name__)
def test_normuon_mutants_caught(mutant):
    with pytest.raises((AssertionError, ValueError)):
        pins.check_normuon(mutant)


def muon_plus_columns_first(U, eps):
    U = U / np.sqrt(np.sum(U * U, axis=0, keepdims=True) + eps)
    return U / np.sqrt(np.sum(U * U, axis=1, keepdims=True) + eps)


def muon_plus_eps_outside(U, eps):
    U = U / (np.sqrt(np.sum(U * U, axis=1, keepdims=True)) + eps)
    return U / (np.sqrt(np.sum(U * U, axis=0, keepdims=True)) + eps)


def muon_plus_unit_rms(U, eps):
    """Rows, then columns, scaled to unit RMS instead of unit L2 norm."""
    U = U / np.sqrt(np.mean(U * U, axis=1, keepdims=True) + eps)
    U = U / np.sqrt(np.mean(U * U, axis=0, keepdims=True) + eps)
    return U


@pytest.mark.parametrize("mutant", [muon_plus_columns_first, muon_plus_eps_outside, muon_plus_unit_rms],
                         ids=lambda f: f.__name__)
def test_muon_plus_mutants_caught(mutant):
    with pytest.raises(AssertionError):
        pins.check_muon_plus(mutant)


def wrapper_ge(W, U, G, lr, wd, s):
    delta = lr * wd * W + lr * s * U
    mask = (delta * G) >= 0.0
    return np.where(mask, W - delta, W), mask


def wrapper_no_decay(W, U, G, lr, wd, s):
    delta = lr * s * U
    mask = (delta * G) > 0.0
    return np.where(mask, W - lr * wd * W - delta, W), mask


def wdmask_strict(W, U, lr, wd, s):
    mask = (U * W) > 0.0
    return W - lr * s * U - lr * wd * np.where(mask, W, 0.0)


def test_cautious_mutants_caught():
    with pytest.raises(AssertionError):
        pins.check_cautious(wrapper=wrapper_ge)
    with pytest.raises(AssertionError):
        pins.check_cautious(wrapper=wrapper_no_decay)
    with pytest.raises(AssertionError):
        pins.check_cautious(wdmask=wdmask_strict)


def adamw_eps_inside(p, g, m, v, lr, wd, b1, b2, eps, step):
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    mh, vh = m / (1 - b1 ** step), v / (1 - b2 ** step)
    return p - lr * (mh / np.sqrt(vh + eps) + wd * p), m, v


def adamw_no_bias_correction(p, g, m, v, lr, wd, b1, b2, eps, step):
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    return p - lr * (m / (np.sqrt(v) + eps) + wd * p), m, v


def adamw_coupled_decay(p, g, m, v, lr, wd, b1, b2, eps, step):
    g = g + wd * p
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    mh, vh = m / (1 - b1 ** step), v / (1 - b2 ** step)
    return p - lr * mh / (np.sqrt(vh) + eps), m, v


def adamw_bias_next_step(p, g, m, v, lr, wd, b1, b2, eps, step):
    """Bias correction with the next step's count."""
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    mh, vh = m / (1 - b1 ** (step + 1)), v / (1 - b2 ** (step + 1))
    return p - lr * (mh / (np.sqrt(vh) + eps) + wd * p), m, v


def adamw_decay_not_lr_scaled(p, g, m, v, lr, wd, b1, b2, eps, step):
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    mh, vh = m / (1 - b1 ** step), v / (1 - b2 ** step)
    return p - lr * mh / (np.sqrt(vh) + eps) - wd * p, m, v


@pytest.mark.parametrize("mutant", [adamw_eps_inside, adamw_no_bias_correction, adamw_coupled_decay,
                                    adamw_bias_next_step, adamw_decay_not_lr_scaled],
                         ids=lambda f: f.__name__)
def test_adamw_mutants_caught(mutant):
    with pytest.raises(AssertionError):
        pins.check_adamw(mutant)


def bf16_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    return (x.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_via_f32(x):
    """Double rounding through binary32: differs from one rounding near ties."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


@pytest.mark.parametrize("mutant", [bf16_truncate, bf16_via_f32], ids=lambda f: f.__name__)
def test_bf16_rounding_mutants_caught(mutant):
    with pytest.raises(AssertionError):
        pins.check_bf16_rounding(mutant)



# -- next rows: stochastic rounding, cautious AdamW, global norm, NS table ---
from oracle import adamw as oadamw  # noqa: E402
from oracle import gradnorm as ognorm  # noqa: E402
from oracle import storage as ostorage  # noqa: E402


def _sr_wide_noise(x32, key, index0=0):
    """17 noise bits instead of 16: rounds up too often."""
    x32 = np.asarray(x32, dtype=np.float32)
    u = x32.reshape(-1).view(np.uint32).astype(np.uint64)
    idx = np.arange(u.size, dtype=np.uint64) + np.uint64(index0 + 1)
    with np.errstate(over="ignore"):
        r = ostorage.splitmix64_mix(np.uint64(key) + idx * np.uint64(ostorage.SPLITMIX_GAMMA)) >> np.uint64(47)
    return ((u + r) >> np.uint64(16)).astype(np.uint16).reshape(x32.shape)


def _sr_no_nan_rule(x32, key, index0=0):
    """Plain add-and-truncate, NaN not special-cased."""
    x32 = np.asarray(x32, dtype=np.float32)
    u = x32.reshape(-1).view(np.uint32).astype(np.uint64)
    idx = np.arange(u.size, dtype=np.uint64) + np.uint64(index0 + 1)
    with np.errstate(over="ignore"):
        r = ostorage.splitmix64_mix(np.uint64(key) + idx * np.uint64(ostorage.SPLITMIX_GAMMA)) >> np.uint64(48)
    return ((u + r) >> np.uint64(16)).astype(np.uint16).reshape(x32.shape)


# the mutant without the NaN rule hands NaN on as bits; decoding them warns
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("mutant", [_sr_wide_noise, _sr_no_nan_rule], ids=lambda f: f.__name__)
def test_stochastic_rounding_mutants_caught(mutant, monkeypatch):
    monkeypatch.setattr(ostorage, "stochastic_round_bf16_bits", mutant)
    with pytest.raises(AssertionError):
        pins.test_stochastic_rounding_keeps_exact_values_and_specials()
        for f in (0.1, 0.25, 0.5, 0.9):
            pins.test_stochastic_rounding_probability_is_distance(f)


def _adamw_cautious_ge(p, g, m, v, lr, wd, beta1, beta2, eps, step, cautious=False):
    p2, m2, v2 = oadamw_orig(p, g, m, v, lr, wd, beta1, beta2, eps, step)
    if cautious:
        p2 = np.where((p - p2) * g >= 0.0, p2, p)
    return p2, m2, v2


def _adamw_cautious_after_update(p, g, m, v, lr, wd, beta1, beta2, eps, step, cautious=False):
    """Mask from the new parameter instead of the observed update."""
    p2, m2, v2 = oadamw_orig(p, g, m, v, lr, wd, beta1, beta2, eps, step)
    if cautious:
        p2 = np.where(p2 * g > 0.0, p2, p)
    return p2, m2, v2


oadamw_orig = oadamw.adamw_update


@pytest.mark.parametrize("mutant", [_adamw_cautious_ge, _adamw_cautious_after_update], ids=lambda f: f.__name__)
def test_cautious_adamw_mutants_caught(mutant, monkeypatch):
    monkeypatch.setattr(oadamw, "adamw_update", mutant)
    with pytest.raises(AssertionError):
        pins.test_cautious_adamw_masks_against_the_gradient()


def test_grad_norm_without_sqrt_caught(monkeypatch):
    orig = ognorm.global_norm
    monkeypatch.setattr(ognorm, "global_norm", lambda grads: orig(grads) ** 2)
    with pytest.raises(AssertionError):
        pins.test_global_norm_and_clip_closed_forms()


def _clip_always(norm, max_norm):
    """Rescales to max_norm also when the norm is below it."""
    finite = math.isfinite(norm)
    return (max_norm / norm if (finite and max_norm > 0) else 1.0), not finite


def _clip_skip_when_large(norm, max_norm):
    """Skips the step when the norm exceeds max_norm instead of when it is not finite."""
    finite = math.isfinite(norm)
    big = max_norm > 0 and norm > max_norm
    return (max_norm / norm if (finite and big) else 1.0), (not finite) or big


def _clip_with_eps(norm, max_norm):
    """max_norm / (norm + 1e-6), the form some libraries use."""
    finite = math.isfinite(norm)
    return (max_norm / (norm + 1e-6) if (finite and max_norm > 0 and norm > max_norm) else 1.0), not finite


@pytest.mark.parametrize("mutant", [_clip_always, _clip_skip_when_large, _clip_with_eps], ids=lambda f: f.__name__)
def test_clip_mutants_caught(mutant, monkeypatch):
    monkeypatch.setattr(ognorm, "clip_state", mutant)
    with pytest.raises(AssertionError):
        pins.test_global_norm_and_clip_closed_forms()


def test_ns_table_reversed_caught(monkeypatch):
    orig = omuon.newton_schulz

    def reversed_table(M, steps=5, eps=1e-7, coeffs=omuon.NS_COEFFS, table=None, norm_scale=1.0):
        return orig(M, steps, eps, coeffs, None if table is None else list(table)[::-1], norm_scale)

    monkeypatch.setattr(omuon, "newton_schulz", reversed_table)
    with pytest.raises(AssertionError):
        pins.test_ns_table_closed_forms_and_order()


# -- the wide-model composition: Newton-Schulz -> Muon+ -> scale -> wrapper on G --
def _wrapper_fed_nesterov_q(W, G, Bm, V, views, hp, lr, wd):
    """The wrapper's mask taken against the Nesterov Q instead of the raw gradient."""
    beta = hp.get("beta", 0.95)
    B_new = omuon.momentum_ema(Bm, G, beta)
    Q = omuon.nesterov_lerp(G, B_new, beta)
    m = W.shape[1] // views
    Wn = np.empty_like(W)
    for b in range(W.shape[0]):
        for v in range(views):
            sl = slice(v * m, (v + 1) * m)
            Wn[b, sl], _, _ = omuon.matrix_update(Q[b, sl], W[b, sl], Q[b, sl], None, hp, lr, wd)
    return Wn, B_new, None, None


def _muon_plus_after_scale(Q, W, G, V, hp, lr, wd):
    """Muon+ applied to s*U: the normalisation then removes the shape scale."""
    m, n = Q.shape
    s = omuon.shape_scale(m, n)
    U = omuon.newton_schulz(Q)
    U_dir = omuon.muon_plus_row_col(s * U, hp.get("muon_plus_eps", 1e-8))
    W_new, _ = omuon.apply_cautious_wrapper(W, U_dir, G, lr, wd, 1.0)
    return W_new, V, U


def _mask_before_muon_plus(Q, W, G, V, hp, lr, wd):
    """The wrapper's mask decided on the Newton-Schulz output before Muon+."""
    m, n = Q.shape
    s = omuon.shape_scale(m, n)
    U = omuon.newton_schulz(Q)
    U_dir = omuon.muon_plus_row_col(U, hp.get("muon_plus_eps", 1e-8))
    delta = lr * wd * W + lr * s * U_dir
    mask = (lr * wd * W + lr * s * U) * G > 0.0
    return np.where(mask, W - delta, W), V, U


def test_wrapper_fed_nesterov_q_caught():
    with pytest.raises(AssertionError):
        pins.check_muon_plus_wrapper_step(_wrapper_fed_nesterov_q)


@pytest.mark.parametrize("mutant", [_muon_plus_after_scale, _mask_before_muon_plus], ids=lambda f: f.__name__)
def test_muon_plus_composition_mutants_caught(mutant, monkeypatch):
    monkeypatch.setattr(omuon, "matrix_update", mutant)
    with pytest.raises(AssertionError):
        pins.check_muon_plus_wrapper_step()


# -- the MoE composition: Newton-Schulz -> NorMuon (V carried) -> scale -> wd mask --
def _wd_mask_on_gradient(Q, W, G, V, hp, lr, wd):
    """The decay mask decided against the raw gradient instead of the update.
    (A mask on the Newton-Schulz output before NorMuon is no slip: NorMuon
    scales each row by a positive factor and keeps every sign.)"""
    m, n = Q.shape
    U = omuon.newton_schulz(Q)
    U_dir, V_new = omuon.normuon(U, V, hp.get("normuon_beta2", 0.95))
    s = omuon.shape_scale(m, n)
    keep = (G * W) >= 0.0
    return W - lr * s * U_dir - lr * wd * np.where(keep, W, 0.0), V_new, U


def _decay_scaled_by_shape(Q, W, G, V, hp, lr, wd):
    """The shape scale multiplies the decay term too."""
    m, n = Q.shape
    U = omuon.newton_schulz(Q)
    U_dir, V_new = omuon.normuon(U, V, hp.get("normuon_beta2", 0.95))
    s = omuon.shape_scale(m, n)
    return omuon.apply_cautious_wd(W, U_dir, lr, s * wd, s), V_new, U


def test_normuon_state_not_carried_caught(monkeypatch):
    plain = omuon.normuon
    monkeypatch.setattr(omuon, "normuon", lambda U, V, beta2: plain(U, np.zeros_like(V), beta2))
    with pytest.raises(AssertionError):
        pins.check_normuon_wdmask_two_steps()


@pytest.mark.parametrize("mutant", [_wd_mask_on_gradient, _decay_scaled_by_shape], ids=lambda f: f.__name__)
def test_normuon_composition_mutants_caught(mutant, monkeypatch):
    monkeypatch.setattr(omuon, "matrix_update", mutant)
    with pytest.raises(AssertionError):
        pins.check_normuon_wdmask_two_steps()


# -- bf16 moments: the stochastic-rounding key -----------------------------------
def _key_without_tensor(seed, step, leaf, moment):
    return _REAL_KEY(seed, step, 0, moment)


def _key_without_step(seed, step, leaf, moment):
    return _REAL_KEY(seed, 0, leaf, moment)


_REAL_KEY = ostorage.sr_key


@pytest.mark.parametrize("mutant", [_key_without_tensor, _key_without_step], ids=lambda f: f.__name__)
def test_rounding_key_mutants_caught(mutant, monkeypatch):
    monkeypatch.setattr(ostorage, "sr_key", mutant)
    with pytest.raises(AssertionError):
        pins.test_adamw_bf16_moments_use_the_step_tensor_and_moment_keys()


# -- the library pins (torch.optim.Muon, torch.optim.AdamW in float64) catch the
# -- same slips on their own ---------------------------------------------------
STEP_MUTANTS = [("momentum_ema", momentum_no_dampening), ("momentum_ema", momentum_swapped),
                ("nesterov_lerp", nesterov_old_sign), ("shape_scale", scale_swapped),
                ("shape_scale", scale_no_sqrt), ("apply_decoupled", decay_not_lr_scaled),
                ("apply_decoupled", decay_dropped), ("apply_decoupled", decay_after_update)]


@pytest.mark.parametrize("name,mutant", STEP_MUTANTS, ids=lambda x: x if isinstance(x, str) else x.__name__)
def test_torch_muon_pin_catches_step_mutants(name, mutant, monkeypatch):
    monkeypatch.setattr(omuon, name, mutant)
    with pytest.raises(AssertionError):
        pins.test_muon_steps_match_torch_optim_muon()


@pytest.mark.parametrize("mutant", [adamw_eps_inside, adamw_no_bias_correction, adamw_coupled_decay,
                                    adamw_bias_next_step, adamw_decay_not_lr_scaled], ids=lambda f: f.__name__)
def test_torch_adamw_pin_catches_adamw_mutants(mutant, monkeypatch):
    def wrapped(p, g, m, v, lr, wd, b1, b2, eps, step, cautious=False):
        return mutant(p, g, m, v, lr, wd, b1, b2, eps, step)
    monkeypatch.setattr(oadamw, "adamw_update", wrapped)
    with pytest.raises(AssertionError):
        pins.test_adamw_matches_torch_optim_adamw()
