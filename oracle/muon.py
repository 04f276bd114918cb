"""Muon matrix update, fp64 CPU oracle (test infrastructure only).

Sources, by page title and section:

* speedtronic "v2 optimizers" page -- "Newton-Schulz" section (quintic iteration,
  coefficients (3.4445, -4.7750, 2.0315), 5 steps, eps 1e-7, tall matrices
  transposed internally, zero matrices stay finite), "Muon update" section
  (momentum EMA, Nesterov lerp, shape scale max(1, rows/columns)^0.5, decoupled
  weight decay, FP32 momentum), "Muon+" section (row_col normalisation with eps
  inside each square root) and "Cautious updates" section (mask from the
  observed update times the gradient, decay included).
* flaxchat "Optimizer" page -- "Muon Algorithm" steps 1-4 (the same momentum and
  Nesterov form, the wide/tall forms of the iteration, NorMuon variance
  reduction, cautious weight decay).
* kimi-k3 "Optimization" chapter -- "A tensor's storage shape can be misleading"
  (a packed gate/up parameter registered as (2, rows, columns) is two matrices;
  state is not duplicated) and the guarantee that an expert without gradient
  is neither moved nor decayed.

Readings where the pages are silent or disagree (each is listed in the design
notes): normalisation divides by (||X||_F * s + eps) with s = 1 by default, the
speedtronic form, and s = 1.01 giving flaxchat's ||g||*1.01 (with its eps); the
same (a, b, c) is used in every iteration unless a per-iteration table is given
(flaxchat "Muon Algorithm" step 2 loops over a list of triples); "tall" means
rows > cols; the shape scale uses the view's own (rows, cols); NorMuon reduces
over each stored row and rescales to preserve ||U||_F; Muon+ normalises to unit
L2 norm; the order is NS -> (NorMuon | Muon+) -> scale -> decay/apply.
"""
import numpy as np

from . import storage

NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_STEPS = 5
NS_EPS = 1e-7
TINY = 1e-30


# -- speedtronic "Muon update": B <- momentum*B + (1 - momentum)*gradient ------
def momentum_ema(B, G, beta):
    return beta * B + (1.0 - beta) * G


# -- speedtronic "Muon update": Q <- lerp(gradient, B, momentum) (Nesterov) ----
def nesterov_lerp(G, B, beta):
    return G + beta * (B - G)


# -- speedtronic "Newton-Schulz" section ----------------------------------------
def newton_schulz(M, steps=NS_STEPS, eps=NS_EPS, coeffs=NS_COEFFS, table=None, norm_scale=1.0):
    """Quintic Newton-Schulz: transpose a tall matrix, normalise by its Frobenius
    norm (times norm_scale) plus eps, iterate A = X X^T; X <- aX + (bA + cA^2)X,
    transpose back. ``table``: one (a, b, c) per iteration, else ``coeffs`` for
    every iteration."""
    X = np.array(M, dtype=np.float64, copy=True)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = X / (np.linalg.norm(X) * norm_scale + eps)
    for i in range(steps):
        a, b, c = coeffs if table is None else table[i]
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    if tall:
        X = X.T
    return X


# -- speedtronic "Muon update": max(1, rows/columns)^0.5 ------------------------
def shape_scale(m, n):
    return max(1.0, m / n) ** 0.5


# -- flaxchat "Muon Algorithm" step 3: NorMuon variance reduction ----------------
def normuon(U, V, beta2):
    """v_mean = mean(U^2) over each stored row; V <- lerp(V, v_mean, 1 - beta2);
    U <- U * rsqrt(V) per row, rescaled so ||U||_F is preserved."""
    v_mean = np.mean(U * U, axis=1)
    V_new = V + (1.0 - beta2) * (v_mean - V)
    U_hat = U * (np.maximum(V_new, TINY) ** -0.5)[:, None]
    scale = np.linalg.norm(U) / max(np.linalg.norm(U_hat), TINY)
    return U_hat * scale, V_new


# -- speedtronic "Muon+": rows first, then columns, eps inside each sqrt --------
def muon_plus_row_col(U, eps):
    U = U / np.sqrt(np.sum(U * U, axis=1, keepdims=True) + eps)
    U = U / np.sqrt(np.sum(U * U, axis=0, keepdims=True) + eps)
    return U


# -- the apply step in its three forms ------------------------------------------
def apply_decoupled(W, U, lr, wd, s):
    """speedtronic "Muon update": W <- (1 - lr*wd) W - lr * s * U."""
    return (1.0 - lr * wd) * W - lr * s * U


def apply_cautious_wd(W, U, lr, wd, s):
    """flaxchat "Muon Algorithm" step 4: the decay term only where U*W >= 0."""
    mask = (U * W) >= 0.0
    return W - lr * s * U - lr * wd * np.where(mask, W, 0.0)


def apply_cautious_wrapper(W, U, G, lr, wd, s):
    """speedtronic "Cautious updates": the observed update (decay included) is
    kept only where it times the gradient is > 0; elsewhere W is unchanged."""
    delta = lr * wd * W + lr * s * U
    mask = (delta * G) > 0.0
    return np.where(mask, W - delta, W), mask


def matrix_update(Q, W, G, V, hp, lr, wd):
    """One matrix (one view of one batch entry), all in float64.

    Returns (W_new, V_new, U) with U the Newton-Schulz output (before NorMuon or
    Muon+) in the stored m x n orientation.
    """
    m, n = Q.shape
    U = newton_schulz(Q, hp.get("ns_steps", NS_STEPS), hp.get("ns_eps", NS_EPS),
                      hp.get("ns_coeffs", NS_COEFFS), hp.get("ns_table"), hp.get("ns_norm_scale", 1.0))
    U_dir = U
    V_new = V
    if hp.get("normuon", False):
        U_dir, V_new = normuon(U_dir, V, hp.get("normuon_beta2", 0.95))
    if hp.get("muon_plus", False):
        U_dir = muon_plus_row_col(U_dir, hp.get("muon_plus_eps", 1e-8))
    s = shape_scale(m, n)
    mode = hp.get("cautious", "none")
    if mode == "none":
        W_new = apply_decoupled(W, U_dir, lr, wd, s)
    elif mode == "wd_mask":
        W_new = apply_cautious_wd(W, U_dir, lr, wd, s)
    elif mode == "wrapper":
        W_new, _ = apply_cautious_wrapper(W, U_dir, G, lr, wd, s)
    else:
        raise ValueError(f"unknown cautious mode {mode!r}")
    return W_new, V_new, U


def muon_tensor_step(W, G, B, V, views, hp, lr, wd):
    """One parameter tensor of shape (batch, rows, cols) in float64.

    An absent gradient (G is None) leaves parameter and state untouched
    (kimi-k3 "Optimization": an expert with no gradient is not decayed).
    Momentum and the NorMuon second moment belong to the packed parent; each
    view's rows are one matrix (kimi-k3, matrix views).

    Returns (W_new, B_new, V_new, U) in float64; U holds the per-matrix
    Newton-Schulz outputs stacked like W.
    """
    if G is None:
        return W.copy(), B.copy(), None if V is None else V.copy(), None
    beta = hp.get("beta", 0.95)
    B_new = momentum_ema(B, G, beta)
    Q = nesterov_lerp(G, B_new, beta) if hp.get("nesterov", True) else B_new
    batch, rows, cols = W.shape
    m = rows // views
    W_new = np.empty_like(W)
    U_all = np.empty_like(W)
    V_new = None if V is None else np.empty_like(V)
    for b in range(batch):
        for v in range(views):
            sl = slice(v * m, (v + 1) * m)
            Vv = None if V is None else V[b, sl]
            Wn, Vn, U = matrix_update(Q[b, sl], W[b, sl], G[b, sl], Vv, hp, lr, wd)
            W_new[b, sl] = Wn
            U_all[b, sl] = U
            if V is not None:
                V_new[b, sl] = Vn if Vn is not None else Vv
    return W_new, B_new, V_new, U_all


def muon_step(tensors, hp, clip=None):
    """Whole Muon half of the hybrid step.

    ``clip``: (factor, skip) from the global-norm clip (oracle.gradnorm), or
    None. The gradient enters scaled by the factor; a skipped step returns
    every stored input unchanged (kimi-k3 "Optimization": an overflow skips the
    whole hybrid update).

    ``tensors``: list of dicts with stored inputs
      param (array, float32 or bf16 bits), param_dtype, grad (or None),
      grad_dtype, momentum (float32), row_v (float32 or None), views, lr, wd,
      shape (batch, rows, cols).
    Returns a list of dicts with the stored outputs (param in its dtype,
    momentum and row_v as float32) and the float64 intermediates.
    """
    out = []
    for t in tensors:
        shape = t["shape"]
        W = storage.decode(t["param"], t["param_dtype"]).reshape(shape)
        G = None if t["grad"] is None else storage.decode(t["grad"], t["grad_dtype"]).reshape(shape)
        if clip is not None and clip[1]:
            out.append({"param": np.array(t["param"], copy=True), "momentum": np.array(t["momentum"], copy=True),
                        "row_v": None if t.get("row_v") is None else np.array(t["row_v"], copy=True),
                        "W64": None, "B64": None, "V64": None, "U64": None})
            continue
        if clip is not None and G is not None:
            G = clip[0] * G
        B = storage.decode(t["momentum"], "f32").reshape(shape)
        V = None if t.get("row_v") is None else storage.decode(t["row_v"], "f32").reshape(shape[0], shape[1])
        W_new, B_new, V_new, U = muon_tensor_step(W, G, B, V, t.get("views", 1), hp, t["lr"], t["wd"])
        out.append({
            "param": storage.round_to(W_new, t["param_dtype"]),
            "momentum": storage.round_f32(B_new),
            "row_v": None if V_new is None else storage.round_f32(V_new),
            "W64": W_new, "B64": B_new, "V64": V_new, "U64": U,
        })
    return out
