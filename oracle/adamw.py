"""AdamW, fp64 CPU oracle (test infrastructure only).

Source: the dew.training.optim page (``OPTIMIZER_MAP`` routes 'adamw' to
optax.adamw; ``bf16_moments`` names optax's scale_by_adam state of two moments
and a step count) and the speedtronic "v2 optimizers" page ("CPU/CUDA/MPS
behavior": the torch AdamW). Both define the same update: Adam moments with
bias correction, eps added outside the square root (optax's eps_root is 0),
and decoupled weight decay scaled by the learning rate.
"""
import numpy as np

from . import storage


def adamw_update(p, g, m, v, lr, wd, beta1, beta2, eps, step):
    """One AdamW step in float64; ``step`` counts successful updates from 1."""
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * (m_hat / (np.sqrt(v_hat) + eps) + wd * p)
    return p, m, v


def adamw_step(tensors, hp):
    """``tensors``: dicts with param, param_dtype, grad, grad_dtype, m, v (float32),
    lr, wd. ``hp``: beta1, beta2, eps, step. Returns stored outputs + float64."""
    out = []
    for t in tensors:
        p = storage.decode(t["param"], t["param_dtype"])
        g = storage.decode(t["grad"], t["grad_dtype"])
        m = storage.decode(t["m"], "f32")
        v = storage.decode(t["v"], "f32")
        p2, m2, v2 = adamw_update(p, g, m, v, t["lr"], t["wd"], hp["beta1"], hp["beta2"],
                                  hp["eps"], hp["step"])
        out.append({"param": storage.round_to(p2, t["param_dtype"]),
                    "m": storage.round_f32(m2), "v": storage.round_f32(v2),
                    "p64": p2, "m64": m2, "v64": v2})
    return out
