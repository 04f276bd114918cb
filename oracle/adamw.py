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


def adamw_update(p, g, m, v, lr, wd, beta1, beta2, eps, step, cautious=False):
    """One AdamW step in float64; ``step`` counts successful updates from 1.

    ``cautious``: the speedtronic "Cautious updates" wrapper over AdamW (the
    wrapper applies to either base optimizer): the observed update p - p_new,
    decay included, is kept only where it times the gradient is > 0;
    elsewhere p stays as it was. The moments are the base optimizer's either
    way (the section leaves AdamW's own state untouched by the mask)."""
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p_new = p - lr * (m_hat / (np.sqrt(v_hat) + eps) + wd * p)
    if cautious:
        p_new = np.where((p - p_new) * g > 0.0, p_new, p)
    return p_new, m, v


def adamw_step(tensors, hp, clip=None):
    """``tensors``: dicts with param, param_dtype, grad, grad_dtype, m, v, lr, wd
    and optionally moment_dtype ("f32" default, or "bf16": uint16 bits).
    ``hp``: beta1, beta2, eps, step, optionally cautious, seed. ``clip``:
    (factor, skip) from oracle.gradnorm or None. Returns stored outputs and
    the float64 values.

    bf16 moments (dew.training.optim "bf16_moments"): widened to fp32 for the
    update, the new fp32 moments written back with stochastic_round_bf16,
    seeded by (seed, step, tensor index, moment) as in storage.sr_key."""
    out = []
    for k, t in enumerate(tensors):
        mdt = t.get("moment_dtype", "f32")
        if clip is not None and clip[1]:
            out.append({"param": np.array(t["param"], copy=True), "m": np.array(t["m"], copy=True),
                        "v": np.array(t["v"], copy=True), "p64": None, "m64": None, "v64": None})
            continue
        p = storage.decode(t["param"], t["param_dtype"])
        g = storage.decode(t["grad"], t["grad_dtype"])
        if clip is not None:
            g = clip[0] * g
        m = storage.decode(t["m"], mdt)
        v = storage.decode(t["v"], mdt)
        p2, m2, v2 = adamw_update(p, g, m, v, t["lr"], t["wd"], hp["beta1"], hp["beta2"],
                                  hp["eps"], hp["step"], hp.get("cautious", False))
        if mdt == "bf16":
            seed, step = hp.get("seed", 0), hp["step"]
            ms = storage.stochastic_round_bf16_bits(storage.round_f32(m2), storage.sr_key(seed, step, k, 0))
            vs = storage.stochastic_round_bf16_bits(storage.round_f32(v2), storage.sr_key(seed, step, k, 1))
        else:
            ms, vs = storage.round_f32(m2), storage.round_f32(v2)
        out.append({"param": storage.round_to(p2, t["param_dtype"]), "m": ms, "v": vs,
                    "p64": p2, "m64": m2, "v64": v2})
    return out
