"""Global gradient norm and clip, fp64 CPU oracle (test infrastructure only).

Sources: the dew.training.optim page, "build_optimizer" (the global-norm clip
reads every gradient together, before the parameter groups split them), and
the kimi-k3 "Optimization" chapter, "Keep the arithmetic and gradients under
control" (with max_grad_norm > 0 the global norm is clipped if necessary, with 0
it is only observed; an FP16 overflow skips the whole hybrid update).

Readings (listed in the design notes): the norm is the L2 norm over every
element of every gradient; clipping rescales by max_norm / ||g|| when ||g||
exceeds max_norm (optax's clip_by_global_norm); an overflow is a norm that is
not finite.
"""
import math

import numpy as np

from . import storage


def global_norm(grads):
    """``grads``: list of (stored array, dtype) or None. Returns ||g||_2 in fp64."""
    s = 0.0
    for g in grads:
        if g is None:
            continue
        x = storage.decode(g[0], g[1])
        s += float(np.sum(x * x))
    return math.sqrt(s)


def clip_state(norm, max_norm):
    """(factor, skip): factor = max_norm / norm when max_norm > 0 and the norm
    exceeds it, else 1; skip when the norm is not finite."""
    finite = math.isfinite(norm)
    factor = max_norm / norm if (finite and max_norm > 0 and norm > max_norm) else 1.0
    return factor, not finite
