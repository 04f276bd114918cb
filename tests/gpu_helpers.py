"""Glue shared by the GPU parity tests: run the HIP path through the binding,
feed the same stored inputs to the oracle, compare."""
import numpy as np
import torch

import muon_adamw_amd as ma
import workloads
from oracle import storage


def rel(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    d = np.linalg.norm(x - y)
    n = np.linalg.norm(y)
    return d / n if n > 0 else d


def check_local(got, want, tol, what=""):
    """Relative Frobenius error below `tol`, and no error concentrated in one
    place:
      - every row and every column within 3 tol of the average row (column)
        norm;
      - every 128 x 128 block within 3 tol of its own norm (at least half the
        average block norm);
      - every element within 6 tol of (RMS + |expected element|), which
        allows for the spikes that gradient outliers leave in the
        orthogonalised update.
    The CPU emulation of the bf16 chain (bf16 operands, fp32 sums) stays
    within 0.023 per row or column, 0.018 per block and 0.047 per element at
    the workload shapes (with 1% outliers x100 included), against a global
    error of 0.008-0.013; a wrong row, a tile 10% off or a single wrong
    element exceeds these bars while the Frobenius bar alone passes them."""
    x = np.asarray(got, dtype=np.float64)
    y = np.asarray(want, dtype=np.float64)
    e = rel(x, y)
    assert e < tol, (what, "frobenius", e)
    d = x - y
    fro = np.linalg.norm(y)
    if fro == 0:
        assert np.abs(d).max() == 0, (what, "nonzero where the oracle is zero")
        return e
    rms = fro / np.sqrt(y.size)
    elem = (np.abs(d) / (rms + np.abs(y))).max()
    assert elem < 6 * tol, (what, "element", elem)
    if y.ndim >= 2:
        y2, d2 = y.reshape(-1, y.shape[-1]), d.reshape(-1, y.shape[-1])
        m, n = y2.shape
        rows = np.linalg.norm(d2, axis=1).max() / (fro / np.sqrt(m))
        cols = np.linalg.norm(d2, axis=0).max() / (fro / np.sqrt(n))
        assert rows < 3 * tol, (what, "row", rows)
        assert cols < 3 * tol, (what, "column", cols)
        b = 128
        avg = fro * b / np.sqrt(m * n)          # norm of a full block at the average density
        worst = 0.0
        for i0 in range(0, m, b):
            for j0 in range(0, n, b):
                yb, db = y2[i0:i0 + b, j0:j0 + b], d2[i0:i0 + b, j0:j0 + b]
                floor = 0.5 * avg * np.sqrt(yb.size) / b
                worst = max(worst, np.linalg.norm(db) / max(np.linalg.norm(yb), floor))
        assert worst < 3 * tol, (what, "block", worst)
    return e


def bf16_ulps(got_bits, want_bits):
    """Distance in bf16 units in the last place (sign-magnitude bit patterns
    mapped onto a monotone integer line)."""
    def line(b):
        b = np.asarray(b, dtype=np.int64) & 0xFFFF
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(line(got_bits) - line(want_bits))


def host(t):
    """Stored values of a tensor as float64 (bf16 decoded by the oracle's rule)."""
    a = workloads.to_numpy(t)
    return storage.decode(a, "bf16" if t.dtype == torch.bfloat16 else "f32")


def hp_c(h: workloads.MuonHParams):
    return ma.muon_hparams(h.beta, h.nesterov, h.ns_steps, h.ns_coeffs, h.ns_eps, h.ns_dtype, h.normuon,
                           h.normuon_beta2, h.muon_plus, h.muon_plus_eps, h.cautious)


def hp_dict(h: workloads.MuonHParams):
    return {"beta": h.beta, "nesterov": h.nesterov, "ns_steps": h.ns_steps, "ns_coeffs": h.ns_coeffs,
            "ns_eps": h.ns_eps, "normuon": h.normuon, "normuon_beta2": h.normuon_beta2,
            "muon_plus": h.muon_plus, "muon_plus_eps": h.muon_plus_eps, "cautious": h.cautious}


def muon_params(data: workloads.WorkloadData):
    return [ma.MuonParam(t.param, t.grad, t.momentum, t.row_v, t.spec.views, t.spec.lr, t.spec.wd)
            for t in data.muon if t is not None]


def adamw_params(data: workloads.WorkloadData):
    return [ma.AdamWParam(t.param, t.grad, t.m, t.v, t.spec.lr, t.spec.wd) for t in data.adamw]


def snapshot(t):
    return None if t is None else t.detach().clone()


def to_gpu(data: workloads.WorkloadData, device="cuda"):
    for t in data.muon:
        if t is None:
            continue
        t.param = t.param.to(device)
        t.grad = None if t.grad is None else t.grad.to(device)
        t.momentum = t.momentum.to(device)
        t.row_v = None if t.row_v is None else t.row_v.to(device)
    for t in data.adamw:
        t.param, t.grad, t.m, t.v = (x.to(device) for x in (t.param, t.grad, t.m, t.v))
    return data


def flush(msg):
    print(msg, flush=True)


def bf16_spacing(v):
    """Spacing of bf16 values at |v| (8 significant bits)."""
    _, e = np.frexp(np.abs(np.asarray(v, dtype=np.float64)))
    return np.where(v == 0, 2.0 ** -133, np.ldexp(1.0, e - 8))


def check_update(W_gpu, W0, W_want, G, U_dir, h, lr, wd, s, param_dtype, tol, tol_ns):
    """The stored parameters against the oracle's.

    A cautious mask is a decision on the update direction, which the two
    sides compute to different precision: an element may take the other
    branch only where the oracle's own margin is inside the direction's
    element bar (6 tol_ns of the RMS update), and then it is compared with
    the branch it is closer to (both branches rounded to the parameter
    dtype). Inside that band the two branches often differ by less than the
    update's element bar (the weight-decay mask moves an element by lr wd W
    only), so being closer to the other branch says nothing. A flip counts
    where the value is outside the element bar of the expected branch: at
    most 3% of elements with bf16 Newton-Schulz, 0.1% with fp32. The kernel
    sources on the CPU simulator put 1.2-4.6% of elements closer to the
    other branch on the small mixed shapes and flip none.

    fp32 parameters: the update W - W0 within `tol` of the oracle's, under
    the localized bars. bf16 parameters: every element within one bf16
    spacing of the oracle's rounded value plus the update's element bar (6
    tol of its RMS plus its own size); with bf16 Newton-Schulz also the
    update within `tol` (relative Frobenius); with fp32 Newton-Schulz at most
    0.1% of the elements one spacing off (there one straddled rounding
    boundary moves a whole bf16 spacing, a large relative error on an update
    of a few spacings, so the Frobenius measure says nothing)."""
    lr_s_U = lr * s * U_dir
    band = 6 * tol_ns * np.sqrt(np.mean(lr_s_U * lr_s_U))
    if h["cautious"] == "wd_mask":
        alt = W0 - lr_s_U - lr * wd * np.where((U_dir * W0) >= 0.0, 0.0, W0)
        near = np.abs(lr_s_U) < band
    elif h["cautious"] == "wrapper":
        delta = lr * wd * W0 + lr_s_U
        alt = np.where((delta * G) > 0.0, W0, W0 - delta)
        near = np.abs(delta) < band
    else:
        alt, near = W_want, np.zeros(W_want.shape, dtype=bool)
    rounded = lambda x: storage.decode(storage.round_to(x, param_dtype), param_dtype)
    R_want, R_alt = rounded(W_want), rounded(alt)
    closer = near & (np.abs(W_gpu - R_alt) < np.abs(W_gpu - R_want))
    dW0 = W_want - W0
    bar = 6 * tol * (np.sqrt(np.mean(dW0 * dW0)) + np.abs(dW0))
    if param_dtype == "bf16":
        bar = bar + bf16_spacing(R_want)
    flipped = closer & (np.abs(W_gpu - R_want) > bar)
    loose = tol_ns > 1e-3
    assert flipped.mean() <= (0.03 if loose else 1e-3), ("mask flips", float(flipped.mean()))
    exact = np.where(closer, alt, W_want)
    W_ref = np.where(closer, R_alt, R_want)
    if param_dtype == "bf16":
        dW = exact - W0
        allowed = bf16_spacing(W_ref) + 6 * tol * (np.sqrt(np.mean(dW * dW)) + np.abs(dW))
        worst = (np.abs(W_gpu - W_ref) / allowed).max()
        assert worst <= 1.0, ("bf16 element", float(worst))
        if loose:
            e = np.linalg.norm((W_gpu - W0) - (W_ref - W0)) / np.linalg.norm(W_ref - W0)
            assert e < tol, ("update", e)
        else:
            share = float((W_gpu != W_ref).mean())
            assert share <= 1e-3, ("bf16 spacing share", share)
    else:
        check_local(W_gpu - W0, W_ref - W0, tol, "update")
