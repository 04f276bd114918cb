"""Stricter checks of the HIP path against the fp64 oracle (needs an MI355X).

- Localized bars (``check_local``: rows, columns, 128 x 128 blocks, elements)
  on every Newton-Schulz output and every fp32 parameter update, besides the
  relative Frobenius bar; bf16 parameters element by element within one bf16
  spacing of the oracle's rounded result plus the update's element bar.
- The device status of every step (``muon_step_status``) is 0, and on an
  MI355X the persistent Newton-Schulz launch is the one that runs.
- The epilogues (NorMuon, Muon+ row_col, both cautious masks) with fp32
  Newton-Schulz, where the whole chain is within 1e-5 of the oracle, so the
  epilogue arithmetic is checked at that precision.
- Gradients near the top of the fp32 range: the global norm clips instead of
  skipping, and Newton-Schulz stays finite and scale-free.
- The wide-model workload's 28672 x 8192 bucket at full size, through
  properties that hold at any size, and (last, marked slow) one such matrix
  in the workload's full step against the oracle's whole chain (about 44
  TFLOP of fp64 host arithmetic).

Every expected value comes from the oracle run on the stored inputs, or from
a closed property of the Newton-Schulz map.
"""
import ctypes
import math
import os

import numpy as np
import pytest
import torch

import muon_adamw_amd as ma
import workloads
from oracle import adamw as oadamw
from oracle import gradnorm as ognorm
from oracle import muon as omuon
from oracle import storage
from tests.gpu_helpers import check_local, check_update, flush, host, hp_c, hp_dict, muon_params, to_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def randn(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32) * scale


def ns_with_status(x, hp):
    """Newton-Schulz alone through the binding, with its own workspace so
    that the step's status can be read back."""
    need = ma.load_library().ma_newton_schulz_workspace_bytes(
        *((1, *x.shape) if x.dim() == 2 else tuple(x.shape)), ma._dtype_code(x), ctypes.byref(hp))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    out = ma.newton_schulz(x, hp, workspace=ws)
    assert ma.muon_step_status(ws) == 0
    return out


# ---------------------------------------------------------------------------
# Newton-Schulz alone, localized bars
# ---------------------------------------------------------------------------
BF16_SHAPES = [(1, 1), (7, 3), (128, 128), (300, 200), (200, 300), (129, 1000), (768, 768), (768, 3072),
               (3072, 768), (1408, 2048), (2304, 2560)]


@pytest.mark.parametrize("shape", BF16_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_newton_schulz_bf16_local(shape):
    flush(f"ns bf16 local {shape}")
    x = randn(shape, 300 + shape[0] + 5 * shape[1]).to(torch.bfloat16)
    out = ns_with_status(x.to(DEV), ma.muon_hparams(ns_dtype="bf16"))
    check_local(host(out), omuon.newton_schulz(host(x)), 2e-2, shape)


F32_SHAPES = [(1, 1), (4, 3), (37, 100), (100, 37), (128, 256), (256, 128), (64, 300), (384, 128)]


@pytest.mark.parametrize("shape", F32_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_newton_schulz_f32_local(shape):
    """fp32 throughout, aspect ratio >= 2 (or trivially small): 1e-5 with the
    localized bars."""
    flush(f"ns f32 local {shape}")
    x = randn(shape, 400 + 3 * shape[0] + shape[1])
    out = ns_with_status(x.to(DEV), ma.muon_hparams(ns_dtype="f32"))
    check_local(out.cpu().double().numpy(), omuon.newton_schulz(x.double().numpy()), 1e-5, shape)


# ---------------------------------------------------------------------------
# Whole steps: status, localized bars, narrow mask-flip bands
# ---------------------------------------------------------------------------
def oracle_inputs(data):
    return [{"param": workloads.to_numpy(t.param), "param_dtype": t.spec.param_dtype,
             "grad": None if t.grad is None else workloads.to_numpy(t.grad), "grad_dtype": t.spec.grad_dtype,
             "momentum": workloads.to_numpy(t.momentum),
             "row_v": None if t.row_v is None else workloads.to_numpy(t.row_v),
             "views": t.spec.views, "lr": t.spec.lr, "wd": t.spec.wd, "shape": t.spec.shape}
            for t in data.muon if t is not None]


def run_step_checked(wl, tol_ns, sample=None, update_tol=None):
    """One Muon step of workload `wl` on the GPU; its status; per matrix (all,
    or those `sample` picks): momentum at 1e-5, the oracle's whole chain for
    the Newton-Schulz output (localized bars at tol_ns), NorMuon's V (twice
    tol_ns) and the stored parameters (check_update). `sample` is a set of matrix indices
    or a predicate on (index, matrix_info)."""
    h = hp_dict(wl.muon_hp)
    data = to_gpu(workloads.generate(wl, device="cpu" if wl.gen_device == "cpu" else DEV))
    params = muon_params(data)
    hp = hp_c(wl.muon_hp)
    nmat, _ = ma.plan_counts(params, hp)
    infos = [ma.matrix_info(params, hp, kk) for kk in range(nmat)]
    picked = sample if callable(sample) else (lambda kk, info: sample is None or kk in sample)
    sel = [kk for kk in range(nmat) if picked(kk, infos[kk])]
    assert sel, "no matrix picked"
    tens = sorted({infos[kk]["tensor"] for kk in sel})
    before = {ti: (data.muon[ti].param.clone(), data.muon[ti].momentum.clone(),
                   None if data.muon[ti].row_v is None else data.muon[ti].row_v.clone()) for ti in tens}
    flush(f"workload {wl.name}: muon_step, {len(sel)} of {nmat} matrices checked")
    ws = ma.muon_step(params, hp)
    assert ma.muon_step_status(ws) == 0
    for kk in sel:
        info = infos[kk]
        t = data.muon[info["tensor"]]
        m, n, bi, v = info["m"], info["n"], info["batch_index"], info["view"]
        rs = slice(v * m, (v + 1) * m)
        pick = (lambda x: x[bi, rs]) if t.param.dim() == 3 else (lambda x: x[rs])
        b = before[info["tensor"]]
        W0, G, B0 = host(pick(b[0])), host(pick(t.grad)), host(pick(b[1]))
        V0 = None if b[2] is None else host(b[2][bi, rs])
        B1 = omuon.momentum_ema(B0, G, h["beta"])
        check_local(host(pick(t.momentum)), B1, 1e-5, (kk, "momentum"))
        Q = omuon.nesterov_lerp(G, B1, h["beta"]) if h["nesterov"] else B1
        W_want, V_want, U_want = omuon.matrix_update(Q, W0, G, V0, h, t.spec.lr, t.spec.wd)
        U = ma.workspace_u(ws, info, wl.muon_hp.ns_dtype).cpu().float().double().numpy()[: info["r"], : info["c"]]
        check_local(U.T if info["transposed"] else U, U_want, tol_ns, (kk, "newton-schulz"))
        if V0 is not None:
            check_local(host(t.row_v[bi, rs]), V_want, 2 * tol_ns, (kk, "normuon V"))
        U_dir = U_want
        if h["normuon"]:
            U_dir, _ = omuon.normuon(U_dir, V0, h["normuon_beta2"])
        if h["muon_plus"]:
            U_dir = omuon.muon_plus_row_col(U_dir, h["muon_plus_eps"])
        tol_p = update_tol or (2 if t.spec.param_dtype == "f32" else 3) * tol_ns
        check_update(host(pick(t.param)), W0, W_want, G, U_dir, h, t.spec.lr, t.spec.wd,
                     omuon.shape_scale(m, n), t.spec.param_dtype, tol_p, tol_ns)
    return data, ws


def aspect2_workload(name, seed, **hp):
    """Tall, packed and wide matrices of aspect ratio >= 2, where fp32
    Newton-Schulz reaches 1e-5 of the oracle."""
    pd = hp.pop("param_dtype", "f32")
    specs = (workloads.MuonTensorSpec("a", 1, 384, 128, param_dtype=pd, grad_dtype=pd),
             workloads.MuonTensorSpec("b", 2, 2 * 64, 160, views=2, param_dtype=pd, grad_dtype=pd),
             workloads.MuonTensorSpec("c", 1, 64, 500, param_dtype=pd, grad_dtype=pd))
    return workloads.Workload(name, seed, specs, (), workloads.MuonHParams(**hp))


@pytest.mark.parametrize("variant", [
    dict(),
    dict(muon_plus=True, cautious="wrapper"),
    dict(normuon=True, cautious="wd_mask"),
    dict(muon_plus=True, cautious="wrapper", param_dtype="bf16"),
    dict(normuon=True, cautious="wd_mask", param_dtype="bf16"),
], ids=lambda d: "-".join(f"{k}={v}" for k, v in d.items()) or "default")
def test_epilogues_with_fp32_newton_schulz(variant):
    """NorMuon, Muon+ row_col, both cautious masks and the bf16 store with
    fp32 Newton-Schulz: the Newton-Schulz output and the fp32 update within
    1e-5 of the oracle's whole chain, under the localized bars."""
    wl = aspect2_workload("epilogue_f32", 41, ns_dtype="f32", **variant)
    run_step_checked(wl, 1e-5, update_tol=1e-5)


@pytest.mark.parametrize("variant", [
    dict(),
    dict(muon_plus=True, cautious="wrapper"),
    dict(normuon=True, cautious="wd_mask"),
    dict(muon_plus=True, cautious="wrapper", param_dtype="bf16"),
], ids=lambda d: "-".join(f"{k}={v}" for k, v in d.items()) or "default")
def test_epilogues_with_bf16_newton_schulz(variant):
    wl = aspect2_workload("epilogue_bf16", 42, ns_dtype="bf16", **variant)
    run_step_checked(wl, 2e-2)


def test_gpt_12L_d768_local():
    """All 72 matrices of the GPT workload under the localized bars."""
    run_step_checked(workloads.workload(2), 2e-2)


def test_moe_64x2048_wider_sample():
    """16 of the 192 expert matrices (gate and up views, down), spread over
    the experts, under the localized bars: NorMuon and the weight-decay mask."""
    sample = {0, 1, 30, 31, 62, 63, 64, 65, 100, 127, 128, 129, 150, 170, 190, 191}
    run_step_checked(workloads.workload(4), 2e-2, sample=sample)


def test_llama_8L_d4096_local():
    """Layer 0 of the Llama workload (bf16 parameters and gradients, 1% of the
    gradient x100) under the localized bars: the second view of the packed
    gate_up (14336 x 4096, tall, at a nonzero offset in its parent) and down
    (4096 x 14336, wide)."""
    run_step_checked(workloads.workload(3), 2e-2,
                     sample=lambda kk, info: (info["tensor"] == 4 and info["view"] == 1) or info["tensor"] == 5)


def test_single_256x128_f32_local():
    run_step_checked(workloads.workload(1), 1e-5, update_tol=1e-5)


# ---------------------------------------------------------------------------
# Schedule in use and status under both schedules
# ---------------------------------------------------------------------------
def test_persistent_schedule_runs_and_reports_ok():
    """On an MI355X (one device of 8 XCDs) the GPT workload's Newton-Schulz
    runs as the one persistent launch followed by its status check, and the
    status is 0; with one launch per product the status is 0 as well."""
    wl = workloads.workload(2)
    data = to_gpu(workloads.generate(wl, device="cpu"))
    hp = hp_c(wl.muon_hp)
    ma.profile_begin()
    ws = ma.muon_step(muon_params(data), hp)
    names = set(ma.profile_end())
    assert {"ns_persistent_bf16", "ns_status"} <= names, names
    assert ma.muon_step_status(ws) == 0
    os.environ["MA_NS_SCHEDULE"] = "launches"
    try:
        ma.profile_begin()
        ws = ma.muon_step(muon_params(data), hp, workspace=ws)
        names = set(ma.profile_end())
    finally:
        del os.environ["MA_NS_SCHEDULE"]
    assert "ns_persistent_bf16" not in names and "ns_apply_bf16" in names, names
    assert ma.muon_step_status(ws) == 0


# ---------------------------------------------------------------------------
# Gradients near the top of the fp32 range
# ---------------------------------------------------------------------------
def test_huge_gradients_clip_instead_of_skipping():
    """Gradients of magnitude ~1e20 (their squares overflow fp32): the global
    norm is finite and within 1e-6 of the oracle's, so the step is clipped,
    not skipped; the clipped Muon (fp32 Newton-Schulz) and AdamW steps match
    the oracle's."""
    wl = aspect2_workload("huge_clip", 43, ns_dtype="f32")
    data = to_gpu(workloads.generate(wl, device="cpu"))
    for t in data.muon:
        t.grad.mul_(1e23)                           # grad_std 1e-3 -> ~1e20
    inp = oracle_inputs(data)
    n = 70000
    p, g = randn((n,), 90, 0.02), randn((n,), 91, 1e20)
    ap = [ma.AdamWParam(p.clone().to(DEV), g.clone().to(DEV), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV),
                        1e-3, 0.1)]
    grads = [t.grad for t in data.muon] + [ap[0].grad]
    want_norm = ognorm.global_norm([(workloads.to_numpy(x), "f32") for x in grads])
    assert math.isfinite(want_norm) and want_norm > 1e21
    state = ma.global_grad_norm(grads, 1.0)
    st = state.cpu().numpy()
    assert st[2] == 0.0 and abs(st[0] - want_norm) / want_norm < 1e-6
    clip = ognorm.clip_state(want_norm, 1.0)
    assert abs(st[1] - clip[0]) / clip[0] < 1e-6
    h = wl.muon_hp
    hpc = ma.muon_hparams(h.beta, h.nesterov, h.ns_steps, h.ns_coeffs, h.ns_eps, h.ns_dtype, clip=state)
    ws = ma.muon_step(muon_params(data), hpc)
    ma.adamw_step(ap, 0.9, 0.999, 1e-8, 1, clip=state)
    assert ma.muon_step_status(ws) == 0
    want = omuon.muon_step(inp, hp_dict(h), clip=clip)
    for t, w, i in zip(data.muon, want, inp):
        W0 = storage.decode(i["param"], "f32").reshape(w["W64"].shape)
        check_local(host(t.param) - W0, w["W64"] - W0, 1e-5, "clipped update")
        check_local(host(t.momentum), w["B64"], 1e-5, "clipped momentum")
    wa = oadamw.adamw_step([{"param": workloads.to_numpy(p), "param_dtype": "f32",
                             "grad": workloads.to_numpy(g), "grad_dtype": "f32",
                             "m": np.zeros(n, np.float32), "v": np.zeros(n, np.float32), "lr": 1e-3, "wd": 0.1}],
                           {"beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "step": 1}, clip=clip)[0]
    check_local(host(ap[0].param), wa["p64"], 1e-6, "clipped adamw")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [1e25, 1e-25])
def test_newton_schulz_is_scale_free_at_the_range_ends(dtype, scale):
    """Newton-Schulz of X times 1e25 (whose first Gram would overflow fp32
    without the power-of-two rescale) or 1e-25 equals the oracle's
    Newton-Schulz of the same stored input."""
    flush(f"ns scale {scale} {dtype}")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    x = (randn((384, 128), 95) * scale).to(tdt)
    out = ns_with_status(x.to(DEV), ma.muon_hparams(ns_dtype=dtype))
    got = out.cpu().double().numpy() if dtype == "f32" else host(out)
    assert np.isfinite(got).all()
    xin = x.double().numpy() if dtype == "f32" else host(x)
    check_local(got, omuon.newton_schulz(xin), 1e-5 if dtype == "f32" else 2e-2, (scale, dtype))


def test_huge_gradients_without_clip_step_like_the_oracle():
    """No clip state: a Muon step on gradients ~1e20 (bf16 Newton-Schulz).
    Momentum is 0.05 G, and since Newton-Schulz is scale-free the update is
    the oracle's: the Newton-Schulz output and the update under the localized
    bars."""
    wl = aspect2_workload("huge_noclip", 44, ns_dtype="bf16")
    data = to_gpu(workloads.generate(wl, device="cpu"))
    for t in data.muon:
        t.grad.mul_(1e23)
    h = hp_dict(wl.muon_hp)
    params = muon_params(data)
    hp = hp_c(wl.muon_hp)
    W0s = [host(t.param) for t in data.muon]
    inp = oracle_inputs(data)
    ws = ma.muon_step(params, hp)
    assert ma.muon_step_status(ws) == 0
    want = omuon.muon_step(inp, h)
    k = 0
    for ti, (t, w) in enumerate(zip(data.muon, want)):
        check_local(host(t.momentum), w["B64"], 1e-5, (ti, "momentum"))
        check_local(host(t.param) - W0s[ti], w["W64"] - W0s[ti], 4e-2, (ti, "update"))
        for _ in range(t.spec.batch * t.spec.views):
            info = ma.matrix_info(params, hp, k)
            U = ma.workspace_u(ws, info, "bf16").cpu().float().double().numpy()[: info["r"], : info["c"]]
            m = info["m"]
            rs = slice(info["view"] * m, (info["view"] + 1) * m)
            Uw = w["U64"][info["batch_index"], rs]
            check_local(U.T if info["transposed"] else U, Uw, 2e-2, (k, "newton-schulz"))
            k += 1


# ---------------------------------------------------------------------------
# The wide-model workload's 28672 x 8192 bucket at full size
# ---------------------------------------------------------------------------
def test_wide_4L_d8192_tall_bucket_properties():
    """The MLP up projection of the wide-model workload (28672 x 8192, bf16)
    through Newton-Schulz at full size. With X = W S V^T the map keeps the
    singular vectors: NS(X) = W f(S) V^T, with f(s) in [0.68, 1.21] for a
    Gaussian matrix of this aspect (its smallest normalised singular value,
    ~0.005, is inside the quintic's band). So
      - the tall input and its transpose give transposed outputs, bit for bit;
      - X^T NS(X) = V S f(S) V^T is symmetric (to the bf16 error);
      - the mean of f(S)^2, ||NS(X)||_F^2 / 8192, lies in the band;
      - the largest and smallest singular values of NS(X), estimated by 60
        power iterations on NS(X)^T NS(X) (estimates that lie inside the true
        range), lie in the band widened to [0.64, 1.25] (the CPU emulation of
        the bf16 chain moves them by about 0.001).
    Also the workload's own step on layer 0's up and down matrices: status 0,
    their momentum within 1e-5 of the oracle's."""
    flush("wide tall bucket")
    g = torch.Generator(device=DEV).manual_seed(77)
    X = (torch.randn(28672, 8192, generator=g, device=DEV) * 1e-4).to(torch.bfloat16)
    U = ns_with_status(X, ma.muon_hparams(ns_dtype="bf16"))
    Ut = ns_with_status(X.t().contiguous(), ma.muon_hparams(ns_dtype="bf16"))
    assert torch.equal(U.t().contiguous().view(torch.int16), Ut.view(torch.int16))
    del Ut
    Xf, Uf = X.float(), U.float()
    M = Xf.t().contiguous() @ Uf                      # 8192 x 8192
    asym = (torch.linalg.norm(M - M.t()) / torch.linalg.norm(M)).item()
    assert asym < 2e-2, asym
    assert (torch.diagonal(M) > 0).all()
    del M, Xf
    msq = (torch.linalg.norm(Uf) ** 2 / 8192).item()
    assert 0.68 ** 2 < msq < 1.21 ** 2, msq
    G = Uf.t().contiguous() @ Uf                      # f(S)^2 in the basis V
    v = torch.randn(8192, 1, generator=g, device=DEV)
    for _ in range(60):
        v = G @ v
        v = v / torch.linalg.norm(v)
    lmax = (v.t() @ G @ v).item()
    c = 1.6
    H = c * torch.eye(8192, device=DEV) - G
    v = torch.randn(8192, 1, generator=g, device=DEV)
    for _ in range(60):
        v = H @ v
        v = v / torch.linalg.norm(v)
    lmin = c - (v.t() @ H @ v).item()
    assert 0.64 ** 2 < lmin <= lmax < 1.25 ** 2, (lmin, lmax)
    del G, H, Uf, U, X
    torch.cuda.empty_cache()

    wl = workloads.workload(5)
    data = to_gpu(workloads.generate(wl, device=DEV, only=(4, 5)))
    params = muon_params(data)
    hp = hp_c(wl.muon_hp)
    before = {i: (data.muon[i].momentum.clone(), data.muon[i].grad) for i in (4, 5)}
    ws = ma.muon_step(params, hp)
    assert ma.muon_step_status(ws) == 0
    h = hp_dict(wl.muon_hp)
    for i in (4, 5):
        t = data.muon[i]
        for rows in (slice(0, 1024), slice(t.spec.rows - 1024, t.spec.rows)):
            B1 = omuon.momentum_ema(host(before[i][0][0, rows]), host(before[i][1][0, rows]), h["beta"])
            check_local(host(t.momentum[0, rows]), B1, 1e-5, (i, "momentum"))


# ---------------------------------------------------------------------------
# At the planner's limits
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(65536, 129), (129, 65536)], ids=["tall", "wide"])
def test_newton_schulz_at_the_largest_dimension(shape, dt):
    """The largest dimension the planner accepts (65536) beside a ragged one:
    canonical 129 x 65536, padded to 256 x 65536, a contraction of 65536 in
    the Gram and one row of 256 APPLY tiles; against the oracle under the
    localized bars. bf16: 2e-2. fp32: 1e-4, not 1e-5: each thread of the fp32
    Gram adds its 65536 products one fp32 FMA after another, and such a sum
    carries a relative error of about u sqrt(K) / sqrt(3) ~ 9e-6 (u = 2^-24);
    emulated exactly that way, the whole chain lands at 1.8e-5 (rows 4.1e-5)
    of the fp64 oracle."""
    flush(f"ns largest dimension {shape} {dt}")
    x = randn(shape, 900 + shape[0] % 7)
    if dt == "bf16":
        x = x.to(torch.bfloat16)
    out = ns_with_status(x.to(DEV), ma.muon_hparams(ns_dtype=dt))
    want = omuon.newton_schulz(x.double().numpy())
    check_local(out.cpu().double().numpy(), want, 1e-4 if dt == "f32" else 2e-2, (shape, dt))


def test_step_with_more_matrices_than_the_persistent_queues_take():
    """70000 batched 64 x 64 matrices, more than the 65536 the persistent
    launch's queues are built for: the step takes the per-launch schedule
    over 70000-tile launches; status 0; momentum, the
    Newton-Schulz output and the updated parameters of 66 matrices spread
    over the batch (every 1111th, the second and the last) against the
    oracle."""
    # square: the emulated bf16 chain stays under 0.015 of the oracle at
    # 64 x 64 (tall 16 x 4 matrices reach 0.06, too few elements to average)
    spec = workloads.MuonTensorSpec("many", 70000, 64, 64, grad_std=1.0)
    wl = workloads.Workload("many_64x64", 51, (spec,), (), workloads.MuonHParams(ns_dtype="bf16"))
    sample = set(range(0, 70000, 1111)) | {1, 69999}
    run_step_checked(wl, 2e-2, sample=sample)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_wide_4L_d8192_up_projection_whole_chain():
    """Layer 0's MLP up projection of the wide-model workload (28672 x 8192,
    bf16, tall: the bucket that carries most of the step's Newton-Schulz
    work), in the workload's full step, against the oracle's whole chain on
    its stored inputs under the localized bars: momentum at 1e-5, the
    Newton-Schulz output, then Muon+ row_col, the shape scale sqrt(3.5) and
    the cautious wrapper on the stored bf16 parameters. The oracle's fp64
    Newton-Schulz of this matrix is about 44 TFLOP of host arithmetic (one to
    two minutes on 8 to 16 cores)."""
    run_step_checked(workloads.workload(5), 2e-2, sample=lambda kk, info: info["tensor"] == 4)
