"""HIP path vs the fp64 oracle on the same seeded inputs (needs an MI355X).

Tolerances: fp32 paths 1e-5 relative (Frobenius, per tensor) on updated
parameters and momentum; bf16 matrix-core Newton-Schulz 2e-2 relative
Frobenius per matrix against the fp64 oracle, and twice that on what follows
from it (NorMuon second moment, the fp32 parameter update; three times for the
update of bf16 parameters, rounded like the oracle's, with every element
within one bf16 spacing plus the update's element bar); cautious masks may
take the other branch only where the oracle's margin is inside 6 times the
Newton-Schulz tolerance of the RMS update, on at most 3% (bf16) or 0.1%
(fp32) of the elements; AdamW 1e-6 relative on p, m, v. Every expected value
comes from the oracle run on the stored inputs.
"""
import math
import os

import numpy as np
import pytest
import torch

import muon_adamw_amd as ma
import workloads
from oracle import adamw as oadamw
from oracle import muon as omuon
from oracle import storage
from tests.gpu_helpers import (adamw_params, check_update, flush, host, hp_c, hp_dict, muon_params, rel, snapshot,
                               to_gpu)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def randn(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32) * scale


# ---------------------------------------------------------------------------
# Newton-Schulz alone
# ---------------------------------------------------------------------------
F32_SHAPES = [(1, 1), (4, 3), (3, 4), (5, 5), (37, 100), (100, 37), (128, 256), (256, 128), (130, 129),
              (64, 300), (200, 200)]


@pytest.mark.parametrize("shape", F32_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_newton_schulz_f32(shape):
    flush(f"ns f32 {shape}")
    x = randn(shape, 100 + shape[0] * 7 + shape[1])
    out = ma.newton_schulz(x.to(DEV), ma.muon_hparams(ns_dtype="f32"))
    torch.cuda.synchronize()
    want = omuon.newton_schulz(x.double().numpy())
    err = rel(out.cpu().double().numpy(), want)
    # fp32 rounding is amplified by up to phi'(0)^5 = 3.4445^5 ~ 490 on the
    # smallest singular directions of near-square Gaussian inputs
    tol = 1e-5 if max(shape) >= 2 * min(shape) else 2e-4
    assert err < tol, err


def test_newton_schulz_f32_well_conditioned():
    """256x128 with singular values in [0.1, 1] (condition 10): fp32 to 1e-5."""
    g = torch.Generator().manual_seed(7)
    U, _ = torch.linalg.qr(torch.randn(256, 128, generator=g, dtype=torch.float64))
    V, _ = torch.linalg.qr(torch.randn(128, 128, generator=g, dtype=torch.float64))
    S = torch.logspace(0, -1, 128, dtype=torch.float64)
    x = ((U * S) @ V.T).float()
    out = ma.newton_schulz(x.to(DEV), ma.muon_hparams(ns_dtype="f32"))
    err = rel(out.cpu().double().numpy(), omuon.newton_schulz(x.double().numpy()))
    assert err < 1e-5, err


BF16_SHAPES = [(1, 1), (7, 3), (128, 128), (256, 128), (300, 200), (200, 300), (129, 1000), (768, 768),
               (768, 3072), (3072, 768), (1408, 2048)]


@pytest.mark.parametrize("shape", BF16_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_newton_schulz_bf16(shape):
    flush(f"ns bf16 {shape}")
    x = randn(shape, 200 + shape[0] + 3 * shape[1]).to(torch.bfloat16)
    out = ma.newton_schulz(x.to(DEV), ma.muon_hparams(ns_dtype="bf16"))
    torch.cuda.synchronize()
    want = omuon.newton_schulz(host(x))
    err = rel(host(out), want)
    assert err < 2e-2, err


def test_newton_schulz_batched_bf16():
    x = randn((3, 300, 200), 5).to(torch.bfloat16)
    out = ma.newton_schulz(x.to(DEV), ma.muon_hparams(ns_dtype="bf16"))
    xs, os_ = host(x), host(out)
    for b in range(3):
        assert rel(os_[b], omuon.newton_schulz(xs[b])) < 2e-2


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_newton_schulz_transpose_bitwise(dt):
    """NS(X^T) = NS(X)^T holds bit for bit: a tall input is the same canonical
    matrix as its wide transpose."""
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    x = randn((200, 520), 11).to(tdt)
    hp = ma.muon_hparams(ns_dtype=dt)
    a = ma.newton_schulz(x.to(DEV), hp)
    b = ma.newton_schulz(x.t().contiguous().to(DEV), hp)
    assert torch.equal(a.t().contiguous(), b)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_newton_schulz_zero_stays_finite(dt):
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    z = torch.zeros((96, 200), dtype=tdt, device=DEV)
    out = ma.newton_schulz(z, ma.muon_hparams(ns_dtype=dt))
    assert torch.isfinite(out.float()).all() and (out == 0).all()


# ---------------------------------------------------------------------------
# Whole Muon step
# ---------------------------------------------------------------------------
def oracle_inputs(data):
    """Host copies of every Muon tensor's stored inputs, for the oracle."""
    out = []
    for t in data.muon:
        if t is None:
            continue
        out.append({"param": workloads.to_numpy(t.param), "param_dtype": t.spec.param_dtype,
                    "grad": None if t.grad is None else workloads.to_numpy(t.grad),
                    "grad_dtype": t.spec.grad_dtype, "momentum": workloads.to_numpy(t.momentum),
                    "row_v": None if t.row_v is None else workloads.to_numpy(t.row_v),
                    "views": t.spec.views, "lr": t.spec.lr, "wd": t.spec.wd, "shape": t.spec.shape})
    return out


def check_momentum(gpu_mom, want_f32, tol=1e-5):
    got = gpu_mom.cpu().double().numpy().ravel()
    assert rel(got, want_f32.astype(np.float64).ravel()) < tol


def test_single_256x128_f32_end_to_end():
    """One fp32 256x128 tall matrix, fp32 Newton-Schulz: parameters, momentum
    and the orthogonalised update all within 1e-5 of the fp64 oracle."""
    wl = workloads.workload(1)
    data = to_gpu(workloads.generate(wl, device="cpu"))
    inp = oracle_inputs(data)
    hp = hp_c(wl.muon_hp)
    ws = ma.muon_step(muon_params(data), hp)
    torch.cuda.synchronize()
    want = omuon.muon_step(inp, hp_dict(wl.muon_hp))[0]
    t = data.muon[0]
    assert rel(t.param.cpu().double().numpy(), want["W64"]) < 1e-5
    check_momentum(t.momentum, want["momentum"])
    info = ma.matrix_info(muon_params(data), hp, 0)
    assert info["transposed"] == 1 and abs(info["scale"] - math.sqrt(2)) < 1e-7
    U = ma.workspace_u(ws, info, "f32").cpu().double().numpy()[: info["r"], : info["c"]]
    assert rel(U.T, want["U64"][0]) < 1e-5
    # the update itself, not just the decayed parameters
    W0 = storage.decode(inp[0]["param"], "f32").reshape(want["W64"].shape)
    dW_gpu = t.param.cpu().double().numpy() - W0
    assert rel(dW_gpu, want["W64"] - W0) < 1e-5


def gpu_u_stored(ws, info, ns_dtype):
    U = ma.workspace_u(ws, info, ns_dtype).cpu().float().double().numpy()[: info["r"], : info["c"]]
    return U.T if info["transposed"] else U


def oracle_direction(U, V0, hp):
    """The oracle's post-Newton-Schulz direction (NorMuon / Muon+) from its own U."""
    if hp["normuon"]:
        U, _ = omuon.normuon(U, V0, hp["normuon_beta2"])
    if hp["muon_plus"]:
        U = omuon.muon_plus_row_col(U, hp["muon_plus_eps"])
    return U


def run_and_check_muon(k, matrix_filter=None, oracle_filter=None, tol_ns=2e-2):
    """Runs a workload's Muon step on the GPU in the launch configuration the
    bench times (every matrix of the step in one persistent Newton-Schulz
    launch) and checks, per selected matrix: momentum against the oracle
    (1e-5); and for the matrices `oracle_filter` picks (all by default), the
    oracle's whole chain from the stored inputs: the Newton-Schulz output
    (bf16: 2e-2), the NorMuon second moment and the updated parameters."""
    wl = workloads.workload(k) if isinstance(k, int) else k
    h = hp_dict(wl.muon_hp)
    data = to_gpu(workloads.generate(wl, device="cpu" if wl.gen_device == "cpu" else DEV))
    params = muon_params(data)
    hp = hp_c(wl.muon_hp)
    nmat, _ = ma.plan_counts(params, hp)
    infos = [ma.matrix_info(params, hp, kk) for kk in range(nmat)]
    sel = [kk for kk in range(nmat) if matrix_filter is None or matrix_filter(kk, infos[kk])]
    # device copies of the state the step overwrites (only tensors with a
    # selected matrix); host copies are taken one matrix at a time below
    tens = sorted({infos[kk]["tensor"] for kk in sel})
    before = {ti: (snapshot(data.muon[ti].param), snapshot(data.muon[ti].momentum),
                   snapshot(data.muon[ti].row_v)) for ti in tens}
    flush(f"workload {wl.name}: muon_step ({len(sel)} of {nmat} matrices checked)")
    ws = ma.muon_step(params, hp)
    assert ma.muon_step_status(ws) == 0
    torch.cuda.synchronize()
    for kk in sel:
        info = infos[kk]
        ti = info["tensor"]
        t = data.muon[ti]
        m, n = info["m"], info["n"]
        bi, v = info["batch_index"], info["view"]
        rs = slice(v * m, (v + 1) * m)
        pick = (lambda x: x[bi, rs]) if t.param.dim() == 3 else (lambda x: x[rs])
        W0, G, B0 = host(pick(before[ti][0])), host(pick(t.grad)), host(pick(before[ti][1]))
        V0 = None if t.row_v is None else host(before[ti][2][bi, rs])
        B1 = omuon.momentum_ema(B0, G, h["beta"])
        assert rel(host(pick(t.momentum)), B1) < 1e-5, (kk, "momentum")
        if oracle_filter is not None and not oracle_filter(kk, info):
            continue
        flush(f"  matrix {kk} ({m}x{n}): oracle chain")
        Q = omuon.nesterov_lerp(G, B1, h["beta"]) if h["nesterov"] else B1
        W_want, V_want, U_want = omuon.matrix_update(Q, W0, G, V0, h, t.spec.lr, t.spec.wd)
        e = rel(gpu_u_stored(ws, info, wl.muon_hp.ns_dtype), U_want)
        assert e < tol_ns, (kk, "newton-schulz", e)
        if V0 is not None:
            e = rel(host(t.row_v[bi, rs]), V_want)
            assert e < 2 * tol_ns, (kk, "normuon V", e)
        U_dir = oracle_direction(U_want, V0, h)
        # bf16 parameters: the update is a few ulps of W, so the Newton-Schulz
        # difference also moves elements across rounding boundaries (measured
        # on the oracle: 1.5% noise on U gives 3-3.6% on the rounded update)
        check_update(host(pick(t.param)), W0, W_want, G, U_dir, h, t.spec.lr, t.spec.wd,
                     omuon.shape_scale(m, n), t.spec.param_dtype,
                     (2 if t.spec.param_dtype == "f32" else 3) * tol_ns, tol_ns)
    return data, ws


def test_gpt_12L_d768_muon_full():
    """GPT 12L d768: all 72 matrices against the oracle."""
    run_and_check_muon(2)


def test_gpt_12L_d768_adamw():
    wl = workloads.workload(2)
    data = to_gpu(workloads.generate(wl, device="cpu"))
    before = [(workloads.to_numpy(t.param), workloads.to_numpy(t.grad), workloads.to_numpy(t.m),
               workloads.to_numpy(t.v)) for t in data.adamw]
    h = wl.adamw_hp
    flush("gpt_12L_d768 adamw_step")
    ma.adamw_step(adamw_params(data), h.beta1, h.beta2, h.eps, h.step)
    torch.cuda.synchronize()
    tens = [{"param": p, "param_dtype": t.spec.param_dtype, "grad": g, "grad_dtype": t.spec.grad_dtype,
             "m": m, "v": v, "lr": t.spec.lr, "wd": t.spec.wd}
            for (p, g, m, v), t in zip(before, data.adamw)]
    want = oadamw.adamw_step(tens, {"beta1": h.beta1, "beta2": h.beta2, "eps": h.eps, "step": h.step})
    for t, w in zip(data.adamw, want):
        assert rel(host(t.param), w["p64"]) < 1e-6
        assert rel(host(t.m), w["m64"]) < 1e-6
        assert rel(host(t.v), w["v64"]) < 1e-6


def test_adamw_two_steps_bf16_params_and_tail():
    """bf16 params/grads, a ragged length, two steps; each side continues from
    its own stored state after step 1."""
    n = 100003
    p = randn((n,), 1, 0.02).to(torch.bfloat16)
    g1 = randn((n,), 2, 1e-3).to(torch.bfloat16)
    g2 = randn((n,), 3, 1e-3).to(torch.bfloat16)
    P = ma.AdamWParam(p.to(DEV), g1.to(DEV), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV),
                      1e-3, 0.05)
    ma.adamw_step([P], 0.9, 0.999, 1e-8, 1)
    torch.cuda.synchronize()
    p1, m1, v1 = oadamw.adamw_update(host(p), host(g1), np.zeros(n), np.zeros(n), 1e-3, 0.05, 0.9, 0.999,
                                     1e-8, 1)
    assert rel(host(P.m), m1) < 1e-6 and rel(host(P.v), v1) < 1e-6
    bits = workloads.to_numpy(P.param).astype(np.int32)
    assert np.abs(bits - storage.round_bf16_bits(p1).astype(np.int32)).max() <= 1
    p1o = storage.decode(storage.round_bf16_bits(p1), "bf16")
    m1o, v1o = storage.round_f32(m1).astype(np.float64), storage.round_f32(v1).astype(np.float64)
    P.grad = g2.to(DEV)
    ma.adamw_step([P], 0.9, 0.999, 1e-8, 2)
    torch.cuda.synchronize()
    p2, m2, v2 = oadamw.adamw_update(p1o, host(g2), m1o, v1o, 1e-3, 0.05, 0.9, 0.999, 1e-8, 2)
    assert rel(host(P.m), m2) < 1e-6 and rel(host(P.v), v2) < 1e-6
    bits = workloads.to_numpy(P.param).astype(np.int32)
    assert np.abs(bits - storage.round_bf16_bits(p2).astype(np.int32)).max() <= 1


def test_moe_64x2048_sampled():
    """MoE 64 experts: NorMuon + cautious weight-decay mask. Every matrix's
    momentum; the oracle's whole chain on a sample of gate, up and down
    matrices."""
    sample = {0, 1, 77, 128, 191}
    run_and_check_muon(4, oracle_filter=lambda kk, info: kk in sample)


def test_llama_8L_d4096_sampled():
    """Llama 8L d4096 (bf16 parameters, 1% gradient outliers), the full step in
    the bench's launch configuration: momentum of layer 0's q, k and both
    gate_up views; the oracle's whole chain on q (4096x4096), k (1024x4096)
    and the gate view (14336x4096, tall)."""
    run_and_check_muon(3, matrix_filter=lambda kk, info: info["tensor"] in (0, 1, 4),
                       oracle_filter=lambda kk, info: info["view"] == 0)


def test_wide_4L_d8192_sampled():
    """4L d8192 (bf16, Muon+ row_col and the cautious wrapper), the full step
    in the bench's launch configuration: momentum of layer 0's q and k, the
    oracle's whole chain on k (8192x8192; an 8192x28672 matrix takes the fp64
    oracle minutes)."""
    run_and_check_muon(5, matrix_filter=lambda kk, info: info["tensor"] in (0, 1),
                       oracle_filter=lambda kk, info: info["tensor"] == 1)


# ---------------------------------------------------------------------------
# Edge cases of the step
# ---------------------------------------------------------------------------
def small_workload(param_dtype="f32", grad_dtype="f32", ns_dtype="bf16", cautious="none", normuon=False,
                   muon_plus=False):
    specs = (workloads.MuonTensorSpec("a", 1, 300, 200, param_dtype=param_dtype, grad_dtype=grad_dtype),
             workloads.MuonTensorSpec("b", 2, 2 * 96, 160, views=2, param_dtype=param_dtype,
                                      grad_dtype=grad_dtype),
             workloads.MuonTensorSpec("c", 1, 64, 500, param_dtype=param_dtype, grad_dtype=grad_dtype),
             workloads.MuonTensorSpec("d", 1, 37, 23, param_dtype=param_dtype, grad_dtype=grad_dtype))
    hp = workloads.MuonHParams(ns_dtype=ns_dtype, cautious=cautious, normuon=normuon, muon_plus=muon_plus)
    return workloads.Workload("small", 9, specs, (), hp)


@pytest.mark.parametrize("variant", [
    dict(),
    dict(ns_dtype="f32"),
    dict(param_dtype="bf16", grad_dtype="bf16"),
    dict(cautious="wd_mask", normuon=True),
    dict(cautious="wrapper", muon_plus=True),
    dict(cautious="wrapper", muon_plus=True, param_dtype="bf16", grad_dtype="bf16"),
    dict(cautious="wd_mask", normuon=True, ns_dtype="f32"),
], ids=lambda d: "-".join(f"{k}={v}" for k, v in d.items()) or "default")
def test_small_mixed_shapes(variant):
    """Ragged tall/wide matrices, a batch and views in one call; every matrix
    against the oracle (fp32 Newton-Schulz: 1e-4 for these Gaussian, partly
    near-square inputs; bf16: 2e-2)."""
    wl = small_workload(**variant)
    run_and_check_muon(wl, tol_ns=1e-4 if wl.muon_hp.ns_dtype == "f32" else 2e-2)


def test_small_f32_end_to_end():
    """fp32 Newton-Schulz: the whole step (not staged) within 1e-5 of the
    oracle on tall, wide and packed matrices with aspect ratio >= 1.5."""
    specs = (workloads.MuonTensorSpec("a", 1, 384, 128),
             workloads.MuonTensorSpec("b", 2, 2 * 64, 160, views=2),
             workloads.MuonTensorSpec("c", 1, 64, 500))
    wl = workloads.Workload("small_f32", 21, specs, (), workloads.MuonHParams(ns_dtype="f32"))
    data = to_gpu(workloads.generate(wl, device="cpu"))
    inp = oracle_inputs(data)
    ma.muon_step(muon_params(data), hp_c(wl.muon_hp))
    torch.cuda.synchronize()
    want = omuon.muon_step(inp, hp_dict(wl.muon_hp))
    for t, w, i in zip(data.muon, want, inp):
        W0 = storage.decode(i["param"], "f32").reshape(w["W64"].shape)
        assert rel(host(t.param), w["W64"]) < 1e-5
        assert rel(host(t.param) - W0, w["W64"] - W0) < 1e-5
        check_momentum(t.momentum, w["momentum"])


def test_absent_gradient_and_zero_gradient():
    wl = small_workload()
    data = to_gpu(workloads.generate(wl, device="cpu"))
    data.muon[1].grad = None                         # inactive expert
    data.muon[2].grad = torch.zeros_like(data.muon[2].grad)
    keep_p, keep_m = data.muon[1].param.clone(), data.muon[1].momentum.clone()
    p2 = data.muon[2].param.clone()
    ma.muon_step(muon_params(data), hp_c(wl.muon_hp))
    torch.cuda.synchronize()
    assert torch.equal(data.muon[1].param, keep_p) and torch.equal(data.muon[1].momentum, keep_m)
    decay = torch.tensor(1.0 - 0.02 * 0.1, dtype=torch.float64).float().item()
    assert torch.equal(data.muon[2].param, p2 * decay)
    assert (data.muon[2].momentum == 0).all()
    assert not torch.equal(data.muon[0].param, data.muon[0].param * 0)


def test_views_match_separate_tensors_bitwise():
    """A (2, m, n) packed parameter steps exactly like its two halves passed
    as separate tensors."""
    g = torch.Generator().manual_seed(3)
    P = (torch.randn(1, 2 * 96, 160, generator=g) * 0.02).to(DEV)
    G = torch.randn(1, 2 * 96, 160, generator=g).to(DEV)
    M = torch.zeros_like(P)
    P2, M2 = P.clone(), M.clone()
    hp = ma.muon_hparams()
    ma.muon_step([ma.MuonParam(P, G, M, views=2)], hp)
    halves = [ma.MuonParam(P2[:, :96].contiguous(), G[:, :96].contiguous(), M2[:, :96].contiguous()),
              ma.MuonParam(P2[:, 96:].contiguous(), G[:, 96:].contiguous(), M2[:, 96:].contiguous())]
    ma.muon_step(halves, hp)
    torch.cuda.synchronize()
    assert torch.equal(P[:, :96], halves[0].param) and torch.equal(P[:, 96:], halves[1].param)
    assert torch.equal(M[:, :96], halves[0].momentum)


def test_two_steps_continue_from_state():
    """Step, then step again: the GPU's second step equals the oracle's second
    step, each side continuing from its own stored state; and saving/restoring
    the GPU state in between changes nothing (bitwise)."""
    wl = small_workload(ns_dtype="f32")
    h = hp_dict(wl.muon_hp)
    data = to_gpu(workloads.generate(wl, device="cpu"))
    inp1 = oracle_inputs(data)
    hp = hp_c(wl.muon_hp)
    ma.muon_step(muon_params(data), hp)
    torch.cuda.synchronize()
    want1 = omuon.muon_step(inp1, h)
    saved = [(t.param.cpu().clone(), t.momentum.cpu().clone()) for t in data.muon]
    for t in data.muon:
        t.grad = torch.randn(t.grad.shape, generator=torch.Generator().manual_seed(99)).to(DEV)
    inp2 = [dict(i, param=w["param"], momentum=w["momentum"], grad=workloads.to_numpy(t.grad.cpu()))
            for i, w, t in zip(inp1, want1, data.muon)]
    # a copy restored from host state
    clone = [ma.MuonParam(p.to(DEV), t.grad, m.to(DEV), None, t.spec.views, t.spec.lr, t.spec.wd)
             for (p, m), t in zip(saved, data.muon)]
    ma.muon_step(muon_params(data), hp)
    ma.muon_step(clone, hp)
    torch.cuda.synchronize()
    want = omuon.muon_step(inp2, h)
    for t, c, w in zip(data.muon, clone, want):
        assert torch.equal(t.param, c.param) and torch.equal(t.momentum, c.momentum)
        check_momentum(t.momentum, w["momentum"])
        assert rel(host(t.param), w["W64"]) < 1e-5


def test_operand_layouts_same_bits():
    """SQUARE and APPLY read their symmetric operand row-wise or k-major
    (chosen by size); both readings see the same values, so the results are
    the same bits, tall and ragged matrices included."""
    flush("operand layouts")
    xs = [randn((4, 768, 768), 81).to(torch.bfloat16), randn((3072, 768), 82).to(torch.bfloat16),
          randn((300, 200), 83).to(torch.bfloat16), randn((2304, 2560), 84).to(torch.bfloat16)]
    hp = ma.muon_hparams(ns_dtype="bf16")
    outs = {}
    for mode in ("rows", "kmajor"):
        os.environ["MA_NS_OPERANDS"] = mode
        try:
            outs[mode] = [ma.newton_schulz(x.to(DEV), hp).cpu() for x in xs]
        finally:
            del os.environ["MA_NS_OPERANDS"]
    for i in range(len(xs)):
        assert torch.equal(outs["rows"][i].view(torch.int16), outs["kmajor"][i].view(torch.int16)), i
    assert rel(host(outs["rows"][3]), omuon.newton_schulz(host(xs[3]))) < 2e-2


def test_symmetric_products_stored_symmetric():
    """A = X X^T and B = bA + cA^2 hold equal values in both triangles, bit
    for bit (one triangle is computed and stored twice), so SQUARE and APPLY
    may read them along either index. Config 2 after a full step: the last
    iteration's A and B of a 768x768 and both 768x3072 shapes."""
    wl = workloads.workload(2)
    data = to_gpu(workloads.generate(wl, device="cpu"))
    params = muon_params(data)
    hp = hp_c(wl.muon_hp)
    ws = ma.muon_step(params, hp)
    torch.cuda.synchronize()
    for kk in (0, 4, 5):
        info = ma.matrix_info(params, hp, kk)
        rp = info["rp"]
        for nm in ("a_offset", "b_offset"):
            o = info[nm]
            M = ws[o:o + rp * rp * 2].view(torch.int16).view(rp, rp)
            assert torch.equal(M, M.t()), (kk, nm, int((M != M.t()).sum()))
            assert (M != 0).any()


@pytest.mark.gpu
def test_persistent_schedule_matches_launches():
    """The one-launch Newton-Schulz schedule (per-XCD task queues with
    completion counters) gives the same bits as three launches per iteration,
    run after run: every tile reads only data its producers finished."""
    flush("persistent vs launches")
    xs = [randn((4, 768, 768), 91).to(torch.bfloat16), randn((768, 3072), 92).to(torch.bfloat16),
          randn((300, 200), 93).to(torch.bfloat16)]
    hp = ma.muon_hparams(ns_dtype="bf16")
    outs = {}
    for sched in ("launches", "persistent"):
        os.environ["MA_NS_SCHEDULE"] = sched
        try:
            outs[sched] = [[ma.newton_schulz(x.to(DEV), hp).cpu() for _ in range(2)] for x in xs]
        finally:
            del os.environ["MA_NS_SCHEDULE"]
    torch.cuda.synchronize()
    for i in range(len(xs)):
        ref = outs["launches"][i][0].view(torch.int16)
        for sched in ("launches", "persistent"):
            for o in outs[sched][i]:
                assert torch.equal(o.view(torch.int16), ref), (i, sched)
