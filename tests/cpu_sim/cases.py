"""Parity cases of the kernels' source run on the CPU simulator, against the oracle.

Each case calls the library's C entry points (the simulator build) on seeded
inputs in guarded buffers and compares every output with the fp64 oracle, at
the bars the GPU parity tests use. One case per child process:

    python -m tests.cpu_sim.cases <case> [--mode tail|head] [--workers N] [--immediate-dma] [--lib PATH]
        [--schedule together|waves-up|waves-down] [--no-poison]

Workspaces and outputs start as 0xFF bytes (NaN in both float formats): the
header promises that a workspace's contents on entry do not matter, and
fresh zeroed memory would hide a read of padding the library never wrote.

Exit status 0: passed. 1: a mismatch or a simulator fault (message on
stderr). Killed by SIGSEGV: an access outside a buffer hit a guard page.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys
import traceback

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import muon_adamw_amd as ma  # noqa: E402
import workloads  # noqa: E402
from oracle import adamw as oadamw  # noqa: E402
from oracle import gradnorm as ognorm  # noqa: E402
from oracle import muon as omuon  # noqa: E402
from oracle import storage  # noqa: E402
from tests import cpu_sim  # noqa: E402
from tests.gpu_helpers import check_local, check_update, hp_c, hp_dict  # noqa: E402

DT = {"f32": ma.MA_F32, "bf16": ma.MA_BF16}


class Sim:
    def __init__(self, mode="tail", workers=8, deferred=True, lib=None, schedule=0, poison=False):
        self.lib = cpu_sim.load(lib or cpu_sim.LIB)
        self.lib.hipsim_set_schedule(schedule)
        self.lib.hipsim_set_workers(workers)
        self.lib.hipsim_set_dma_deferred(1 if deferred else 0)
        self.arena = cpu_sim.Arena(mode, poison)

    def ok(self, status, what=""):
        fault = self.lib.hipsim_fault().decode()
        assert not fault, f"{what}: simulator fault: {fault}"
        assert status == 0, f"{what}: status {status}: {self.lib.ma_last_error().decode()}"

    def put(self, a):
        return self.arena.like(np.ascontiguousarray(a))


def dec(a, dt):
    return storage.decode(a, dt)


def randn(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# global norm and clip state
# ---------------------------------------------------------------------------
def grad_norm(sim, grads, max_norm):
    """grads: list of (stored array, dtype) or None. Returns the state."""
    lib = sim.lib
    arr = (ma.GradRefC * max(len(grads), 1))()
    bufs = []
    for i, g in enumerate(grads):
        if g is None:
            continue
        b = sim.put(g[0])
        bufs.append(b)
        arr[i].grad, arr[i].numel, arr[i].dtype = cpu_sim.addr(b), b.size, DT[g[1]]
    need = lib.ma_grad_norm_workspace_bytes(arr, len(grads))
    assert need > 0, lib.ma_last_error()
    ws = sim.arena.bytes(need)
    st = sim.arena.array((4,), np.float32)
    sim.ok(lib.ma_global_grad_norm(arr, len(grads), float(max_norm), cpu_sim.addr(st), cpu_sim.addr(ws), need,
                                   None), "global norm")
    return st


def case_grad_norm(sim):
    rng = np.random.default_rng(5)
    f32 = lambda a: storage.round_f32(a)
    bf = lambda a: storage.round_bf16_bits(a)
    grads = [(f32(rng.standard_normal(70001) * 1e-3), "f32"), None,
             (bf(rng.standard_normal((33, 129)) * 2e-3), "bf16"), (f32(rng.standard_normal(5)), "f32")]
    st = grad_norm(sim, grads, 0.05)
    want = ognorm.global_norm(grads)
    f, skip = ognorm.clip_state(want, 0.05)
    assert abs(st[0] - want) <= 1e-6 * want, (st[0], want)
    assert abs(st[1] - f) <= 1e-6 * f and st[2] == float(skip) == 0.0, (st, f, skip)
    # |g| ~ 1e20: fp32 squares overflow, the fp64 partials do not: a clip, not a skip
    huge = [(f32(rng.standard_normal(4099) * 1e20), "f32"), (bf(rng.standard_normal(300) * 3e20), "bf16")]
    st = grad_norm(sim, huge, 1.0)
    want = ognorm.global_norm(huge)
    f, skip = ognorm.clip_state(want, 1.0)
    assert not skip and np.isfinite(st[0]) and abs(st[0] - want) <= 1e-6 * want, (st, want)
    assert abs(st[1] - f) <= 1e-6 * f and st[2] == 0.0, (st, f)
    # a non-finite gradient: the step is skipped
    bad = f32(rng.standard_normal(1000))
    bad[777] = np.nan
    st = grad_norm(sim, [(bad, "f32")], 1.0)
    assert st[2] != 0.0, st
    # no clipping asked: factor 1
    st = grad_norm(sim, grads, 0.0)
    assert st[1] == 1.0 and st[2] == 0.0, st


# ---------------------------------------------------------------------------
# AdamW
# ---------------------------------------------------------------------------
def rel(x, y):
    d, n = np.linalg.norm(np.asarray(x) - y), np.linalg.norm(y)
    return d / n if n > 0 else d


def case_adamw(sim):
    """fp32 and bf16 parameters, fp32 and bf16 moments (stochastic rounding),
    ragged lengths, with and without the cautious wrapper and a clip: p, m, v
    within 1e-6 of the oracle (bf16 parameters within one bf16 unit of its
    rounded value; masked entries bit for bit); bf16 moment bits the
    oracle's except at most 0.2% one neighbour off."""
    lib = sim.lib
    rng = np.random.default_rng(11)
    specs = [("f32", "f32", "f32", 70001), ("bf16", "bf16", "f32", 4097), ("bf16", "bf16", "bf16", 12289),
             ("f32", "bf16", "bf16", 2048 * 3 + 5), ("f32", "f32", "f32", 1)]
    for cautious in (False, True):
        for clip in (False, True):
            ts = []
            for i, (pd, gd, md, n) in enumerate(specs):
                ts.append({"param": storage.round_to(rng.standard_normal(n) * 0.02, pd), "param_dtype": pd,
                           "grad": storage.round_to(rng.standard_normal(n) * 1e-3, gd), "grad_dtype": gd,
                           "m": storage.round_to(rng.standard_normal(n) * 1e-4, md),
                           "v": storage.round_to(np.abs(rng.standard_normal(n)) * 1e-7, md),
                           "moment_dtype": md, "lr": 3e-4 * (i + 1), "wd": 5.0 if cautious else 0.1 * (i % 2)})
            state, cl = None, None
            if clip:
                state = grad_norm(sim, [(t["grad"], t["grad_dtype"]) for t in ts], 0.01)
                cl = ognorm.clip_state(ognorm.global_norm([(t["grad"], t["grad_dtype"]) for t in ts]), 0.01)
                assert cl[0] < 1.0 and abs(state[1] - cl[0]) <= 1e-6 * cl[0], (state, cl)
            arr = (ma.AdamWTensorC * len(ts))()
            bufs = []
            for i, t in enumerate(ts):
                P, G, M, V = (sim.put(t[k]) for k in ("param", "grad", "m", "v"))
                bufs.append((P, G, M, V))
                d = arr[i]
                d.param, d.grad, d.m, d.v = (cpu_sim.addr(x) for x in (P, G, M, V))
                d.numel = P.size
                d.param_dtype, d.grad_dtype, d.moment_dtype = (DT[t[k]] for k in ("param_dtype", "grad_dtype",
                                                                                   "moment_dtype"))
                d.lr, d.weight_decay = t["lr"], t["wd"]
            step, seed = 7, 1234
            hp = ma.AdamWHParamsC(0.9, 0.95, 1e-8, step)
            hp.cautious = ma.CAUTIOUS["wrapper"] if cautious else 0
            hp.seed = seed
            hp.clip = None if state is None else cpu_sim.addr(state)
            sim.ok(lib.adamw_step(arr, len(ts), ctypes.byref(hp), None), "adamw")
            want = oadamw.adamw_step(ts, {"beta1": 0.9, "beta2": 0.95, "eps": 1e-8, "step": step, "seed": seed,
                                          "cautious": cautious}, clip=None if cl is None else (float(state[1]), False))
            for i, (t, (P, G, M, V), w) in enumerate(zip(ts, bufs, want)):
                what = (i, t["param_dtype"], t["moment_dtype"], cautious, clip)
                p0 = dec(t["param"], t["param_dtype"])
                upd = p0 - w["p64"]
                near = np.abs(upd) < 1e-6 * np.sqrt(np.mean(upd * upd)) if cautious else np.zeros(upd.shape, bool)
                if cautious:
                    g = dec(t["grad"], t["grad_dtype"])
                    masked = ~((upd * g) > 0)
                    assert np.all((dec(P, t["param_dtype"]) == p0)[masked & ~near]), what
                if t["param_dtype"] == "f32":
                    assert rel(dec(P, "f32")[~near], w["p64"][~near]) < 1e-6, what
                else:
                    assert np.abs(P.astype(np.int64) - w["param"].astype(np.int64))[~near].max(initial=0) <= 1, what
                if t["moment_dtype"] == "f32":
                    assert rel(dec(M, "f32"), w["m64"]) < 1e-6 and rel(dec(V, "f32"), w["v64"]) < 1e-6, what
                else:
                    # one bf16 spacing of the new moment, plus the fp32 evaluation error of
                    # its two terms (m can cancel to near zero)
                    g = dec(t["grad"], t["grad_dtype"]) * (1.0 if cl is None else float(state[1]))
                    terms = (0.9 * np.abs(dec(t["m"], "bf16")) + 0.1 * np.abs(g),
                             0.95 * np.abs(dec(t["v"], "bf16")) + 0.05 * g * g)
                    for got, wb, w64, term in ((M, w["m"], w["m64"], terms[0]), (V, w["v"], w["v64"], terms[1])):
                        gv = dec(got, "bf16")
                        assert np.all(np.abs(gv - w64) <= np.abs(w64) * 2.0 ** -7 + term * 2.0 ** -20), what
                        assert np.mean(got != wb) < 2e-3, (what, float(np.mean(got != wb)))


# ---------------------------------------------------------------------------
# Newton-Schulz alone
# ---------------------------------------------------------------------------
def newton_schulz(sim, x_stored, dt, hp=None, want_status=0):
    lib = sim.lib
    shape = x_stored.shape
    batch, rows, cols = (1, *shape) if len(shape) == 2 else shape
    hp = hp or ma.muon_hparams(ns_dtype=dt)
    X = sim.put(x_stored)
    out = sim.arena.array(shape, x_stored.dtype)
    need = lib.ma_newton_schulz_workspace_bytes(batch, rows, cols, DT[dt], ctypes.byref(hp))
    assert need > 0, lib.ma_last_error()
    ws = sim.arena.bytes(need)
    sim.ok(lib.ma_newton_schulz(cpu_sim.addr(X), cpu_sim.addr(out), batch, rows, cols, DT[dt], ctypes.byref(hp),
                                cpu_sim.addr(ws), need, None), f"newton-schulz {shape} {dt}")
    st = ctypes.c_int32(-1)
    sim.ok(lib.ma_muon_step_status(cpu_sim.addr(ws), ctypes.byref(st), None), "status")
    assert st.value == want_status, ("status word", st.value, want_status)
    return out


def case_ns_f32(sim):
    for k, shape in enumerate([(1, 1), (4, 3), (37, 100), (100, 37), (128, 256), (256, 128), (64, 300)]):
        x = storage.round_f32(randn(shape, 400 + k))
        out = newton_schulz(sim, x, "f32")
        check_local(dec(out, "f32"), omuon.newton_schulz(dec(x, "f32")), 1e-5, shape)


def case_ns_bf16(sim):
    for k, shape in enumerate([(1, 1), (7, 3), (128, 128), (300, 200), (200, 300), (129, 600)]):
        x = storage.round_bf16_bits(randn(shape, 300 + k))
        out = newton_schulz(sim, x, "bf16")
        check_local(dec(out, "bf16"), omuon.newton_schulz(dec(x, "bf16")), 2e-2, shape)


def case_ns_schedules(sim):
    """The persistent launch and the per-launch schedule give the same bits."""
    for k, shape in enumerate([(300, 700), (640, 256), (3, 5, 130)]):
        x = storage.round_bf16_bits(randn(shape, 500 + k))
        a = newton_schulz(sim, x, "bf16").copy()
        os.environ["MA_NS_SCHEDULE"] = "launches"
        try:
            b = newton_schulz(sim, x, "bf16").copy()
        finally:
            del os.environ["MA_NS_SCHEDULE"]
        assert np.array_equal(a, b), (shape, int(np.sum(a != b)))


def case_ns_layouts(sim):
    """SQUARE and APPLY read their operands k-major (at most 2048 padded rows)
    or row-wise (larger matrices): forced each way, the same bits, and the
    row-wise results within the oracle's bar."""
    for k, shape in enumerate([(300, 700), (640, 256), (2, 260, 130)]):
        x = storage.round_bf16_bits(randn(shape, 600 + k))
        outs = []
        for layout in ("rows", "kmajor"):
            os.environ["MA_NS_OPERANDS"] = layout
            try:
                outs.append(newton_schulz(sim, x, "bf16").copy())
            finally:
                del os.environ["MA_NS_OPERANDS"]
        assert np.array_equal(outs[0], outs[1]), (shape, int(np.sum(outs[0] != outs[1])))
        xs = x if x.ndim == 3 else x[None]
        got = outs[0] if x.ndim == 3 else outs[0][None]
        for b in range(xs.shape[0]):
            check_local(dec(got[b], "bf16"), omuon.newton_schulz(dec(xs[b], "bf16")), 2e-2, (shape, b))


def case_status_undrained(sim):
    """Workgroups reach only four of the eight XCD queues (a device where some
    XCD gets none): the persistent launch finishes and its status word says
    a queue was left (NS_QUEUE_UNDRAINED); with all eight, 0 and the
    oracle's result."""
    x = storage.round_bf16_bits(randn((16, 128, 256), 700))
    sim.lib.hipsim_set_xcds(4)
    try:
        newton_schulz(sim, x, "bf16", want_status=ma.NS_QUEUE_UNDRAINED)
    finally:
        sim.lib.hipsim_set_xcds(8)
    out = newton_schulz(sim, x, "bf16")
    for b in range(0, 16, 5):
        check_local(dec(out[b], "bf16"), omuon.newton_schulz(dec(x[b], "bf16")), 2e-2, b)


def case_mfma_ceiling(sim):
    """The matrix-core ceiling loop: each block's sink value is eight times
    the sum of lane 0's sixteen accumulators after `iters` products of the
    kernel's fixed operands (exact in fp32)."""
    blocks, iters = 3, 5
    sink = sim.arena.array((blocks,), np.float32)
    sim.ok(sim.lib.ma_mfma_bf16_ceiling(cpu_sim.addr(sink), blocks, iters, None), "ceiling")
    A = np.array([[0.125 * (((32 * (k // 8) + i) + k % 8) & 7) for k in range(16)] for i in range(32)])
    B = np.array([[0.0625 * (((32 * (k // 8) + c) + 3 * (k % 8)) & 15) for c in range(32)] for k in range(16)])
    rows = [8 * (r // 4) + r % 4 for r in range(16)]
    want = 8 * iters * (A @ B)[rows, 0].sum()
    assert np.all(sink == np.float32(want)), (sink, want)


# ---------------------------------------------------------------------------
# whole Muon steps
# ---------------------------------------------------------------------------
def load_muon(sim, tens):
    """Guarded copies of the tensors' buffers and their C descriptors."""
    arr = (ma.MuonTensorC * len(tens))()
    bufs = []
    for i, t in enumerate(tens):
        P = sim.put(workloads.to_numpy(t.param))
        G = None if t.grad is None else sim.put(workloads.to_numpy(t.grad))
        M = sim.put(workloads.to_numpy(t.momentum))
        V = None if t.row_v is None else sim.put(workloads.to_numpy(t.row_v))
        bufs.append((P, G, M, V))
        d = arr[i]
        d.param, d.momentum = cpu_sim.addr(P), cpu_sim.addr(M)
        d.grad = None if G is None else cpu_sim.addr(G)
        d.row_v = None if V is None else cpu_sim.addr(V)
        d.batch, d.rows, d.cols, d.views = t.spec.batch, t.spec.rows, t.spec.cols, t.spec.views
        d.param_dtype, d.grad_dtype = DT[t.spec.param_dtype], DT[t.spec.grad_dtype]
        d.lr, d.weight_decay = t.spec.lr, t.spec.wd
    return arr, bufs


def run_muon(sim, arr, n, hp, what="muon_step"):
    """One muon_step on the descriptors; returns (matrix infos, workspace)."""
    lib = sim.lib
    nm, nb = ctypes.c_int32(0), ctypes.c_int32(0)
    sim.ok(lib.ma_muon_plan_counts(arr, n, ctypes.byref(hp), ctypes.byref(nm), ctypes.byref(nb)), "plan")
    infos = []
    for k in range(nm.value):
        info = ma.MatrixInfoC()
        sim.ok(lib.ma_muon_matrix_info(arr, n, ctypes.byref(hp), k, ctypes.byref(info)), "info")
        infos.append({f: getattr(info, f) for f, _ in ma.MatrixInfoC._fields_ if f != "pad_"})
    need = lib.ma_muon_workspace_bytes(arr, n, ctypes.byref(hp))
    ws = sim.arena.bytes(need)
    sim.ok(lib.muon_step(arr, n, ctypes.byref(hp), cpu_sim.addr(ws), need, None), what)
    st = ctypes.c_int32(-1)
    sim.ok(lib.ma_muon_step_status(cpu_sim.addr(ws), ctypes.byref(st), None), "status")
    assert st.value == 0, ("status word", st.value)
    return infos, ws


def muon_step(sim, wl, tol_ns, update_tol=None, only=None, data=None, hp=None, clip=1.0, h_extra=None):
    """One step of workload `wl` (or of `data`); every matrix against the
    oracle's chain: momentum at 1e-5, the Newton-Schulz output (localized
    bars at tol_ns), NorMuon's V (twice tol_ns) and the stored parameters.
    `clip`: the factor the gradient is read with (hp.clip then points at
    the state); `h_extra`: oracle settings beyond the workload's (a
    coefficient table)."""
    h = dict(hp_dict(wl.muon_hp), **(h_extra or {}))
    data = data or workloads.generate(wl, device="cpu", gen_device="cpu", only=only)
    tens = [t for t in data.muon if t is not None]
    arr, bufs = load_muon(sim, tens)
    before = [(P.copy(), M.copy(), None if V is None else V.copy()) for P, _, M, V in bufs]
    infos, ws = run_muon(sim, arr, len(tens), hp or hp_c(wl.muon_hp), f"muon_step {wl.name}")
    es = 2 if wl.muon_hp.ns_dtype == "bf16" else 4
    for kk, info in enumerate(infos):
        ti = info["tensor"]
        spec = tens[ti].spec
        P, G, M, V = bufs[ti]
        m, n, bi, v = info["m"], info["n"], info["batch_index"], info["view"]
        rs = slice(v * m, (v + 1) * m)
        W0 = dec(before[ti][0][bi, rs], spec.param_dtype)
        Gm = dec(G[bi, rs], spec.grad_dtype) * clip
        B0 = dec(before[ti][1][bi, rs], "f32")
        V0 = None if V is None else dec(before[ti][2][bi, rs], "f32")
        B1 = omuon.momentum_ema(B0, Gm, h["beta"])
        check_local(dec(M[bi, rs], "f32"), B1, 1e-5, (kk, "momentum"))
        Q = omuon.nesterov_lerp(Gm, B1, h["beta"]) if h["nesterov"] else B1
        W_want, V_want, U_want = omuon.matrix_update(Q, W0, Gm, V0, h, spec.lr, spec.wd)
        raw = ws[info["u_offset"]: info["u_offset"] + info["rp"] * info["cp"] * es]
        U = dec(raw.view(np.uint16 if es == 2 else np.float32).reshape(info["rp"], info["cp"]),
                wl.muon_hp.ns_dtype)[: info["r"], : info["c"]]
        check_local(U.T if info["transposed"] else U, U_want, tol_ns, (kk, "newton-schulz"))
        if V0 is not None:
            check_local(dec(V[bi, rs], "f32"), V_want, 2 * tol_ns, (kk, "normuon V"))
        U_dir = U_want
        if h["normuon"]:
            U_dir, _ = omuon.normuon(U_dir, V0, h["normuon_beta2"])
        if h["muon_plus"]:
            U_dir = omuon.muon_plus_row_col(U_dir, h["muon_plus_eps"])
        tol_p = update_tol or (2 if spec.param_dtype == "f32" else 3) * tol_ns
        check_update(dec(P[bi, rs], spec.param_dtype), W0, W_want, Gm, U_dir, h, spec.lr, spec.wd,
                     omuon.shape_scale(m, n), spec.param_dtype, tol_p, tol_ns)
    return infos, ws, bufs


def aspect2_workload(name, seed, **hp):
    pd = hp.pop("param_dtype", "f32")
    specs = (workloads.MuonTensorSpec("a", 1, 384, 128, param_dtype=pd, grad_dtype=pd),
             workloads.MuonTensorSpec("b", 2, 2 * 64, 160, views=2, param_dtype=pd, grad_dtype=pd),
             workloads.MuonTensorSpec("c", 1, 64, 500, param_dtype=pd, grad_dtype=pd))
    return workloads.Workload(name, seed, specs, (), workloads.MuonHParams(**hp))


VARIANTS = [dict(), dict(muon_plus=True, cautious="wrapper"), dict(normuon=True, cautious="wd_mask"),
            dict(muon_plus=True, cautious="wrapper", param_dtype="bf16"),
            dict(normuon=True, cautious="wd_mask", param_dtype="bf16")]


def case_muon_f32(sim):
    for v in VARIANTS:
        muon_step(sim, aspect2_workload("epilogue_f32", 41, ns_dtype="f32", **dict(v)), 1e-5, update_tol=1e-5)


def case_muon_bf16(sim):
    for v in VARIANTS[:4]:
        muon_step(sim, aspect2_workload("epilogue_bf16", 42, ns_dtype="bf16", **dict(v)), 2e-2)


def case_gpt_layer0(sim):
    """Layer 0 of the GPT 12L d768 workload at its real shapes (q, k, v, o
    768 x 768, up 3072 x 768 tall, down 768 x 3072): multi-tile matrices,
    fp32 storage, bf16 Newton-Schulz."""
    muon_step(sim, workloads.workload(2), 2e-2, only=range(6))


def minis():
    """Each larger workload's structure and hyperparameters at a size the
    simulator runs in seconds."""
    S = workloads.MuonTensorSpec
    bf = dict(param_dtype="bf16", grad_dtype="bf16")
    # k keeps 512 rows: with 1% of the gradient x100, a bf16 chain over 128-256
    # rows already puts single columns near the column bar (the workload's k
    # has 1024 rows, where the bars were calibrated)
    llama = workloads.Workload("llama_mini", 12, (
        S("q", 1, 512, 512, **bf, outlier_frac=0.01, outlier_scale=100.0),
        S("k", 1, 512, 1536, **bf, outlier_frac=0.01, outlier_scale=100.0),
        S("gate_up", 1, 2 * 896, 512, views=2, **bf, outlier_frac=0.01, outlier_scale=100.0),
        S("down", 1, 512, 896, **bf, outlier_frac=0.01, outlier_scale=100.0)),
        (), workloads.MuonHParams(ns_dtype="bf16"))
    moe = workloads.Workload("moe_mini", 13, (
        S("experts.gate_up", 4, 2 * 352, 512, views=2), S("experts.down", 4, 512, 352)),
        (), workloads.MuonHParams(ns_dtype="bf16", normuon=True, normuon_beta2=0.95, cautious="wd_mask"))
    wide = workloads.Workload("wide_mini", 14, (
        S("q", 1, 512, 512, **bf, param_std=0.01, grad_std=1e-4),
        S("up", 1, 1792, 512, **bf, param_std=0.01, grad_std=1e-4),
        S("down", 1, 512, 1792, **bf, param_std=0.01, grad_std=1e-4)),
        (), workloads.MuonHParams(ns_dtype="bf16", muon_plus=True, muon_plus_eps=1e-8, cautious="wrapper"))
    return {"llama": llama, "moe": moe, "wide": wide}


def case_llama_mini(sim):
    muon_step(sim, minis()["llama"], 2e-2)


def case_moe_mini(sim):
    muon_step(sim, minis()["moe"], 2e-2)


def case_wide_mini(sim):
    muon_step(sim, minis()["wide"], 2e-2)


def adamw_call(sim, ts, step, clip_state=None, cautious=False, seed=0, betas=(0.9, 0.999)):
    """adamw_step on guarded copies of the oracle-format tensors `ts`;
    returns the buffers (P, G, M, V) per tensor."""
    arr = (ma.AdamWTensorC * len(ts))()
    bufs = []
    for i, t in enumerate(ts):
        P, G, M, V = (sim.put(t[k]) for k in ("param", "grad", "m", "v"))
        bufs.append((P, G, M, V))
        d = arr[i]
        d.param, d.grad, d.m, d.v = (cpu_sim.addr(x) for x in (P, G, M, V))
        d.numel = P.size
        d.param_dtype, d.grad_dtype, d.moment_dtype = (DT[t[k]] for k in ("param_dtype", "grad_dtype", "moment_dtype"))
        d.lr, d.weight_decay = t["lr"], t["wd"]
    hp = ma.AdamWHParamsC(betas[0], betas[1], 1e-8, step)
    hp.cautious = ma.CAUTIOUS["wrapper"] if cautious else 0
    hp.seed = seed
    hp.clip = None if clip_state is None else cpu_sim.addr(clip_state)
    sim.ok(sim.lib.adamw_step(arr, len(ts), ctypes.byref(hp), None), "adamw")
    return bufs


def adam_tensor(n, seed):
    r = np.random.default_rng(seed)
    return {"param": storage.round_f32(r.standard_normal(n) * 0.02), "param_dtype": "f32",
            "grad": storage.round_f32(r.standard_normal(n) * 1e-3), "grad_dtype": "f32",
            "m": storage.round_f32(r.standard_normal(n) * 1e-4),
            "v": storage.round_f32(np.abs(r.standard_normal(n)) * 1e-6 + 1e-8), "moment_dtype": "f32",
            "lr": 1e-3, "wd": 0.1}


def case_clip_and_skip(sim):
    """max_norm a quarter of the norm: Muon (fp32 Newton-Schulz) and AdamW
    read the gradient times the clip factor, within 1e-5 / 1e-6 of the
    oracle's clipped step. A non-finite gradient: the state says skip, and
    every Muon and AdamW buffer keeps its bits."""
    wl = aspect2_workload("clip", 33, ns_dtype="f32")
    data = workloads.generate(wl, device="cpu", gen_device="cpu")
    adam = [adam_tensor(70000, 70)]
    grads = [(workloads.to_numpy(t.grad), t.spec.grad_dtype) for t in data.muon] + [(adam[0]["grad"], "f32")]
    norm = ognorm.global_norm(grads)
    state = grad_norm(sim, grads, norm / 4)
    cf, skip = ognorm.clip_state(norm, norm / 4)
    assert not skip and abs(state[1] - cf) <= 1e-6 * cf
    hp = hp_c(wl.muon_hp)
    hp.clip = cpu_sim.addr(state)
    muon_step(sim, wl, 1e-5, update_tol=1e-5, data=data, hp=hp, clip=float(state[1]))
    (P, G, M, V), = adamw_call(sim, adam, 1, clip_state=state)
    w = oadamw.adamw_step(adam, {"beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "step": 1}, clip=(float(state[1]), False))[0]
    assert rel(dec(P, "f32"), w["p64"]) < 1e-6 and rel(dec(M, "f32"), w["m64"]) < 1e-6

    specs = (workloads.MuonTensorSpec("a", 1, 300, 200), workloads.MuonTensorSpec("b", 2, 192, 160, views=2))
    wl = workloads.Workload("skip", 31, specs, (), workloads.MuonHParams(ns_dtype="bf16", normuon=True,
                                                                          cautious="wd_mask"))
    for bad in (np.inf, np.nan):
        data = workloads.generate(wl, device="cpu", gen_device="cpu")
        data.muon[1].grad[0, 5, 7] = float(bad)
        grads = [(workloads.to_numpy(t.grad), "f32") for t in data.muon] + [(adam[0]["grad"], "f32")]
        state = grad_norm(sim, grads, 1.0)
        assert state[2] == 1.0, state
        arr, bufs = load_muon(sim, data.muon)
        before = [[None if x is None else x.copy() for x in b] for b in bufs]
        hp = hp_c(wl.muon_hp)
        hp.clip = cpu_sim.addr(state)
        run_muon(sim, arr, len(data.muon), hp, "skipped muon_step")
        abuf = adamw_call(sim, adam, 1, clip_state=state)
        for b0, b1 in zip(before, bufs):
            for x0, x1 in zip(b0, b1):
                assert x0 is None or np.array_equal(x0.view(np.uint8), x1.view(np.uint8)), bad
        for x0, k in zip(abuf[0], ("param", "grad", "m", "v")):
            assert np.array_equal(x0, adam[0][k]), (bad, k)


NS_TABLE = [(3.4445, -4.7750, 2.0315), (3.1, -4.1, 1.8), (2.9, -3.6, 1.5), (2.4, -2.6, 1.0), (1.875, -1.25, 0.375)]


def case_ns_table(sim):
    """A different (a, b, c) per iteration and the 1.01 normalisation factor,
    against the oracle with the same table (bf16: 2e-2, fp32 on a matrix of
    aspect >= 2: 1e-5); a table of five equal rows gives the same bits as
    none; with a table the persistent launch and the per-launch schedule
    agree bit for bit."""
    for dt, shape, tol in (("bf16", (2, 256, 640), 2e-2), ("f32", (64, 300), 1e-5)):
        rnd = storage.round_bf16_bits if dt == "bf16" else storage.round_f32
        x = rnd(randn(shape, 90))
        out = newton_schulz(sim, x, dt, ma.muon_hparams(ns_dtype=dt, ns_table=NS_TABLE, ns_norm_scale=1.01))
        xs, os_ = (x, out) if x.ndim == 3 else (x[None], out[None])
        for b in range(xs.shape[0]):
            check_local(dec(os_[b], dt), omuon.newton_schulz(dec(xs[b], dt), table=NS_TABLE, norm_scale=1.01),
                        tol, (dt, b))
        plain = newton_schulz(sim, x, dt).copy()
        const = newton_schulz(sim, x, dt, ma.muon_hparams(ns_dtype=dt, ns_table=[omuon.NS_COEFFS] * 5))
        assert np.array_equal(plain, const), dt
    x = storage.round_bf16_bits(randn((2, 384, 768), 91))
    hp = ma.muon_hparams(ns_dtype="bf16", ns_table=NS_TABLE)
    outs = []
    for sched in ("launches", "persistent"):
        os.environ["MA_NS_SCHEDULE"] = sched
        try:
            outs.append(newton_schulz(sim, x, "bf16", hp).copy())
        finally:
            del os.environ["MA_NS_SCHEDULE"]
    assert np.array_equal(outs[0], outs[1])
    # the whole step with a table: Newton-Schulz inside muon_step follows it
    wl = aspect2_workload("table", 43, ns_dtype="f32")
    hp = ma.muon_hparams(ns_dtype="f32", ns_table=NS_TABLE, ns_norm_scale=1.01)
    muon_step(sim, wl, 1e-5, update_tol=1e-5, hp=hp, h_extra={"ns_table": NS_TABLE, "ns_norm_scale": 1.01})


def case_state_and_views(sim):
    """Two steps, each side continuing from its own stored state (fp32
    Newton-Schulz: parameters within 1e-5); Nesterov off; an absent gradient
    leaves its tensor alone and a zero gradient only decays it; a packed
    tensor of two views steps exactly like its halves passed separately."""
    wl = aspect2_workload("two_steps", 21, ns_dtype="f32")
    data = workloads.generate(wl, device="cpu", gen_device="cpu")
    h = hp_dict(wl.muon_hp)
    inp = [{"param": workloads.to_numpy(t.param), "param_dtype": "f32", "grad": workloads.to_numpy(t.grad),
            "grad_dtype": "f32", "momentum": workloads.to_numpy(t.momentum), "row_v": None, "views": t.spec.views,
            "lr": t.spec.lr, "wd": t.spec.wd, "shape": t.spec.shape} for t in data.muon]
    arr, bufs = load_muon(sim, data.muon)
    hp = hp_c(wl.muon_hp)
    run_muon(sim, arr, len(data.muon), hp, "step 1")
    want1 = omuon.muon_step(inp, h)
    r = np.random.default_rng(99)
    for (P, G, M, V) in bufs:
        G[...] = storage.round_f32(r.standard_normal(G.shape))
    inp2 = [dict(i, param=w["param"], momentum=w["momentum"], grad=b[1].copy()) for i, w, b in zip(inp, want1, bufs)]
    run_muon(sim, arr, len(data.muon), hp, "step 2")
    for b, w in zip(bufs, omuon.muon_step(inp2, h)):
        assert rel(dec(b[0], "f32"), w["W64"]) < 1e-5
        check_local(dec(b[2], "f32").reshape(w["B64"].shape), w["B64"], 1e-5, "momentum, step 2")

    muon_step(sim, aspect2_workload("plain_momentum", 22, ns_dtype="f32", nesterov=False), 1e-5, update_tol=1e-5)

    data = workloads.generate(aspect2_workload("absent_zero", 23), device="cpu", gen_device="cpu")
    data.muon[1].grad = None
    data.muon[2].grad = data.muon[2].grad * 0
    arr, bufs = load_muon(sim, data.muon)
    keep = [(b[0].copy(), b[2].copy()) for b in bufs]
    run_muon(sim, arr, len(data.muon), hp_c(data.workload.muon_hp), "absent and zero gradients")
    assert np.array_equal(bufs[1][0], keep[1][0]) and np.array_equal(bufs[1][2], keep[1][1])
    decay = np.float32(1.0 - np.float64(np.float32(0.02)) * np.float64(np.float32(0.1)))
    assert np.array_equal(bufs[2][0], keep[2][0] * decay) and not bufs[2][2].any()
    assert not np.array_equal(bufs[0][0], keep[0][0])

    S = workloads.MuonTensorSpec
    packed = workloads.Workload("packed", 3, (S("p", 1, 2 * 96, 160, views=2),), (), workloads.MuonHParams())
    d1 = workloads.generate(packed, device="cpu", gen_device="cpu")
    t = d1.muon[0]
    halves = workloads.WorkloadData(packed, [
        workloads.MuonTensorData(S("h0", 1, 96, 160), t.param[:, :96].contiguous(), t.grad[:, :96].contiguous(),
                                 t.momentum[:, :96].contiguous(), None),
        workloads.MuonTensorData(S("h1", 1, 96, 160), t.param[:, 96:].contiguous(), t.grad[:, 96:].contiguous(),
                                 t.momentum[:, 96:].contiguous(), None)], [])
    a1, b1 = load_muon(sim, d1.muon)
    a2, b2 = load_muon(sim, halves.muon)
    run_muon(sim, a1, 1, hp_c(packed.muon_hp), "packed")
    run_muon(sim, a2, 2, hp_c(packed.muon_hp), "halves")
    assert np.array_equal(b1[0][0][:, :96], b2[0][0]) and np.array_equal(b1[0][0][:, 96:], b2[1][0])
    assert np.array_equal(b1[0][2][:, :96], b2[0][2])


def case_symmetric_products(sim):
    """A = s X X^T and B = bA + cA^2 are stored with equal triangles, bit for
    bit, after a bf16 step (SQUARE and APPLY may read them along either
    index): every matrix's last A and B."""
    wl = aspect2_workload("symmetric", 44, ns_dtype="bf16")
    infos, ws, _ = muon_step(sim, wl, 2e-2)
    for kk, info in enumerate(infos):
        rp = info["rp"]
        for nm in ("a_offset", "b_offset"):
            o = info[nm]
            Mx = ws[o:o + rp * rp * 2].view(np.uint16).reshape(rp, rp)
            assert np.array_equal(Mx, Mx.T), (kk, nm, int((Mx != Mx.T).sum()))
            assert Mx.any(), (kk, nm)


def case_single_256x128(sim):
    muon_step(sim, workloads.workload(1), 1e-5, update_tol=1e-5)


SCHEDULES = ["together", "waves-up", "waves-down"]
CASES = {name[5:]: fn for name, fn in globals().items() if name.startswith("case_")}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("case", choices=sorted(CASES))
    ap.add_argument("--mode", default="tail", choices=("tail", "head"))
    ap.add_argument("--workers", type=int, default=8)
    ap.add_argument("--immediate-dma", action="store_true")
    ap.add_argument("--lib", default=None, help="another simulator build of the sources")
    ap.add_argument("--schedule", default="together", choices=SCHEDULES)
    ap.add_argument("--no-poison", action="store_true",
                    help="workspaces and outputs start zeroed instead of as NaN bytes")
    a = ap.parse_args(argv)
    sim = Sim(a.mode, a.workers, not a.immediate_dma, a.lib, SCHEDULES.index(a.schedule), not a.no_poison)
    try:
        CASES[a.case](sim)
    except AssertionError:
        traceback.print_exc()
        return 1
    print(f"{a.case} ({a.mode}): ok; launches {cpu_sim.counter(sim.lib, 'launches')}, "
          f"blocks {cpu_sim.counter(sim.lib, 'blocks')}, mfma {cpu_sim.counter(sim.lib, 'mfma')}, "
          f"direct loads {cpu_sim.counter(sim.lib, 'dma')}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
