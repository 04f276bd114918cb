"""HIP path vs the fp64 oracle for the rows after the hot path (needs an
MI355X): the global-norm clip and skip, bf16 Adam moments with stochastic
rounding, the cautious wrapper over AdamW, and per-iteration Newton-Schulz
coefficients with the 1.01 normalisation factor. Every expected value comes
from the oracle run on the stored inputs."""
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
from tests.gpu_helpers import flush, host, hp_c, hp_dict, muon_params, rel, to_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def randn(shape, seed, scale=1.0, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * scale).to(dtype)


def stored(t):
    """Stored values for the oracle: float32 arrays, bf16 as uint16 bits."""
    return workloads.to_numpy(t.detach().cpu())


def dt(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


# ---------------------------------------------------------------------------
# AdamW: cautious wrapper, bf16 moments
# ---------------------------------------------------------------------------
def adam_case(n, seed, pdt=torch.float32, mdt=torch.float32):
    p = randn((n,), seed, 0.02, pdt)
    g = randn((n,), seed + 1, 1e-3, pdt)
    m = randn((n,), seed + 2, 1e-4).to(mdt)
    v = (randn((n,), seed + 3, 1e-6).abs() + 1e-8).to(mdt)
    return p, g, m, v


def run_adam(cases, step, cautious=False, seed=0, clip=None, lr=1e-3, wd=0.1):
    params = [ma.AdamWParam(p.to(DEV), g.to(DEV), m.to(DEV), v.to(DEV), lr, wd) for p, g, m, v in cases]
    ma.adamw_step(params, 0.9, 0.999, 1e-8, step, cautious=cautious, seed=seed, clip=clip)
    torch.cuda.synchronize()
    return params


def oracle_adam(cases, step, cautious=False, seed=0, clip=None, lr=1e-3, wd=0.1):
    ts = [{"param": stored(p), "param_dtype": dt(p), "grad": stored(g), "grad_dtype": dt(g),
           "m": stored(m), "v": stored(v), "moment_dtype": dt(m), "lr": lr, "wd": wd} for p, g, m, v in cases]
    return oadamw.adamw_step(ts, {"beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "step": step,
                                  "cautious": cautious, "seed": seed}, clip=clip)


@pytest.mark.parametrize("pdt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_adamw_cautious_wrapper(pdt):
    """Cautious AdamW: parameters within fp32 rounding of the oracle's; an
    entry may take the other branch only where the oracle's update is below
    1e-6 of its typical size, and masked entries are left bit for bit."""
    flush(f"adamw cautious {pdt}")
    cases = [adam_case(1 << 18, 10, pdt), adam_case(100003, 20, pdt)]
    # a large decay on some entries turns their update against the gradient
    got = run_adam(cases, 3, cautious=True, wd=5.0)
    want = oracle_adam(cases, 3, cautious=True, wd=5.0)
    for (p0, g, _, _), P, w in zip(cases, got, want):
        p0h, gh = host(p0), host(g)
        upd = p0h - w["p64"]
        masked_want = ~((upd * gh) > 0)
        near = np.abs(upd) < 1e-6 * np.sqrt(np.mean(upd * upd))
        pg = host(P.param)
        unchanged = pg == p0h
        assert np.all(unchanged[masked_want & ~near]), "masked entries must stay bit for bit"
        kept = ~masked_want & ~near
        if pdt == torch.float32:
            assert rel(pg[kept], storage.round_f32(w["p64"])[kept]) < 1e-6
        else:
            bits = storage.round_bf16_bits(pg).astype(np.int64)
            want_bits = w["param"].astype(np.int64)
            assert np.abs(bits - want_bits)[kept].max() <= 1
        assert rel(host(P.m), w["m64"]) < 1e-6 and rel(host(P.v), w["v64"]) < 1e-6
        assert 0.05 < masked_want.mean() < 0.95


@pytest.mark.parametrize("pdt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_adamw_bf16_moments(pdt):
    """bf16 moments with stochastic rounding: the stored moment bits equal the
    oracle's (SplitMix64 counter hash of the same key and flat index) except
    where the fp32 moment differs in its last bit and the carry lands
    differently (one adjacent bf16 value, rarely); parameters as for fp32
    moments; two steps, so the second reads rounded moments back (each side
    continues from its own stored state)."""
    flush(f"adamw bf16 moments {pdt}")
    cases = [adam_case(1 << 18, 30, pdt, torch.bfloat16), adam_case(100003, 40, pdt, torch.bfloat16)]
    params = [ma.AdamWParam(p.to(DEV), g.to(DEV), m.to(DEV), v.to(DEV), 1e-3, 0.1) for p, g, m, v in cases]
    ts = [{"param": stored(p), "param_dtype": dt(p), "grad": stored(g), "grad_dtype": dt(g),
           "m": stored(m), "v": stored(v), "moment_dtype": "bf16", "lr": 1e-3, "wd": 0.1} for p, g, m, v in cases]
    same = [np.ones(p.numel(), dtype=bool) for p, _, _, _ in cases]   # both sides' state equal so far
    for step in (1, 2):
        ma.adamw_step(params, 0.9, 0.999, 1e-8, step, seed=1234)
        torch.cuda.synchronize()
        # fp32 evaluation bound of each new moment's two terms (m can cancel to
        # near zero, where fp32 and fp64 may even differ in sign)
        terms = [(0.9 * np.abs(storage.decode(t["m"], "bf16")) + 0.1 * np.abs(storage.decode(t["grad"], t["grad_dtype"])),
                  0.999 * np.abs(storage.decode(t["v"], "bf16")) + 0.001 * storage.decode(t["grad"], t["grad_dtype"]) ** 2)
                 for t in ts]
        want = oadamw.adamw_step(ts, {"beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "step": step, "seed": 1234})
        for t, w in zip(ts, want):
            t["param"], t["m"], t["v"] = w["param"], w["m"], w["v"]
        got = params
        for k, (P, w, tm) in enumerate(zip(got, want, terms)):
            eq = same[k].copy()
            for nm, term in zip(("m", "v"), tm):
                gb, wb = stored(getattr(P, nm)), w[nm]
                gv, wv = storage.decode(gb, "bf16"), storage.decode(wb, "bf16")
                allowed = np.abs(wv) * 2.0 ** -7 + term * 2.0 ** -20
                # where the previous states agreed: one bf16 spacing apart at most
                assert np.all((np.abs(gv - wv) <= allowed)[same[k]]), (nm, step)
                assert np.mean(gb != wb) < 2e-3, (nm, float(np.mean(gb != wb)))
                eq &= gb == wb
            eq &= stored(P.param) == w["param"]
            same[k] = eq
            if pdt == torch.float32:
                assert rel(host(P.param), w["p64"]) < 1e-6
            else:
                pb = storage.decode(stored(P.param), "bf16")
                wp = storage.decode(w["param"], "bf16")
                assert np.all(np.abs(pb - wp) <= np.abs(wp) * 2.0 ** -7 + 1e-12)


def test_stochastic_rounding_is_unbiased_on_gpu():
    """The rounded second moment keeps small increments in expectation: v = 1,
    g^2 = 1.5, beta2 = 0.999 over 2^20 elements (round-to-nearest would keep
    v = 1 everywhere)."""
    n = 1 << 20
    p = torch.zeros(n, device=DEV)
    g = torch.full((n,), 1.5 ** 0.5, device=DEV)
    m = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    v = torch.ones(n, dtype=torch.bfloat16, device=DEV)
    ma.adamw_step([ma.AdamWParam(p, g, m, v, 0.0, 0.0)], 0.9, 0.999, 1e-8, 1, seed=5)
    inc = v.float().mean().item() - 1.0
    assert abs(inc - 0.0005) < 2e-5, inc


# ---------------------------------------------------------------------------
# Global-norm clip and skip
# ---------------------------------------------------------------------------
def test_global_grad_norm_many_tensors():
    """The norm over 70 gradients (more than one launch's table), fp32 and
    bf16, ragged sizes: within 1e-6 of the oracle's fp64 sum; the clip factor
    and flag follow its closed form; the same bits on a second run."""
    gs = [randn((int(1000 + 37 * i),), 50 + i, 1e-2, torch.bfloat16 if i % 3 == 0 else torch.float32)
          for i in range(69)] + [randn((3_000_001,), 7, 1e-3)]
    want = ognorm.global_norm([(stored(g), dt(g)) for g in gs])
    for max_norm in (0.0, want / 3, want * 2):
        st = ma.global_grad_norm([g.to(DEV) for g in gs], max_norm).cpu().numpy()
        assert abs(st[0] - want) / want < 1e-6
        f, skip = ognorm.clip_state(want, max_norm)
        assert abs(st[1] - f) < 1e-6 and st[2] == float(skip) and st[3] == 0.0
    a = ma.global_grad_norm([g.to(DEV) for g in gs], 1.0).cpu()
    b = ma.global_grad_norm([g.to(DEV) for g in gs], 1.0).cpu()
    assert torch.equal(a, b)


@pytest.mark.parametrize("bad", [float("inf"), float("nan")])
def test_skip_leaves_every_buffer(bad):
    """An overflowing gradient skips the whole hybrid step: Muon parameters,
    momentum and NorMuon V, AdamW parameters and moments all bit for bit."""
    flush(f"skip {bad}")
    specs = (workloads.MuonTensorSpec("a", 1, 300, 200), workloads.MuonTensorSpec("b", 2, 192, 160, views=2))
    wl = workloads.Workload("skip", 31, specs, (), workloads.MuonHParams(ns_dtype="bf16", normuon=True,
                                                                          cautious="wd_mask"))
    data = to_gpu(workloads.generate(wl, device="cpu"))
    data.muon[1].grad[0, 5, 7] = bad
    cases = [adam_case(50000, 60)]
    ap = [ma.AdamWParam(p.to(DEV), g.to(DEV), m.to(DEV), v.to(DEV), 1e-3, 0.1) for p, g, m, v in cases]
    grads = [t.grad for t in data.muon] + [a.grad for a in ap]
    state = ma.global_grad_norm(grads, 1.0)
    before = [(t.param.clone(), t.momentum.clone(), t.row_v.clone()) for t in data.muon] + \
             [(a.param.clone(), a.m.clone(), a.v.clone()) for a in ap]
    hp = hp_c(wl.muon_hp)
    hp = ma.muon_hparams(**{**_hp_kwargs(wl.muon_hp), "clip": state})
    ma.muon_step(muon_params(data), hp)
    ma.adamw_step(ap, 0.9, 0.999, 1e-8, 1, clip=state)
    torch.cuda.synchronize()
    assert state.cpu()[2].item() == 1.0
    after = [(t.param, t.momentum, t.row_v) for t in data.muon] + [(a.param, a.m, a.v) for a in ap]
    for b, a in zip(before, after):
        for x, y in zip(b, a):
            assert torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                               y.view(torch.uint8) if y.dtype != torch.uint8 else y)


def _hp_kwargs(h):
    return dict(beta=h.beta, nesterov=h.nesterov, ns_steps=h.ns_steps, ns_coeffs=h.ns_coeffs, ns_eps=h.ns_eps,
                ns_dtype=h.ns_dtype, normuon=h.normuon, normuon_beta2=h.normuon_beta2, muon_plus=h.muon_plus,
                muon_plus_eps=h.muon_plus_eps, cautious=h.cautious)


def test_clipped_step_matches_oracle():
    """max_norm below the norm: both halves see the gradient times the clip
    factor. Muon with fp32 Newton-Schulz (tall, wide and packed matrices of
    aspect >= 1.5): parameters and momentum within 1e-5 of the oracle's
    clipped step; AdamW within 1e-6."""
    specs = (workloads.MuonTensorSpec("a", 1, 384, 128), workloads.MuonTensorSpec("b", 2, 2 * 64, 160, views=2),
             workloads.MuonTensorSpec("c", 1, 64, 500))
    wl = workloads.Workload("clip", 33, specs, (), workloads.MuonHParams(ns_dtype="f32"))
    data = to_gpu(workloads.generate(wl, device="cpu"))
    inp = [{"param": stored(t.param), "param_dtype": "f32", "grad": stored(t.grad), "grad_dtype": "f32",
            "momentum": stored(t.momentum), "row_v": None, "views": t.spec.views, "lr": t.spec.lr,
            "wd": t.spec.wd, "shape": t.spec.shape} for t in data.muon]
    cases = [adam_case(70000, 70)]
    ap = [ma.AdamWParam(p.to(DEV), g.to(DEV), m.to(DEV), v.to(DEV), 1e-3, 0.1) for p, g, m, v in cases]
    grads = [t.grad for t in data.muon] + [a.grad for a in ap]
    norm = ognorm.global_norm([(stored(g), "f32") for g in grads])
    max_norm = norm / 4
    clip = ognorm.clip_state(norm, max_norm)
    state = ma.global_grad_norm(grads, max_norm)
    ma.muon_step(muon_params(data), ma.muon_hparams(**{**_hp_kwargs(wl.muon_hp), "clip": state}))
    ma.adamw_step(ap, 0.9, 0.999, 1e-8, 1, clip=state)
    torch.cuda.synchronize()
    want = omuon.muon_step(inp, hp_dict(wl.muon_hp), clip=clip)
    for t, w, i in zip(data.muon, want, inp):
        W0 = storage.decode(i["param"], "f32").reshape(w["W64"].shape)
        assert rel(host(t.param) - W0, w["W64"] - W0) < 1e-5
        assert rel(host(t.momentum), w["B64"]) < 1e-5
    wa = oracle_adam(cases, 1, clip=clip)[0]
    assert rel(host(ap[0].param), wa["p64"]) < 1e-6 and rel(host(ap[0].m), wa["m64"]) < 1e-6


# ---------------------------------------------------------------------------
# Per-iteration Newton-Schulz coefficients, 1.01 normalisation factor
# ---------------------------------------------------------------------------
TABLE = [(3.4445, -4.7750, 2.0315), (3.1, -4.1, 1.8), (2.9, -3.6, 1.5), (2.4, -2.6, 1.0), (1.875, -1.25, 0.375)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ns_coefficient_table(dtype):
    """A table with a different (a, b, c) per iteration and the 1.01 factor,
    against the oracle with the same table (bf16: 2e-2; fp32: 1e-5 on a
    matrix of aspect >= 2); a constant table gives the same bits as none."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = randn((3, 256, 640) if dtype == "bf16" else (64, 300), 90, dtype=tdt)
    hp = ma.muon_hparams(ns_dtype=dtype, ns_table=TABLE, ns_norm_scale=1.01)
    out = ma.newton_schulz(x.to(DEV), hp)
    xs = host(x)
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for b in range(xs.shape[0] if xs.ndim == 3 else 1):
        xi = xs[b] if xs.ndim == 3 else xs
        oi = host(out)[b] if xs.ndim == 3 else host(out)
        assert rel(oi, omuon.newton_schulz(xi, table=TABLE, norm_scale=1.01)) < tol
    plain = ma.newton_schulz(x.to(DEV), ma.muon_hparams(ns_dtype=dtype))
    const = ma.newton_schulz(x.to(DEV), ma.muon_hparams(ns_dtype=dtype, ns_table=[omuon.NS_COEFFS] * 5))
    assert torch.equal(plain.view(torch.int16 if dtype == "bf16" else torch.int32),
                       const.view(torch.int16 if dtype == "bf16" else torch.int32))


def test_ns_table_persistent_matches_launches():
    """The persistent launch reads iteration it's row from the device table;
    the per-launch schedule passes it per launch: the same bits."""
    x = randn((2, 768, 1536), 91, dtype=torch.bfloat16)
    hp = ma.muon_hparams(ns_dtype="bf16", ns_table=TABLE)
    outs = {}
    for sched in ("launches", "persistent"):
        os.environ["MA_NS_SCHEDULE"] = sched
        try:
            outs[sched] = ma.newton_schulz(x.to(DEV), hp).cpu()
        finally:
            del os.environ["MA_NS_SCHEDULE"]
    assert torch.equal(outs["launches"].view(torch.int16), outs["persistent"].view(torch.int16))
