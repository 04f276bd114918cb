"""Benchmark of the hybrid Muon + AdamW step on one MI355X.

Default workload: the GPT-style 12-layer d=768 parameter set (72 Muon
matrices: Q, K, V, O 768x768, MLP up 3072x768 and down 768x3072, fp32 storage,
bf16 Newton-Schulz; AdamW on the tied 50304x768 embedding and 25 RMSNorm
weights). A step is one muon_step plus one adamw_step over the whole set, with
every input already resident in HBM. Prints one JSON line.

The Newton-Schulz figures use algorithmic FLOPs of what is computed: per
iteration r(r+1)c for the Gram (one triangle), r(r+1)r for A^2 (one triangle)
and 2r^2c for B X, per canonical r x c matrix. With the bf16 chain in one
persistent launch (ns_persistent_bf16), a launch covers all iterations.
"""
import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

BF16_PEAK_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz, dense
HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, help="parameter set 1-5 (default 2)")
    ap.add_argument("--profile-steps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work to time")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip timing the global-norm pass and the AdamW variants")
    return ap.parse_args()


def ns_flops(r, c, steps):
    return steps * (r * (r + 1) * c + r * (r + 1) * r + 2 * r * r * c)


def ns_flops_dense(r, c, steps):
    """Dense-equivalent FLOPs of Newton-Schulz: the full Gram (2 r^2 c), the
    full square (2 r^3) and B X (2 r^2 c). A label for comparison with dense
    GEMM counts; the achieved figures use ns_flops."""
    return steps * (4 * r * r * c + 2 * r ** 3)


def ns_flop_per_step(mats, steps):
    """Newton-Schulz FLOPs of one step, algorithmic (as computed) and
    dense-equivalent, over canonical (r, c) shapes."""
    return {"algorithmic": sum(ns_flops(r, c, steps) for r, c in mats),
            "dense_equivalent": sum(ns_flops_dense(r, c, steps) for r, c in mats)}


def ns_flops_per_launch(mats):
    """Algorithmic FLOPs of one launch of each Newton-Schulz product."""
    gram = sum(r * (r + 1) * c for r, c in mats)
    square = sum(r * (r + 1) * r for r, c in mats)
    apply = sum(2 * r * r * c for r, c in mats)
    return {"ns_gram_bf16": gram, "ns_square_bf16": square, "ns_apply_bf16": apply,
            "ns_gram_f32": gram, "ns_square_f32": square, "ns_apply_f32": apply}


def ns_flops_persistent(mats, steps):
    """Algorithmic FLOPs of the single launch that runs every iteration."""
    return sum(ns_flops(r, c, steps) for r, c in mats)


def next_rows(data, aparams, ah, stream, reps):
    """Kernel times of the rows after the hot path, outside the timed step:
    the global-norm pass over every gradient of the step (one read of each),
    and AdamW with bf16 moments (20 B per fp32 element) and with the cautious
    wrapper (28 B). Runs on copies; the step's own state is untouched."""
    import torch
    import muon_adamw_amd as ma
    out = {}
    grads = [t.grad for t in data.muon if t.grad is not None] + [a.grad for a in aparams]
    gbytes = sum(g.numel() * g.element_size() for g in grads)
    state = torch.zeros(4, dtype=torch.float32, device=grads[0].device)
    ma.global_grad_norm(grads, 1.0, state)
    ma.profile_begin()
    for _ in range(reps):
        ma.global_grad_norm(grads, 1.0, state, stream=stream)
    prof = ma.profile_end()
    us = sum(v[1] for v in prof.values()) / reps * 1e3
    out["global_grad_norm"] = {"avg_us": us, "bytes": gbytes, "achieved": gbytes / us / 1e3,
                               "unit": "GB/s", "frac": gbytes / us / 1e3 / HBM_PEAK_GBPS,
                               "kernels": {k: v[1] / reps * 1e3 for k, v in prof.items()}}
    if aparams:
        n = sum(a.param.numel() for a in aparams)
        for name, kw, mdt, per in (("adamw_bf16_moments", {}, torch.bfloat16, 20),
                                   ("adamw_cautious", {"cautious": True}, torch.float32, 28)):
            cp = [ma.AdamWParam(a.param.clone(), a.grad, a.m.to(mdt), a.v.to(mdt), a.lr, a.weight_decay)
                  for a in aparams]
            ma.adamw_step(cp, ah.beta1, ah.beta2, ah.eps, ah.step, stream, **kw)
            ma.profile_begin()
            for i in range(reps):
                ma.adamw_step(cp, ah.beta1, ah.beta2, ah.eps, ah.step + 1 + i, stream, **kw)
            prof = ma.profile_end()
            us = prof["adamw"][1] / prof["adamw"][0] * 1e3
            by = n * per if all(a.param.dtype == torch.float32 for a in aparams) else None
            out[name] = {"avg_us": us, "bytes": by, "achieved": None if by is None else by / us / 1e3,
                         "unit": "GB/s", "frac": None if by is None else by / us / 1e3 / HBM_PEAK_GBPS}
            del cp
    torch.cuda.synchronize()
    return out


def progress(msg):
    """One line per finished phase on stderr (a long profiled run shows it is
    alive; the JSON line on stdout stays the only result)."""
    print(f"# {msg}", file=sys.stderr, flush=True)


def elementwise_bytes(wl):
    """Algorithmic HBM bytes of one launch of each elementwise kernel."""
    es = {"f32": 4, "bf16": 2}
    nsb = es[wl.muon_hp.ns_dtype]
    mom = 0
    app = 0
    for t in wl.muon:
        if not t.has_grad:
            continue
        n = t.numel
        mom += n * (es[t.grad_dtype] + 4 + 4 + nsb)
        app += n * (2 * es[t.param_dtype] + nsb + (es[t.grad_dtype] if wl.muon_hp.cautious == "wrapper" else 0))
    adam = sum(t.numel * (2 * es[t.param_dtype] + es[t.grad_dtype] + 16) for t in wl.adamw)
    return {"momentum": mom, "apply_update": app, "adamw": adam}


def reduction_bytes(wl):
    """Algorithmic HBM bytes per step of the NorMuon / Muon+ reductions: one
    read of U (ns dtype) per pass. A canonical-row pass covers the wide
    matrices (NorMuon; Muon+ stage 1) and, with Muon+, the tall ones in stage 2;
    a canonical-column pass the other way round."""
    h = wl.muon_hp
    if not (h.normuon or h.muon_plus):
        return {}
    es = 2 if h.ns_dtype == "bf16" else 4
    wide = sum(m * n * es for (_, _, _, m, n) in wl.matrices() if m <= n)
    tall = sum(m * n * es for (_, _, _, m, n) in wl.matrices() if m > n)
    if h.muon_plus:
        return {"rowsum": wide + tall, "colsum": wide + tall}
    return {"rowsum": wide, "colsum": tall}


def single_matrix_latency(stream, reps=200):
    """Step time of the single fp32 256x128 matrix with fp32 Newton-Schulz (a
    latency-bound step of 18 launches), timed with events over `reps` steps."""
    import torch
    import muon_adamw_amd as ma
    import workloads
    wl = workloads.workload(1)
    d = workloads.generate(wl, device="cuda")
    h = wl.muon_hp
    hp = ma.muon_hparams(h.beta, h.nesterov, h.ns_steps, h.ns_coeffs, h.ns_eps, h.ns_dtype)
    ps = [ma.MuonParam(t.param, t.grad, t.momentum, None, t.spec.views, t.spec.lr, t.spec.wd) for t in d.muon]
    ws = torch.empty(ma.muon_workspace_bytes(ps, hp), dtype=torch.uint8, device="cuda")
    for _ in range(10):
        ma.muon_step(ps, hp, ws, stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        ma.muon_step(ps, hp, ws, stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    return {"step_us": round(ev[0].elapsed_time(ev[1]) / reps * 1e3, 2), "steps": reps}


def cpu_baseline(wl, data, budget_s):
    """The fp64 oracle, untuned, on a bounded sample of the same workload:
    whole Muon updates of the first matrices in tensor order until the time
    budget is spent. Reported in the same unit as the GPU figure."""
    from oracle import muon as omuon
    from workloads import to_numpy
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"] or threadpool_info()
        threads = max([p.get("num_threads", 1) for p in pools] or [os.cpu_count()])
        blas = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in pools})) or "unknown"
    except Exception:  # pragma: no cover
        threads, blas = os.cpu_count(), "unknown"
    h = wl.muon_hp
    hp = {"beta": h.beta, "nesterov": h.nesterov, "ns_steps": h.ns_steps, "ns_coeffs": h.ns_coeffs,
          "ns_eps": h.ns_eps, "normuon": h.normuon, "normuon_beta2": h.normuon_beta2,
          "muon_plus": h.muon_plus, "muon_plus_eps": h.muon_plus_eps, "cautious": h.cautious}
    flops = 0
    nmat = 0
    spent = 0.0
    for t in data.muon:
        if t is None or t.grad is None:
            continue
        inp = {"param": to_numpy(t.param), "param_dtype": t.spec.param_dtype, "grad": to_numpy(t.grad),
               "grad_dtype": t.spec.grad_dtype, "momentum": to_numpy(t.momentum),
               "row_v": None if t.row_v is None else to_numpy(t.row_v), "views": t.spec.views,
               "lr": t.spec.lr, "wd": t.spec.wd, "shape": t.spec.shape}
        t0 = time.perf_counter()
        omuon.muon_step([inp], hp)
        spent += time.perf_counter() - t0
        for (_, _, m, n) in t.spec.matrices():
            flops += ns_flops(min(m, n), max(m, n), h.ns_steps)
            nmat += 1
        if spent >= budget_s:
            break
    total = len(wl.matrices())
    all_flops = sum(ns_flops(min(m, n), max(m, n), h.ns_steps) for (_, _, _, m, n) in wl.matrices())
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"full fp64 Muon update of {nmat} of {total} matrices ({spent:.1f} s)",
            "matrices_per_s": nmat / spent, "os_cpu_count": os.cpu_count(), "blas": blas,
            # the whole Muon half at the sample's rate (extrapolated from nmat of total matrices)
            "muon_step_s_extrapolated": all_flops / (flops / spent)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported: the library "
              "has no multi-GPU path (the sharding across GPUs is a design, not an implementation).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import muon_adamw_amd as ma
    import workloads

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    wl = workloads.workload(args.config)
    dev = "cuda"
    t0 = time.time()
    data = workloads.generate(wl, device=dev)
    print(f"# generated {wl.name} in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    h = wl.muon_hp
    hp = ma.muon_hparams(h.beta, h.nesterov, h.ns_steps, h.ns_coeffs, h.ns_eps, h.ns_dtype, h.normuon,
                         h.normuon_beta2, h.muon_plus, h.muon_plus_eps, h.cautious)
    mparams = [ma.MuonParam(t.param, t.grad, t.momentum, t.row_v, t.spec.views, t.spec.lr, t.spec.wd)
               for t in data.muon]
    aparams = [ma.AdamWParam(t.param, t.grad, t.m, t.v, t.spec.lr, t.spec.wd) for t in data.adamw]
    ah = wl.adamw_hp
    ws = torch.empty(ma.muon_workspace_bytes(mparams, hp), dtype=torch.uint8, device=dev)
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle reads the pre-step state, so time it before the GPU steps
        cpu = cpu_baseline(wl, data, args.cpu_budget)
        print(f"# cpu baseline: {cpu['sample']}", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    step_no = [ah.step]

    def hybrid_step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ma.muon_step(mparams, hp, ws, stream)
        if ev is not None:
            ev[1].record(stream)
        if aparams:
            ma.adamw_step(aparams, ah.beta1, ah.beta2, ah.eps, step_no[0], stream)
            step_no[0] += 1
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        hybrid_step()
    torch.cuda.synchronize()
    progress(f"{args.warmup} warm-up steps done")

    # whole-step timing
    t_start = time.perf_counter()
    for _ in range(args.steps):
        hybrid_step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t_start) / args.steps
    progress(f"{args.steps} timed steps: {wall * 1e3:.3f} ms each")
    # device status of the last timed step (outside the timed region): 0, or
    # the persistent launch's safeguard bits, in which case its results and
    # therefore this line are not to be trusted
    ns_status = ma.muon_step_status(ws, stream)
    if ns_status:
        print(f"warning: muon_step status {ns_status} (a bounded wait ran out or a queue was not drained)",
              file=sys.stderr, flush=True)

    # host time of one muon_step call (binding + validation + cached plan +
    # descriptor upload + launches; the device work is only enqueued)
    host_s = []
    for _ in range(args.steps):
        t0 = time.perf_counter()
        ma.muon_step(mparams, hp, ws, stream)
        host_s.append(time.perf_counter() - t0)
    torch.cuda.synchronize()

    # muon / adamw split with events on the step stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in evs:
        hybrid_step(e)
    torch.cuda.synchronize()
    muon_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs)
    adam_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / len(evs)
    progress(f"event split: muon_step {muon_ms:.3f} ms, adamw_step {adam_ms:.3f} ms")

    # per-kernel HIP-event timing (separate pass: events add gaps)
    ma.profile_begin()
    for _ in range(args.profile_steps):
        hybrid_step()
    prof = ma.profile_end()
    progress("per-kernel timing pass done")

    # measured ceiling of plain streaming: a 1 GiB device-to-device copy
    # (torch's copy kernel), 2 GiB of traffic per copy
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(2 if args.calib_copy else 1):
        b.copy_(a)
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record(stream)
    for _ in range(5):
        b.copy_(a)
    ce[1].record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 5 / (ce[0].elapsed_time(ce[1]) / 1e3) / 1e9
    del a, b
    # measured ceiling of the bf16 matrix cores: the MFMA-only loop (no
    # memory traffic), 1024 workgroups of 4 waves; the counter summary
    # calibrates its MFMA-op counter on the same launch
    from muon_adamw_amd import counters
    sink = torch.empty(counters.CEILING_BLOCKS, dtype=torch.float32, device=dev)
    ma.mfma_bf16_ceiling(sink, counters.CEILING_BLOCKS, counters.CEILING_ITERS // 10, stream)
    ce[0].record(stream)
    mfma_flops = ma.mfma_bf16_ceiling(sink, counters.CEILING_BLOCKS, counters.CEILING_ITERS, stream)
    ce[1].record(stream)
    torch.cuda.synchronize()
    mfma_tflops = mfma_flops / (ce[0].elapsed_time(ce[1]) / 1e3) / 1e12
    progress(f"ceilings: copy {copy_gbps:.0f} GB/s, MFMA loop {mfma_tflops:.0f} TFLOP/s")

    nxt = None if args.no_next_rows else next_rows(data, aparams, ah, stream, args.profile_steps)
    single = None if args.config == 1 or args.no_next_rows else single_matrix_latency(stream)

    mats = [(min(m, n), max(m, n)) for (_, _, _, m, n) in wl.matrices()]
    fl = ns_flops_per_launch(mats)
    fl["ns_persistent_bf16"] = ns_flops_persistent(mats, h.ns_steps)
    ns_total_flops = sum(ns_flops(r, c, h.ns_steps) for r, c in mats)
    by = elementwise_bytes(wl)
    by_step = reduction_bytes(wl)
    kernels = {}
    for name, (launches, total_ms) in prof.items():
        avg_s = total_ms / launches / 1e3
        k = {"launches_per_step": launches / args.profile_steps, "avg_us": avg_s * 1e6}
        if name in fl:
            ach = fl[name] / avg_s / 1e12
            peak = BF16_PEAK_TFLOPS if name.endswith("bf16") else 157.3
            k.update(bound="mfma" if name.endswith("bf16") else "alu", achieved=ach, peak=peak,
                     unit="TFLOP/s", frac=ach / peak)
        elif name in by:
            ach = by[name] / avg_s / 1e9
            k.update(bound="hbm", achieved=ach, peak=HBM_PEAK_GBPS, unit="GB/s", frac=ach / HBM_PEAK_GBPS)
        elif name in by_step:
            # launches of one name differ in size: bytes of a step over its time
            ach = by_step[name] / (total_ms / args.profile_steps / 1e3) / 1e9
            k.update(bound="hbm", achieved=ach, peak=HBM_PEAK_GBPS, unit="GB/s", frac=ach / HBM_PEAK_GBPS)
        else:
            k.update(bound="latency")     # one small block per matrix, or a status word
        kernels[name] = k
    ns_kernel_s = sum(prof[n][1] for n in prof if n.startswith("ns_")) / args.profile_steps / 1e3
    dominant = max(prof, key=lambda n: prof[n][1])
    dk = kernels[dominant]
    # HBM bytes per launch from the committed counter summary of this
    # workload (FETCH_SIZE/WRITE_SIZE passes, copy-calibrated), while the
    # kernel sources are unchanged since it was taken
    summary = os.path.join(HERE, "profiles", f"counters_{wl.name}.json")
    traffic = counters.traffic_for(summary, dominant)
    roofline = {"bound": dk.get("bound"), "achieved": dk.get("achieved"), "peak": dk.get("peak"),
                "unit": dk.get("unit"), "frac": dk.get("frac"), "traffic": traffic, "kernel": dominant}
    # flops the matrix cores executed per launch (MFMA-op counter, calibrated
    # on the ceiling loop), beside the algorithmic flops the rate divides
    counted = counters.flops_for(summary, dominant) if dk.get("bound") == "mfma" else None
    if counted:
        roofline.update(flops_counted=counted, flops_algorithmic=fl.get(dominant))
    # the same achieved figure against the ceilings measured in this run
    measured = {"mfma": mfma_tflops, "hbm": copy_gbps}.get(dk.get("bound"))
    if measured and dk.get("achieved"):
        roofline.update(peak_measured=round(measured, 1), frac_measured=dk["achieved"] / measured)
    muon_s = muon_ms / 1e3
    value = ns_total_flops / muon_s / 1e12
    line = {
        "metric": "Muon step time & NS TFLOP/s (% bf16 MFMA peak); AdamW GB/s, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h.ns_dtype if h.ns_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "muon_matrices": len(mats),
                   "adamw_elements": sum(t.numel for t in wl.adamw), "ns_steps": h.ns_steps,
                   "parallelism": "none (1 GPU)"},
        "muon_step_ms": round(muon_ms, 4),
        "adamw_step_ms": round(adam_ms, 4),
        "matrices_per_s": round(len(mats) / muon_s, 1),
        "ns_flop_per_step": ns_flop_per_step(mats, h.ns_steps),
        "ns_tflops_kernels": round(ns_total_flops / ns_kernel_s / 1e12, 3),
        "ns_frac_of_bf16_peak": round(ns_total_flops / ns_kernel_s / 1e12 / BF16_PEAK_TFLOPS, 4),
        "adamw_GBps": round(by["adamw"] / (adam_ms / 1e3) / 1e9, 1) if aparams else None,
        "roofline": roofline,
        "kernels": kernels,
        "ns_status": ns_status,
        "host_us_per_muon_step": round(1e6 * sorted(host_s)[len(host_s) // 2], 1),
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "mfma_ceiling_TFLOPs": round(mfma_tflops, 1),
        "cpu_baseline": cpu,
        "next_rows": nxt,
        "single_256x128_f32": single,
    }
    if cpu is not None:
        cpu["gpu_speedup_muon_step"] = round(cpu["muon_step_s_extrapolated"] / muon_s, 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
