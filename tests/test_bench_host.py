"""bench.py on a host without a GPU: more than one GPU is refused with a
message (the library runs on one GPU), without a visible GPU the bench fails
loudly instead of falling back to anything, and its algorithmic units and
cpu_baseline leg give the figures the roofline and the baseline report."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line


def test_no_gpu_fails_loudly():
    import pytest
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: the real bench runs instead")
    r = run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert "no GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_units():
    """The per-unit figures the roofline object divides by: Newton-Schulz FLOPs
    per matrix and iteration (one triangle for the Gram and the square, as
    computed) and the elementwise bytes per element (14 B momentum, 10 B apply,
    28 B AdamW for fp32 with bf16 Newton-Schulz buffers) on the d768 set."""
    import bench
    import workloads
    r, c = 256, 768
    assert bench.ns_flops(r, c, 1) == r * (r + 1) * c + r * (r + 1) * r + 2 * r * r * c
    assert bench.ns_flops(r, c, 5) == 5 * bench.ns_flops(r, c, 1)
    per = bench.ns_flops_per_launch([(r, c), (c, c)])
    assert per["ns_gram_bf16"] + per["ns_square_bf16"] + per["ns_apply_bf16"] == \
        bench.ns_flops_persistent([(r, c), (c, c)], 1)
    wl = workloads.workload(2)
    muon = sum(t.numel for t in wl.muon if t.has_grad)
    adam = sum(t.numel for t in wl.adamw)
    b = bench.elementwise_bytes(wl)
    assert b == {"momentum": 14 * muon, "apply_update": 10 * muon, "adamw": 28 * adam}
    assert abs(b["momentum"] / 1e9 - 1.19) < 0.01 and abs(b["adamw"] / 1e9 - 1.08) < 0.01


def test_flop_counts_per_step():
    """Newton-Schulz FLOPs of a whole step on the d768 set: dense-equivalent
    1.6307 TF (full Gram, full square, B X), algorithmic 1.1422 TF (one
    triangle for the Gram and the square, as computed), both over 72 matrices
    (48 of 768 x 768, 24 of 768 x 3072 in canonical orientation)."""
    import bench
    import workloads
    wl = workloads.workload(2)
    mats = [(min(m, n), max(m, n)) for (_, _, _, m, n) in wl.matrices()]
    assert sorted(set(mats)) == [(768, 768), (768, 3072)] and len(mats) == 72
    f = bench.ns_flop_per_step(mats, 5)
    assert abs(f["dense_equivalent"] / 1.6307e12 - 1) < 1e-4, f
    assert abs(f["algorithmic"] / 1.1422e12 - 1) < 1e-4, f
    assert f["algorithmic"] < f["dense_equivalent"]


def test_cpu_baseline_times_the_oracle():
    """The cpu_baseline leg on the small single-matrix set, on the host: the
    oracle timed on a bounded sample, reported in the GPU figure's unit."""
    import bench
    import workloads
    wl = workloads.workload(1)
    out = bench.cpu_baseline(wl, workloads.generate(wl, device="cpu"), 0.0)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert out["sample"].startswith("full fp64 Muon update of 1 of 1 matrices")


def test_reduction_bytes_and_baseline_fields():
    """One read of U per reduction pass: NorMuon (MoE set) reads the wide
    matrices by canonical rows and the tall ones by canonical columns; Muon+
    (wide-model set) reads every matrix in both passes. The baseline names its
    BLAS, the host's core count and the whole Muon half's extrapolated time."""
    import bench
    import workloads
    moe = workloads.workload(4)
    gate_up = 64 * 2 * 1408 * 2048 * 2          # wide 1408x2048 views, bf16 U
    down = 64 * 2048 * 1408 * 2                 # tall 2048x1408
    assert bench.reduction_bytes(moe) == {"rowsum": gate_up, "colsum": down}
    wide = workloads.workload(5)
    every = sum(m * n * 2 for (_, _, _, m, n) in wide.matrices())
    assert bench.reduction_bytes(wide) == {"rowsum": every, "colsum": every}
    assert bench.reduction_bytes(workloads.workload(2)) == {}
    wl = workloads.workload(1)
    out = bench.cpu_baseline(wl, workloads.generate(wl, device="cpu"), 0.0)
    assert out["os_cpu_count"] == os.cpu_count() and isinstance(out["blas"], str)
    assert out["muon_step_s_extrapolated"] > 0
