"""The C-ABI library on the host: it loads, exports every declared symbol,
matches the header's struct layouts, validates arguments without touching the
GPU, and plans the five parameter sets as expected. No GPU work is enqueued:
every call here returns before its first HIP call (invalid arguments, missing
workspace, or an empty step)."""
import ctypes
import math
import os
import re
import subprocess
import sys

import numpy as np
import pytest
import torch

import muon_adamw_amd as ma
import workloads
from oracle import muon as omuon

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_adamw.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ma.LIB_PATH):
        from muon_adamw_amd import build
        build.build()
    return ma.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(ma.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ma.LIB_PATH], capture_output=True, text=True).stdout
    for name in names:
        assert re.search(rf" T {name}$", out, flags=re.M), name


def test_struct_layouts_match_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(f'''
#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
#define S(T) printf(#T " %zu\\n", sizeof(T))
#define O(T, f) printf(#T "." #f " %zu\\n", offsetof(T, f))
int main(void) {{
  S(ma_muon_tensor); O(ma_muon_tensor, batch); O(ma_muon_tensor, views); O(ma_muon_tensor, lr);
  O(ma_muon_tensor, weight_decay);
  S(ma_muon_hparams); O(ma_muon_hparams, normuon_beta2); O(ma_muon_hparams, ns_dtype); O(ma_muon_hparams, cautious);
  S(ma_adamw_tensor); O(ma_adamw_tensor, numel); O(ma_adamw_tensor, weight_decay);
  S(ma_adamw_hparams); O(ma_adamw_hparams, step);
  O(ma_muon_hparams, ns_table); O(ma_muon_hparams, clip); O(ma_muon_hparams, ns_norm_scale);
  O(ma_adamw_tensor, moment_dtype); O(ma_adamw_hparams, cautious); O(ma_adamw_hparams, seed);
  O(ma_adamw_hparams, clip); S(ma_grad_ref); O(ma_grad_ref, dtype);
  S(ma_matrix_info); O(ma_matrix_info, scale); O(ma_matrix_info, u_offset);
  O(ma_matrix_info, a_offset); O(ma_matrix_info, b_offset);
  return 0;
}}''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", str(src), "-o", str(exe)], check=True)
    got = dict(line.rsplit(" ", 1) for line in subprocess.run([str(exe)], capture_output=True,
                                                               text=True).stdout.splitlines())
    want = {
        "ma_muon_tensor": ctypes.sizeof(ma.MuonTensorC),
        "ma_muon_tensor.batch": ma.MuonTensorC.batch.offset,
        "ma_muon_tensor.views": ma.MuonTensorC.views.offset,
        "ma_muon_tensor.lr": ma.MuonTensorC.lr.offset,
        "ma_muon_tensor.weight_decay": ma.MuonTensorC.weight_decay.offset,
        "ma_muon_hparams": ctypes.sizeof(ma.MuonHParamsC),
        "ma_muon_hparams.normuon_beta2": ma.MuonHParamsC.normuon_beta2.offset,
        "ma_muon_hparams.ns_dtype": ma.MuonHParamsC.ns_dtype.offset,
        "ma_muon_hparams.cautious": ma.MuonHParamsC.cautious.offset,
        "ma_adamw_tensor": ctypes.sizeof(ma.AdamWTensorC),
        "ma_adamw_tensor.numel": ma.AdamWTensorC.numel.offset,
        "ma_adamw_tensor.weight_decay": ma.AdamWTensorC.weight_decay.offset,
        "ma_adamw_hparams": ctypes.sizeof(ma.AdamWHParamsC),
        "ma_adamw_hparams.step": ma.AdamWHParamsC.step.offset,
        "ma_muon_hparams.ns_table": ma.MuonHParamsC.ns_table.offset,
        "ma_muon_hparams.clip": ma.MuonHParamsC.clip.offset,
        "ma_muon_hparams.ns_norm_scale": ma.MuonHParamsC.ns_norm_scale.offset,
        "ma_adamw_tensor.moment_dtype": ma.AdamWTensorC.moment_dtype.offset,
        "ma_adamw_hparams.cautious": ma.AdamWHParamsC.cautious.offset,
        "ma_adamw_hparams.seed": ma.AdamWHParamsC.seed.offset,
        "ma_adamw_hparams.clip": ma.AdamWHParamsC.clip.offset,
        "ma_grad_ref": ctypes.sizeof(ma.GradRefC),
        "ma_grad_ref.dtype": ma.GradRefC.dtype.offset,
        "ma_matrix_info": ctypes.sizeof(ma.MatrixInfoC),
        "ma_matrix_info.scale": ma.MatrixInfoC.scale.offset,
        "ma_matrix_info.u_offset": ma.MatrixInfoC.u_offset.offset,
        "ma_matrix_info.a_offset": ma.MatrixInfoC.a_offset.offset,
        "ma_matrix_info.b_offset": ma.MatrixInfoC.b_offset.offset,
    }
    for k, v in want.items():
        assert int(got[k]) == v, (k, got[k], v)


def test_a_c_caller_links_the_library_and_gets_the_same_answers(tmp_path, lib):
    """The boundary from C, without Python: a program that includes the
    header and links libmuon_adamw.so describes the GPT workload's first
    layer (six tensors) with made-up device addresses, asks for the plan
    counts, the workspace size and one matrix's layout, then makes two
    invalid calls; every answer equals the binding's. Only host-side entry
    points are called: nothing reaches the GPU."""
    src = tmp_path / "caller.c"
    src.write_text(f'''
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include "{HEADER}"
int main(void) {{
  const int64_t shapes[6][2] = {{{{768, 768}}, {{768, 768}}, {{768, 768}}, {{768, 768}}, {{3072, 768}}, {{768, 3072}}}};
  ma_muon_tensor t[6];
  memset(t, 0, sizeof(t));
  uintptr_t addr = (uintptr_t)1 << 40;
  for (int i = 0; i < 6; ++i) {{
    const int64_t n = shapes[i][0] * shapes[i][1];
    t[i].param = (void*)addr; addr += (uintptr_t)n * 4 + (1 << 20);
    t[i].grad = (const void*)addr; addr += (uintptr_t)n * 4 + (1 << 20);
    t[i].momentum = (float*)addr; addr += (uintptr_t)n * 4 + (1 << 20);
    t[i].batch = 1; t[i].rows = shapes[i][0]; t[i].cols = shapes[i][1]; t[i].views = 1;
    t[i].param_dtype = MA_F32; t[i].grad_dtype = MA_F32; t[i].lr = 0.02f; t[i].weight_decay = 0.1f;
  }}
  ma_muon_hparams hp;
  memset(&hp, 0, sizeof(hp));
  hp.beta = 0.95; hp.nesterov = 1; hp.ns_steps = 5; hp.ns_a = 3.4445f; hp.ns_b = -4.7750f; hp.ns_c = 2.0315f;
  hp.ns_eps = 1e-7f; hp.ns_dtype = MA_BF16; hp.normuon_beta2 = 0.95; hp.muon_plus_eps = 1e-8f;
  int32_t nm = -1, nb = -1;
  printf("counts %d", (int)ma_muon_plan_counts(t, 6, &hp, &nm, &nb));
  printf(" %d %d\\n", nm, nb);
  printf("workspace %zu\\n", ma_muon_workspace_bytes(t, 6, &hp));
  ma_matrix_info info;
  printf("info %d", (int)ma_muon_matrix_info(t, 6, &hp, 4, &info));
  printf(" %d %d %d %d %d %llu\\n", info.tensor, info.r, info.c, info.rp, info.transposed,
         (unsigned long long)info.u_offset);
  /* the status first, then the message: ma_last_error() reads the state the
     call left behind */
  t[5].views = 7;                                   /* 7 does not divide 768 */
  int st = (int)ma_muon_plan_counts(t, 6, &hp, &nm, &nb);
  printf("views %d %s\\n", st, ma_last_error());
  t[5].views = 1;
  t[2].momentum = t[1].momentum;                    /* two tensors sharing momentum */
  st = (int)muon_step(t, 6, &hp, NULL, 0, NULL);
  printf("alias %d %s\\n", st, ma_last_error());
  return 0;
}}''')
    exe = tmp_path / "caller"
    libdir = os.path.dirname(ma.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", str(src), "-o", str(exe), ma.LIB_PATH, f"-Wl,-rpath,{libdir}"],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines()
    got = {line.split(" ", 1)[0]: line.split(" ", 1)[1] for line in out}
    wl = workloads.workload(2)
    specs = wl.muon[:6]
    arr = (ma.MuonTensorC * 6)()
    addr = 1 << 40
    for i, sp in enumerate(specs):
        n = sp.rows * sp.cols
        arr[i].param = addr; addr += n * 4 + (1 << 20)
        arr[i].grad = addr; addr += n * 4 + (1 << 20)
        arr[i].momentum = addr; addr += n * 4 + (1 << 20)
        arr[i].batch, arr[i].rows, arr[i].cols, arr[i].views = 1, sp.rows, sp.cols, 1
        arr[i].param_dtype = arr[i].grad_dtype = ma.MA_F32
        arr[i].lr, arr[i].weight_decay = 0.02, 0.1
    hp = ma.muon_hparams(ns_dtype="bf16")
    _, nm, nb = counts(lib, arr, 6, hp)
    assert got["counts"] == f"0 {nm} {nb}"
    assert int(got["workspace"]) == lib.ma_muon_workspace_bytes(arr, 6, ctypes.byref(hp))
    i4 = info(lib, arr, 6, hp, 4)
    assert got["info"] == f"0 {i4.tensor} {i4.r} {i4.c} {i4.rp} {i4.transposed} {i4.u_offset}"
    assert got["views"].startswith("1 ") and "views" in got["views"]
    assert got["alias"].startswith("3 ") and "overlapping" in got["alias"]


# ---------------------------------------------------------------------------
# descriptors with fake, non-overlapping device addresses
# ---------------------------------------------------------------------------
BASE = 1 << 40


def fake_descs(wl, gap=1 << 34):
    specs = wl.muon
    arr = (ma.MuonTensorC * len(specs))()
    addr = BASE
    for i, t in enumerate(specs):
        d = arr[i]
        es = 2 if t.param_dtype == "bf16" else 4
        n = t.batch * t.rows * t.cols
        d.param = addr; addr += n * es + gap
        d.grad = addr; addr += n * 4 + gap
        d.momentum = addr; addr += n * 4 + gap
        d.row_v = addr if wl.muon_hp.normuon else None
        addr += t.batch * t.rows * 4 + gap
        d.batch, d.rows, d.cols, d.views = t.batch, t.rows, t.cols, t.views
        d.param_dtype = ma.MA_BF16 if t.param_dtype == "bf16" else ma.MA_F32
        d.grad_dtype = ma.MA_BF16 if t.grad_dtype == "bf16" else ma.MA_F32
        d.lr, d.weight_decay = t.lr, t.wd
    return arr


def hp_of(wl):
    h = wl.muon_hp
    return ma.muon_hparams(h.beta, h.nesterov, h.ns_steps, h.ns_coeffs, h.ns_eps, h.ns_dtype, h.normuon,
                           h.normuon_beta2, h.muon_plus, h.muon_plus_eps, h.cautious)


def counts(lib, arr, n, hp):
    nm, nb = ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = lib.ma_muon_plan_counts(arr, n, ctypes.byref(hp), ctypes.byref(nm), ctypes.byref(nb))
    return st, nm.value, nb.value


@pytest.mark.parametrize("k,nmat,nbucket", [(1, 1, 1), (2, 72, 2), (3, 56, 3), (4, 192, 1), (5, 24, 2)])
def test_plan_counts(lib, k, nmat, nbucket):
    wl = workloads.workload(k)
    arr = fake_descs(wl)
    st, nm, nb = counts(lib, arr, len(wl.muon), hp_of(wl))
    assert st == 0, lib.ma_last_error()
    assert (nm, nb) == (nmat, nbucket)
    assert nm == len(wl.matrices())


def info(lib, arr, n, hp, k):
    out = ma.MatrixInfoC()
    st = lib.ma_muon_matrix_info(arr, n, ctypes.byref(hp), k, ctypes.byref(out))
    assert st == 0, lib.ma_last_error()
    return out


def test_matrix_info_canonical_shapes(lib):
    wl = workloads.workload(2)
    arr, hp = fake_descs(wl), hp_of(wl)
    up = info(lib, arr, len(wl.muon), hp, 4)          # layer 0 mlp.up 3072x768
    assert (up.m, up.n, up.r, up.c, up.transposed) == (3072, 768, 768, 3072, 1)
    assert up.scale == pytest.approx(2.0, abs=0)
    down = info(lib, arr, len(wl.muon), hp, 5)        # 768x3072
    assert (down.transposed, down.r, down.c, down.scale) == (0, 768, 3072, 1.0)
    assert up.bucket == down.bucket
    wl3 = workloads.workload(3)
    arr3, hp3 = fake_descs(wl3), hp_of(wl3)
    gate = info(lib, arr3, len(wl3.muon), hp3, 4)     # first view of l0.gate_up
    upv = info(lib, arr3, len(wl3.muon), hp3, 5)
    assert (gate.tensor, gate.view, upv.view) == (4, 0, 1)
    assert (gate.m, gate.n, gate.r, gate.c, gate.transposed) == (14336, 4096, 4096, 14336, 1)
    assert gate.scale == pytest.approx(math.sqrt(3.5), rel=1e-7)
    wl4 = workloads.workload(4)
    arr4, hp4 = fake_descs(wl4), hp_of(wl4)
    dn = info(lib, arr4, len(wl4.muon), hp4, 128)     # first expert's down 2048x1408
    assert (dn.tensor, dn.batch_index, dn.m, dn.n, dn.r, dn.c, dn.rp, dn.cp) == (1, 0, 2048, 1408, 1408,
                                                                                  2048, 1408, 2048)
    assert dn.transposed == 1


def test_workspace_bytes_cover_buffers(lib):
    wl = workloads.workload(2)
    arr, hp = fake_descs(wl), hp_of(wl)
    need = lib.ma_muon_workspace_bytes(arr, len(wl.muon), ctypes.byref(hp))
    # two X buffers + A + B per matrix at bf16, at least
    floor = sum(2 * (2 * m_r * m_c + 2 * m_r * m_r) for (_, _, _, m, n) in wl.matrices()
                for (m_r, m_c) in [(min(m, n), max(m, n))])
    assert floor <= need < floor * 1.05
    last = info(lib, arr, len(wl.muon), hp, 71)
    assert last.u_offset + last.rp * last.cp * 2 <= need


@pytest.mark.parametrize("seed", range(12))
def test_workspace_buffers_are_disjoint_and_aligned(lib, seed):
    """Random tensor lists (views, batches, ragged and tall shapes, both NS
    dtypes): every matrix's two X buffers, A and B lie past the header, inside
    the workspace, 256-byte aligned and disjoint from every other matrix's.
    The final output lands in the second X buffer after an odd step count and
    in the first after an even one, so plans for 5 and 4 steps give both X
    offsets: the step count only changes the size of tables the step keeps
    beside the buffers (queue segments, coefficients), which shifts every
    matrix's buffers by one common amount, taken from the first matrix's A
    and checked on every A and B."""
    r = np.random.default_rng(1000 + seed)
    nt = int(r.integers(1, 6))
    arr = (ma.MuonTensorC * nt)()
    addr = BASE
    for i in range(nt):
        views = int(r.choice([1, 1, 2, 3]))
        rows, cols, batch = views * int(r.integers(1, 400)), int(r.integers(1, 900)), int(r.integers(1, 4))
        d = arr[i]
        n = batch * rows * cols
        d.param = addr; addr += n * 4 + (1 << 30)
        d.grad = None if r.random() < 0.15 else addr; addr += n * 4 + (1 << 30)
        d.momentum = addr; addr += n * 4 + (1 << 30)
        d.batch, d.rows, d.cols, d.views = batch, rows, cols, views
        d.param_dtype = d.grad_dtype = ma.MA_F32
        d.lr, d.weight_decay = 0.02, 0.1
    for ns_dtype, es in (("bf16", 2), ("f32", 4)):
        hp5, hp4 = ma.muon_hparams(ns_dtype=ns_dtype, ns_steps=5), ma.muon_hparams(ns_dtype=ns_dtype, ns_steps=4)
        ws = lib.ma_muon_workspace_bytes(arr, nt, ctypes.byref(hp5))
        assert lib.ma_muon_workspace_bytes(arr, nt, ctypes.byref(hp4)) <= ws
        nm = ctypes.c_int32(0)
        assert lib.ma_muon_plan_counts(arr, nt, ctypes.byref(hp5), ctypes.byref(nm), None) == 0
        if nm.value == 0:
            assert ws == 0
            continue
        ranges = []
        shift = info(lib, arr, nt, hp5, 0).a_offset - info(lib, arr, nt, hp4, 0).a_offset
        assert shift >= 0 and shift % 256 == 0
        for k in range(nm.value):
            i5, i4 = info(lib, arr, nt, hp5, k), info(lib, arr, nt, hp4, k)
            assert (i5.a_offset, i5.b_offset) == (i4.a_offset + shift, i4.b_offset + shift)
            xb, ab = i5.rp * i5.cp * es, i5.rp * i5.rp * es
            for off, size in ((i4.u_offset + shift, xb), (i5.u_offset, xb), (i5.a_offset, ab), (i5.b_offset, ab)):
                assert off % 256 == 0 and off >= 256 and off + size <= ws, (k, off, size, ws)
                ranges.append((off, off + size, k))
        ranges.sort()
        for (lo0, hi0, k0), (lo1, hi1, k1) in zip(ranges, ranges[1:]):
            assert hi0 <= lo1, ("overlap", k0, k1, (lo0, hi0), (lo1, hi1))


@pytest.mark.parametrize("seed", range(8))
def test_alias_check_against_a_reference(lib, seed):
    """Random placements of parameters, momenta and NorMuon second moments,
    many of them touching or overlapping: the library reports MA_E_ALIAS
    exactly when some two byte ranges [start, start + size) intersect
    (gradients are read only and may be shared; tensors without a gradient
    are not stepped and are not checked)."""
    r = np.random.default_rng(2000 + seed)
    hp = ma.muon_hparams(ns_dtype="bf16", normuon=True)
    for trial in range(60):
        nt = int(r.integers(2, 5))
        arr = (ma.MuonTensorC * nt)()
        ranges = []
        for i in range(nt):
            d = arr[i]
            rows, cols = 2 * int(r.integers(1, 8)), int(r.integers(1, 8))
            d.batch, d.rows, d.cols, d.views = 1, rows, cols, 2
            d.param_dtype = d.grad_dtype = ma.MA_F32
            d.lr, d.weight_decay = 0.02, 0.1
            n = rows * cols
            # addresses on a small grid (even trials: ranges nearly always
            # touch or overlap) or a wider one (odd trials: often disjoint)
            span = 200 if trial % 2 == 0 else 20000
            pick = lambda: BASE + 4 * int(r.integers(0, span))
            d.param, d.momentum, d.row_v = pick(), pick(), pick()
            d.grad = BASE + (1 << 34)
            live = r.random() > 0.1
            if not live:
                d.grad = None
            if live:
                ranges += [(d.param, d.param + 4 * n), (d.momentum, d.momentum + 4 * n),
                           (d.row_v, d.row_v + 4 * rows)]
        ranges.sort()
        overlap = any(a[1] > b[0] for a, b in zip(ranges, ranges[1:]))
        st = lib.ma_muon_workspace_bytes(arr, nt, ctypes.byref(hp))
        err = lib.ma_last_error().decode() if st == 0 else ""
        if not ranges:                       # nothing to step: 0, and no new error
            assert st == 0
        elif overlap:
            assert st == 0 and "overlapping" in err, (trial, ranges)
        else:
            assert st > 0, (trial, err)


def step(lib, arr, n, hp, ws=None, nbytes=0):
    return lib.muon_step(arr, n, ctypes.byref(hp), ws, nbytes, None)


def test_validation_statuses(lib):
    wl = workloads.workload(2)
    n = len(wl.muon)
    hp = hp_of(wl)
    # missing workspace
    assert step(lib, fake_descs(wl), n, hp) == 4
    assert b"workspace" in lib.ma_last_error()
    # misaligned workspace
    assert step(lib, fake_descs(wl), n, hp, ctypes.c_void_p(BASE + 8), 1 << 40) == 4
    # rows not divisible by views
    arr = fake_descs(wl); arr[0].views = 5
    assert step(lib, arr, n, hp) == 1
    # complex / unknown dtype
    arr = fake_descs(wl); arr[3].grad_dtype = 9
    assert step(lib, arr, n, hp) == 2
    assert b"complex" in lib.ma_last_error()
    # tied weights passed twice
    arr = fake_descs(wl); arr[1].param = arr[0].param
    assert step(lib, arr, n, hp) == 3
    # momentum overlapping another tensor's parameter
    arr = fake_descs(wl); arr[2].momentum = arr[1].param + 16
    assert step(lib, arr, n, hp) == 3
    # NorMuon and Muon+ together
    bad = ma.muon_hparams(normuon=True, muon_plus=True)
    assert step(lib, fake_descs(wl), n, bad) == 5
    # NorMuon without row_v
    assert step(lib, fake_descs(wl), n, ma.muon_hparams(normuon=True)) == 1
    # hyperparameters
    for kw in [dict(beta=1.0), dict(ns_steps=0), dict(ns_steps=65), dict(cautious="none", ns_eps=-1.0)]:
        assert step(lib, fake_descs(wl), n, ma.muon_hparams(**kw)) == 1, kw
    hpn = ma.muon_hparams(); hpn.cautious = 3
    assert step(lib, fake_descs(wl), n, hpn) == 1
    hpn = ma.muon_hparams(); hpn.ns_a = float("nan")
    assert step(lib, fake_descs(wl), n, hpn) == 1
    # non-finite lr
    arr = fake_descs(wl); arr[0].lr = float("inf")
    assert step(lib, arr, n, hp) == 1
    # null momentum with a gradient
    arr = fake_descs(wl); arr[0].momentum = None
    assert step(lib, arr, n, hp) == 1


def test_absent_gradients_make_an_empty_step(lib):
    wl = workloads.workload(2)
    arr = fake_descs(wl)
    for i in range(len(wl.muon)):
        arr[i].grad = None
        arr[i].momentum = None
    hp = hp_of(wl)
    assert counts(lib, arr, len(wl.muon), hp)[1] == 0
    assert lib.ma_muon_workspace_bytes(arr, len(wl.muon), ctypes.byref(hp)) == 0
    # nothing to do: no workspace needed, nothing enqueued, status OK
    assert step(lib, arr, len(wl.muon), hp) == 0
    assert step(lib, arr, len(wl.muon), hp) == 0     # nothing to do, no GPU call


def test_adamw_validation(lib):
    t = (ma.AdamWTensorC * 2)()
    for i in range(2):
        t[i].param = BASE + i * (1 << 30)
        t[i].grad = BASE + (1 << 34) + i * (1 << 30)
        t[i].m = BASE + (2 << 34) + i * (1 << 30)
        t[i].v = BASE + (3 << 34) + i * (1 << 30)
        t[i].numel = 1000
        t[i].lr, t[i].weight_decay = 3e-4, 0.1
    good = ma.AdamWHParamsC(0.9, 0.95, 1e-8, 1)
    assert lib.adamw_step(t, 2, ctypes.byref(ma.AdamWHParamsC(0.9, 0.95, 1e-8, 0)), None) == 1
    assert lib.adamw_step(t, 2, ctypes.byref(ma.AdamWHParamsC(1.0, 0.95, 1e-8, 1)), None) == 1
    t[1].param = t[0].param + 400
    assert lib.adamw_step(t, 2, ctypes.byref(good), None) == 3
    t[1].param = BASE + (1 << 30)
    t[1].param_dtype = 4
    assert lib.adamw_step(t, 2, ctypes.byref(good), None) == 2
    t[1].param_dtype = 0
    t[0].grad = None
    t[1].grad = None
    assert lib.adamw_step(t, 2, ctypes.byref(good), None) == 0   # nothing to do


def test_next_row_validation(lib):
    """The clip state, the coefficient table, bf16 moments and cautious AdamW
    are validated before anything is enqueued (no GPU is touched here)."""
    wl = workloads.workload(2)
    n = len(wl.muon)
    # a table entry that is not finite; a negative norm scale; a misaligned clip state
    assert step(lib, fake_descs(wl), n, ma.muon_hparams(ns_table=[(1.0, 2.0, float("nan"))] + [(1, 0, 0)] * 4)) == 1
    assert b"ns_table" in lib.ma_last_error()
    assert step(lib, fake_descs(wl), n, ma.muon_hparams(ns_norm_scale=-1.0)) == 1
    assert step(lib, fake_descs(wl), n, ma.muon_hparams(clip=BASE + 4)) == 1
    t = (ma.AdamWTensorC * 1)()
    t[0].param, t[0].grad, t[0].m, t[0].v = BASE, BASE + (1 << 34), BASE + (2 << 34), BASE + (3 << 34)
    t[0].numel, t[0].lr, t[0].weight_decay = 1000, 3e-4, 0.1
    hp = ma.AdamWHParamsC(0.9, 0.95, 1e-8, 1)
    hp.cautious = 1                                   # Muon's weight-decay mask
    assert lib.adamw_step(t, 1, ctypes.byref(hp), None) == 5
    hp.cautious = 3
    assert lib.adamw_step(t, 1, ctypes.byref(hp), None) == 1
    hp.cautious = 0
    hp.clip = BASE + 8
    assert lib.adamw_step(t, 1, ctypes.byref(hp), None) == 1
    hp.clip = None
    t[0].moment_dtype = 7
    assert lib.adamw_step(t, 1, ctypes.byref(hp), None) == 2
    t[0].moment_dtype = ma.MA_BF16
    t[0].m = BASE + (2 << 34) + 1                     # bf16 moments need 2-byte alignment
    assert lib.adamw_step(t, 1, ctypes.byref(hp), None) == 1
    # bf16 moments occupy 2 bytes per element: ranges 2000 bytes apart do not overlap
    t[0].m, t[0].v = BASE + (2 << 34), BASE + (2 << 34) + 2000
    t[0].grad = None
    assert lib.adamw_step(t, 1, ctypes.byref(hp), None) == 0
    # global norm: workspace size, alignment, state alignment, dtype
    g = (ma.GradRefC * 3)()
    for i in range(3):
        g[i].grad, g[i].numel, g[i].dtype = BASE + i * (1 << 30), 10000 + i, ma.MA_F32
    need = lib.ma_grad_norm_workspace_bytes(g, 3)
    assert need >= 3 * 2 * 4 and need % 256 == 0
    assert lib.ma_global_grad_norm(g, 3, 1.0, BASE + 8, BASE, need, None) == 1
    assert lib.ma_global_grad_norm(g, 3, 1.0, BASE, BASE, need - 256 if need > 256 else 0, None) == 4
    assert lib.ma_global_grad_norm(g, 3, 1.0, BASE, BASE + 16, need, None) == 4
    assert lib.ma_global_grad_norm(g, 3, float("inf"), BASE, BASE, need, None) == 1
    g[1].dtype = 5
    assert lib.ma_global_grad_norm(g, 3, 1.0, BASE, BASE, need, None) == 2


def test_newton_schulz_workspace_query(lib):
    hp = ma.muon_hparams(ns_dtype="bf16")
    assert lib.ma_newton_schulz_workspace_bytes(1, 300, 200, ma.MA_BF16, ctypes.byref(hp)) > 0
    assert lib.ma_newton_schulz_workspace_bytes(1, 0, 200, ma.MA_BF16, ctypes.byref(hp)) == 0
    assert lib.ma_newton_schulz(None, None, 1, 4, 4, ma.MA_F32, ctypes.byref(hp), None, 0, None) == 1


def test_binding_rejects_host_memory_for_device_pointers():
    """The binding checks that every tensor of a call lives on the call's GPU
    before a pointer reaches the library (a host pointer would be dereferenced
    by a kernel): the device helper and the clip-state check, on the host."""
    t = torch.zeros(4)
    with pytest.raises(ValueError, match="must be on cuda:0"):
        ma._check_device(t, torch.device("cuda", 0), "momentum")
    ma._check_device(t, torch.device("cpu"), "momentum")   # same device: accepted
    with pytest.raises(ValueError, match="float32 GPU tensor"):
        ma.muon_hparams(clip=torch.zeros(4))               # a host tensor as the clip state
    with pytest.raises(TypeError):
        ma.muon_hparams(clip="state")
    assert ma.muon_hparams(clip=BASE).clip == BASE         # a raw device address passes through


def one_desc(batch, rows, cols, views=1, dt=ma.MA_F32):
    """A single fake descriptor (addresses only, nothing is dereferenced)."""
    arr = (ma.MuonTensorC * 1)()
    d = arr[0]
    es = 2 if dt == ma.MA_BF16 else 4
    n = batch * rows * cols
    d.param = BASE
    d.grad = BASE + n * es + (1 << 30)
    d.momentum = BASE + 2 * (n * es + (1 << 30))
    d.row_v = None
    d.batch, d.rows, d.cols, d.views = batch, rows, cols, views
    d.param_dtype = d.grad_dtype = dt
    d.lr, d.weight_decay = 0.02, 0.1
    return arr


def test_size_limits_and_degenerate_descriptors(lib):
    """Extents the planner refuses before touching the GPU: empty or negative
    extents, misaligned parameters, a negative tensor count (invalid, 1); one
    dimension above 65536, too many matrices in one tensor, a padded matrix
    above 2^31 elements (unsupported, 5). The largest accepted extents plan."""
    hp = ma.muon_hparams()
    ok = one_desc(1, 300, 200)
    assert counts(lib, ok, 1, hp)[1:] == (1, 1)
    for b, r, c in [(0, 4, 4), (1, 0, 4), (1, 4, 0), (-1, 4, 4)]:
        assert step(lib, one_desc(b, r, c), 1, hp) == 1, (b, r, c)
    arr = one_desc(1, 8, 8); arr[0].param = BASE + 2          # fp32 param not 4-byte aligned
    assert step(lib, arr, 1, hp) == 1
    assert lib.muon_step(ok, -1, ctypes.byref(hp), None, 0, None) == 1
    assert step(lib, one_desc(1, 65537, 8), 1, hp) == 5
    assert step(lib, one_desc(1, 8, 65537), 1, hp) == 5
    assert b"65536" in lib.ma_last_error()
    assert step(lib, one_desc((1 << 20) + 1, 4, 4), 1, hp) == 5
    assert step(lib, one_desc(1, 65536, 65536), 1, hp) == 5   # padded 2^32 elements
    assert b"too large" in lib.ma_last_error()
    # views split the rows: 2 x 65536 rows is two matrices of the largest accepted height
    big = one_desc(1, 2 * 65536, 1024, views=2)
    assert counts(lib, big, 1, hp)[1:] == (2, 1)
    assert lib.ma_muon_workspace_bytes(big, 1, ctypes.byref(hp)) > 0


def test_missing_library_fails_loudly(tmp_path):
    """No CPU fallback: loading a library that is not there raises ImportError
    (every entry point of the binding loads the library first). Checked in a
    fresh interpreter, since the binding caches the library once loaded."""
    code = ("import muon_adamw_amd as ma\n"
            f"ma.LIB_PATH = {str(tmp_path / 'missing.so')!r}\n"
            "try:\n"
            "    ma.load_library(ma.LIB_PATH)\n"
            "except ImportError as e:\n"
            "    print('ImportError', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert "ImportError" in r.stdout and "missing.so" in r.stdout


def test_matrix_expansion_matches_the_oracle_on_random_lists(lib):
    """Random tensor lists (batches, packed views, tall, wide, ragged, absent
    gradients): the planner's matrices, in order, against the oracle's expansion
    (tensor, then batch entry, then view; rows / views x cols each), with the
    canonical shape, the 128-padding, the orientation, the oracle's shape scale
    and first-appearance shape buckets."""
    r = np.random.default_rng(31)
    for trial in range(20):
        n = int(r.integers(1, 7))
        arr = (ma.MuonTensorC * n)()
        addr, expect = BASE, []
        for i in range(n):
            views = int(r.choice([1, 1, 2, 3]))
            m = int(r.choice([1, 7, 64, 128, 129, 300, 768, 1000]))
            cols = int(r.choice([1, 5, 128, 200, 768, 3072]))
            batch = int(r.choice([1, 1, 2, 4]))
            d = arr[i]
            numel = batch * m * views * cols
            d.param = addr; addr += 4 * numel + (1 << 30)
            d.grad = addr if r.random() > 0.2 else None
            addr += 4 * numel + (1 << 30)
            d.momentum = addr; addr += 4 * numel + (1 << 30)
            d.row_v = None
            d.batch, d.rows, d.cols, d.views = batch, m * views, cols, views
            d.param_dtype = d.grad_dtype = ma.MA_F32
            d.lr, d.weight_decay = 0.02, 0.1
            if d.grad:
                expect += [(i, b, v, m, cols) for b in range(batch) for v in range(views)]
        hp = ma.muon_hparams()
        st, nm, nb = counts(lib, arr, n, hp)
        assert st == 0, lib.ma_last_error()
        assert nm == len(expect)
        buckets = {}
        for k, (i, b, v, m, cols) in enumerate(expect):
            mi = info(lib, arr, n, hp, k)
            rr, cc = min(m, cols), max(m, cols)
            assert (mi.tensor, mi.batch_index, mi.view, mi.m, mi.n) == (i, b, v, m, cols)
            assert (mi.r, mi.c, mi.rp, mi.cp) == (rr, cc, -(-rr // 128) * 128, -(-cc // 128) * 128)
            assert mi.transposed == int(m > cols)
            assert mi.scale == pytest.approx(omuon.shape_scale(m, cols), rel=1e-7)
            assert mi.bucket == buckets.setdefault((rr, cc), len(buckets))
        assert nb == len(buckets)


def test_plan_cache_and_errors_are_thread_safe(lib):
    """Host calls from eight threads at once (ctypes releases the GIL during a
    foreign call): 100 tensor-list structures, more than the plan cache keeps
    (64), so it is cleared while other threads still use plans taken from it.
    Every workspace size equals the single-threaded answer, and a thread that
    makes an invalid call reads its own message from ma_last_error."""
    import threading
    rng = np.random.default_rng(5)
    hp = ma.muon_hparams(ns_dtype="bf16")

    def one(batch, rows, cols, views):
        arr = (ma.MuonTensorC * 1)()
        arr[0].param, arr[0].grad, arr[0].momentum = BASE, BASE + (1 << 36), BASE + (2 << 36)
        arr[0].batch, arr[0].rows, arr[0].cols, arr[0].views = batch, rows, cols, views
        arr[0].param_dtype = arr[0].grad_dtype = ma.MA_F32
        arr[0].lr, arr[0].weight_decay = 0.02, 0.1
        return arr

    structs = [one(1 + k % 3, int(rng.integers(1, 700)), int(rng.integers(1, 700)), 1) for k in range(100)]
    want = [lib.ma_muon_workspace_bytes(a, 1, ctypes.byref(hp)) for a in structs]
    assert all(w > 0 for w in want)
    bad = one(1, 30, 40, 7)                             # 7 does not divide 30
    problems = []

    def work(tid):
        r = np.random.default_rng(100 + tid)
        for it in range(400):
            k = int(r.integers(0, len(structs)))
            got = lib.ma_muon_workspace_bytes(structs[k], 1, ctypes.byref(hp))
            if got != want[k]:
                problems.append((tid, k, got, want[k]))
            if it % 40 == tid % 40:
                if lib.ma_muon_workspace_bytes(bad, 1, ctypes.byref(hp)) != 0 or b"views" not in lib.ma_last_error():
                    problems.append((tid, "error message", lib.ma_last_error()))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not problems, problems[:5]


def test_plan_cache_still_validates_every_call(lib):
    """A cached plan skips the planning, never the validation: the same
    structure with a misaligned or an aliased pointer is still rejected."""
    wl = workloads.workload(2)
    n = len(wl.muon)
    hp = hp_of(wl)
    arr = fake_descs(wl)
    assert lib.ma_muon_workspace_bytes(arr, n, ctypes.byref(hp)) > 0   # plan now cached
    bad = fake_descs(wl)
    bad[3].param = bad[3].param + 2                    # fp32 parameter off its 4-byte alignment
    assert step(lib, bad, n, hp) == 1 and b"aligned" in lib.ma_last_error()
    alias = fake_descs(wl)
    alias[5].momentum = alias[4].momentum              # two tensors sharing momentum
    assert step(lib, alias, n, hp) == 3
    nan_lr = fake_descs(wl)
    nan_lr[0].lr = float("nan")
    assert step(lib, nan_lr, n, hp) == 1


def test_plan_does_not_depend_on_pointers_or_values(lib):
    """Two lists of the same structure at other addresses, with other lr and
    wd, get the same workspace size and the same matrix layout."""
    wl = workloads.workload(4)
    n = len(wl.muon)
    hp = hp_of(wl)
    a = fake_descs(wl)
    b = fake_descs(wl, gap=1 << 36)
    for i in range(n):
        b[i].lr, b[i].weight_decay = 0.5, 0.0
    assert lib.ma_muon_workspace_bytes(a, n, ctypes.byref(hp)) == lib.ma_muon_workspace_bytes(b, n, ctypes.byref(hp))
    for k in (0, 63, 64, 191):
        x, y = info(lib, a, n, hp, k), info(lib, b, n, hp, k)
        assert bytes(x) == bytes(y), k


def test_plan_follows_structure_changes(lib):
    """Whatever the plan depends on is in its key: a tensor losing its
    gradient, a changed view count or shape, a changed step count."""
    wl = workloads.workload(2)
    n = len(wl.muon)
    hp = hp_of(wl)
    arr = fake_descs(wl)
    assert counts(lib, arr, n, hp)[1] == 72
    arr[0].grad = None
    assert counts(lib, arr, n, hp)[1] == 71
    arr = fake_descs(wl)
    arr[4].views = 2                                   # 3072x768 up as two 1536x768 views
    assert counts(lib, arr, n, hp)[1:] == (73, 3)
    assert (info(lib, arr, n, hp, 4).m, info(lib, arr, n, hp, 5).view) == (1536, 1)
    arr = fake_descs(wl)
    arr[0].rows = 384
    assert info(lib, arr, n, hp, 0).m == 384
    arr = fake_descs(wl)
    hp3 = hp_of(wl)
    hp3.ns_steps = 3                                   # the final output moves to the other buffer
    i5, i3 = info(lib, arr, n, hp, 0), info(lib, arr, n, hp3, 0)
    assert i5.u_offset != i3.u_offset


def test_workspace_starts_with_the_status_header(lib):
    """The first 256 bytes of a Muon workspace are the status header; the
    descriptors and tables follow, then the matrix buffers."""
    wl = workloads.workload(2)
    n = len(wl.muon)
    hp = hp_of(wl)
    arr = fake_descs(wl)
    first = min(min(info(lib, arr, n, hp, k).u_offset, info(lib, arr, n, hp, k).a_offset) for k in range(72))
    assert first >= 256 + 72 * 176
    assert first % 256 == 0


def test_step_status_query_validation(lib):
    st = ctypes.c_int32(-1)
    assert lib.ma_muon_step_status(None, ctypes.byref(st), None) == 1
    assert lib.ma_muon_step_status(BASE, None, None) == 1
    assert lib.ma_muon_step_status(BASE + 16, ctypes.byref(st), None) == 4
    assert st.value == -1


def test_grad_norm_partials_are_fp64(lib):
    """One fp64 partial per 8192-element chunk, rounded up to 256 bytes."""
    g = (ma.GradRefC * 2)()
    g[0].grad, g[0].numel, g[0].dtype = BASE, 8192 * 100, ma.MA_F32
    g[1].grad, g[1].numel, g[1].dtype = BASE + (1 << 30), 8192 * 27 + 1, ma.MA_BF16
    assert lib.ma_grad_norm_workspace_bytes(g, 2) == 1024     # 128 partials x 8 bytes


def queues(lib, arr, n, hp):
    nseg = (ctypes.c_int32 * 8)()
    assert lib.ma_muon_queue_info(arr, n, ctypes.byref(hp), nseg, None, 0) == 0
    total = sum(nseg)
    segs = (ctypes.c_int32 * max(4 * total, 1))()
    assert lib.ma_muon_queue_info(arr, n, ctypes.byref(hp), nseg, segs, total) == 0
    out, k = [], 0
    for x in range(8):
        out.append([tuple(segs[4 * (k + i): 4 * (k + i) + 4]) for i in range(nseg[x])])
        k += nseg[x]
    return out


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_persistent_queues_are_deadlock_free_and_balanced(lib, k):
    """The invariants the persistent launch's progress rests on, at the four
    bf16 workloads: every matrix sits in one XCD's queue; a queue runs in
    (iteration, product) order; the first task indices are the running tile
    count; a segment's requirement is exactly the tiles of its matrix's
    earlier products, all of which come earlier in the same queue (so a wait
    only ever depends on tasks already handed out); XCD loads differ by at
    most one matrix's work."""
    wl = workloads.workload(k)
    n = len(wl.muon)
    hp = hp_of(wl)
    arr = fake_descs(wl)
    qs = queues(lib, arr, n, hp)
    nmat = counts(lib, arr, n, hp)[1]
    steps = hp.ns_steps

    def tiles(kk):
        i = info(lib, arr, n, hp, kk)
        ntr, ntc = -(-i.rp // 256), -(-i.cp // 256)
        tri = ntr * (ntr + 1) // 2
        return (tri, tri, ntr * ntc), i

    def work(kk, op):
        t, i = tiles(kk)
        return t[op] * (i.cp if op == 0 else i.rp)

    home, loads = {}, []
    for x, q in enumerate(qs):
        start, last, done, load = 0, -1, {}, 0
        for (m, itop, first, need) in q:
            assert home.setdefault(m, x) == x, ("matrix on two XCDs", m)
            assert itop >= last, ("queue order", x)
            last = itop
            it, op = itop >> 2, itop & 3
            assert 0 <= it < steps and op in (0, 1, 2)
            assert first == start
            t, _ = tiles(m)
            assert need == it * sum(t) + (t[0] if op >= 1 else 0) + (t[1] if op >= 2 else 0)
            assert done.get(m, 0) == need, ("requirement not met by earlier segments", x, m, itop)
            done[m] = done.get(m, 0) + t[op]
            start += t[op]
            load += work(m, op)
        for m, d in done.items():
            assert d == steps * sum(tiles(m)[0])
        loads.append(load)
    assert sorted(home) == list(range(nmat))
    # the planner weighs a tile by its contraction length: padded columns for
    # the Gram, padded rows for the square and the apply
    biggest = max(sum(work(m, op) for op in range(3)) * steps for m in range(nmat))
    assert max(loads) - min(loads) <= biggest


def test_queue_info_is_empty_for_fp32_and_validates(lib):
    wl = workloads.workload(1)
    hp = hp_of(wl)
    assert queues(lib, fake_descs(wl), 1, hp) == [[]] * 8
    nseg = (ctypes.c_int32 * 8)()
    assert lib.ma_muon_queue_info(fake_descs(wl), 1, ctypes.byref(hp), None, None, 0) == 1
    assert lib.ma_muon_queue_info(fake_descs(wl), 1, ctypes.byref(hp), nseg, None, 4) == 1


def test_mfma_ceiling_validation(lib):
    """The measurement aid rejects its arguments before enqueueing anything."""
    assert lib.ma_mfma_bf16_ceiling(None, 4, 10, None) == 1
    assert lib.ma_mfma_bf16_ceiling(BASE, 0, 10, None) == 1
    assert lib.ma_mfma_bf16_ceiling(BASE, 4, 0, None) == 1
    assert lib.ma_mfma_bf16_ceiling(BASE, (1 << 20) + 1, 10, None) == 1
    assert lib.ma_mfma_bf16_ceiling(BASE + 2, 4, 10, None) == 1 and b"aligned" in lib.ma_last_error()
