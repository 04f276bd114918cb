"""The library's kernel sources, run on the CPU simulator, against the oracle.

``tests/cpu_sim`` compiles the sources under ``muon_adamw_amd/csrc`` for the
host against a CPU stand-in for HIP. Every lane is a fiber. Cross-lane
builtins, matrix-core products and direct loads into LDS carry the
instructions' semantics. Every buffer sits against a guard page.

First the simulator is checked on small kernels of its own:
- the matrix-core product against a plain matrix product;
- the transposing LDS read, the cross-lane sums, broadcasts and DPP;
- that it exposes a missing barrier, a missing wait for a direct load, a
  cross-lane operation under a divergent branch, and a write past a buffer.

Then the parity cases of ``cases.py`` run the library through its C entry
points, each in a child process, compared with the oracle at the GPU tests'
bars:
- the global norm (also at 1e20) and AdamW (bf16 moments too);
- fp32 and bf16 Newton-Schulz alone; both bf16 schedules, and both operand
  layouts, bit for bit;
- the status word when some XCD's queue gets no workgroup;
- the matrix-core ceiling loop against its closed form;
- whole Muon steps with every epilogue;
- the global-norm clip (both halves read the clipped gradient) and skip
  (every buffer keeps its bits); a per-iteration coefficient table with the
  1.01 normalisation factor; two steps continuing from stored state;
  Nesterov off; absent and zero gradients; packed views against their halves;
  A and B stored symmetric bit for bit;
- layer 0 of the GPT workload at its real shapes, and small copies of the
  Llama, MoE and wide workloads (their dtypes, views, batches, outliers and
  epilogues).
The cases run under the three lane schedules, with guard pages before and
after the buffers, and with every workspace and output filled with NaN
bytes on entry (fresh zeroed memory would hide a read of padding the library
never wrote).

A few cases also run on a build with UndefinedBehaviorSanitizer: signed
overflow in the kernels' index arithmetic, a misaligned vector access or a
bad shift stops them.

Last, the smaller tests of the GPU test files themselves run on CPU tensors
against the simulator build (``tests/cpu_sim/gpu_plugin.py``), so their own
logic and bars are checked against the kernels as written.

This checks the sources' arithmetic, indexing and synchronisation as
written. It does not check the GPU's timing, caches or compiler. A CPU
build stands in for the hardware; the GPU tests are the parity tests proper.
"""
import ctypes
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from oracle import storage
from tests import cpu_sim
from tests.cpu_sim import build as simbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def selftest_lib():
    lib = ctypes.CDLL(simbuild.build_selftest())
    P, I = ctypes.c_void_p, ctypes.c_int
    for name, args in (("st_mfma", [P, P, P, P]), ("st_tr16", [P, P]), ("st_lanes", [P, P, I]),
                       ("st_handoff", [I, I, P]), ("st_dma", [P, I, P]), ("st_divergent", [P]),
                       ("st_overrun", [P, I, I]), ("hipsim_set_schedule", [I]), ("hipsim_set_dma_deferred", [I]),
                       ("hipsim_set_workers", [I])):
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = I
    lib.hipsim_fault.restype = ctypes.c_char_p
    lib.hipsim_clear_fault.restype = None
    return lib


def ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def test_matrix_core_product(selftest_lib):
    rng = np.random.default_rng(1)
    A = storage.round_bf16_bits(rng.standard_normal((32, 16)))
    B = storage.round_bf16_bits(rng.standard_normal((16, 32)))
    C = rng.standard_normal((32, 32)).astype(np.float32)
    D = np.zeros((32, 32), np.float32)
    assert selftest_lib.st_mfma(ptr(A), ptr(B), ptr(C), ptr(D)) == 0
    want = (C.astype(np.float64) + storage.decode(A, "bf16") @ storage.decode(B, "bf16")).astype(np.float32)
    np.testing.assert_array_equal(D, want)


def test_transposing_lds_read(selftest_lib):
    src = np.arange(256, dtype=np.int16)
    out = np.zeros(256, np.int16)
    assert selftest_lib.st_tr16(ptr(src), ptr(out)) == 0
    got = out.reshape(64, 4)
    # lane l holds column l of the 4 x 64 block, rows 0..3
    np.testing.assert_array_equal(got, src.reshape(4, 64).T)


def test_cross_lane_sums_broadcast_and_quad_permute(selftest_lib):
    x = np.random.default_rng(2).standard_normal(3 * 64).astype(np.float32)
    out = np.zeros(3 * 192, np.float32)
    assert selftest_lib.st_lanes(ptr(x), ptr(out), 3) == 0
    for b in range(3):
        o = out[b * 192:(b + 1) * 192]
        np.testing.assert_allclose(o[:64], np.full(64, x[b * 64:(b + 1) * 64].astype(np.float64).sum()), rtol=1e-5)
        assert np.all(o[:64] == o[0])            # every lane ends with the same butterfly sum
        assert np.all(o[64:128] == x[b * 64] + 1.0)
        lanes = np.arange(64)
        np.testing.assert_array_equal(o[128:], (lanes & ~3) | np.array([2, 3, 0, 1])[lanes & 3])


@pytest.mark.parametrize("schedule", [0, 1, 2], ids=["together", "waves-up", "waves-down"])
def test_missing_barrier_shows(selftest_lib, schedule):
    """Wave 1 reads LDS that wave 0 writes. With the barrier every schedule
    gives wave 0's values. Without it, the schedule that runs wave 1 first
    reads the previous launch's values."""
    lib = selftest_lib
    lib.hipsim_set_schedule(schedule)
    try:
        out = np.zeros(64, np.int32)
        for base in (1000, 2000):
            assert lib.st_handoff(1, base, ptr(out)) == 0
            np.testing.assert_array_equal(out, base + np.arange(64))
        assert lib.st_handoff(0, 3000, ptr(out)) == 0
        if schedule == 2:
            np.testing.assert_array_equal(out, 2000 + np.arange(64))
        elif schedule == 1:
            np.testing.assert_array_equal(out, 3000 + np.arange(64))
    finally:
        lib.hipsim_set_schedule(0)


def test_direct_load_needs_its_wait(selftest_lib):
    lib = selftest_lib
    src = np.arange(512, dtype=np.uint16)
    out = np.zeros(512, np.uint16)
    assert lib.st_dma(ptr(src), 1, ptr(out)) == 0
    np.testing.assert_array_equal(out, src)
    assert lib.st_dma(ptr(src), 0, ptr(out)) == 0
    assert np.all(out == 0xFFFF)                 # not landed: the load was never waited for
    lib.hipsim_set_dma_deferred(0)
    try:
        assert lib.st_dma(ptr(src), 0, ptr(out)) == 0
        np.testing.assert_array_equal(out, src)
    finally:
        lib.hipsim_set_dma_deferred(1)


def test_divergent_cross_lane_operation_is_a_fault(selftest_lib):
    lib = selftest_lib
    out = np.zeros(64, np.float32)
    assert lib.st_divergent(ptr(out)) != 0
    assert b"divergent cross-lane operations" in lib.hipsim_fault()
    lib.hipsim_clear_fault()


@pytest.mark.parametrize("extra", [0, 1])
def test_guard_page_stops_a_write_past_the_buffer(selftest_lib, extra):
    code = ("import ctypes, numpy as np\n"
            "from tests import cpu_sim\n"
            f"lib = ctypes.CDLL({simbuild.SELFTEST!r})\n"
            "lib.st_overrun.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int]\n"
            "buf = cpu_sim.Arena('tail').array((100,), np.float32)\n"
            f"print(lib.st_overrun(buf.ctypes.data, 100, {extra}), flush=True)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    if extra:
        assert r.returncode == -11, (r.returncode, r.stderr)   # SIGSEGV at the guard page
    else:
        assert r.returncode == 0 and r.stdout.strip() == "0", r.stderr


# ---------------------------------------------------------------------------
# the library's kernels against the oracle
# ---------------------------------------------------------------------------
CASES = [
    ("grad_norm", ()), ("adamw", ("--mode", "head")),
    ("ns_f32", ()), ("ns_bf16", ()), ("ns_bf16", ("--schedule", "waves-up")),
    ("ns_bf16", ("--schedule", "waves-down", "--mode", "head")), ("ns_schedules", ("--schedule", "waves-down")),
    ("ns_layouts", ("--schedule", "waves-up")), ("status_undrained", ()), ("mfma_ceiling", ()),
    ("single_256x128", ()), ("muon_f32", ("--mode", "head")), ("muon_f32", ("--schedule", "waves-up")),
    ("muon_bf16", ()), ("muon_bf16", ("--schedule", "waves-down", "--mode", "head")),
    ("gpt_layer0", ()), ("llama_mini", ("--schedule", "waves-up")), ("moe_mini", ("--mode", "head")),
    ("wide_mini", ("--schedule", "waves-down")),
    ("clip_and_skip", ("--mode", "head")), ("ns_table", ("--schedule", "waves-up")), ("state_and_views", ()),
    ("symmetric_products", ("--schedule", "waves-down")),
]


# The GPU test files themselves, on CPU tensors against the simulator build
# (tests/cpu_sim/gpu_plugin.py): the smaller tests of each file.
GPU_FILES = [
    ("tests/test_gpu_next_rows.py", "not slow"),
    ("tests/test_gpu_parity.py", "f32 or small or absent or views or two_steps or zero or transpose or "
                                 "1x1 or 7x3 or 300x200 or 200x300"),
    ("tests/test_gpu_strict.py", "f32_local or epilogues or single or range_ends or huge"),
]


# Cases on a build with UndefinedBehaviorSanitizer: signed overflow in the
# kernels' index arithmetic, misaligned vector accesses, bad shifts abort.
UBSAN_CASES = [("adamw", ()), ("grad_norm", ()), ("ns_f32", ()), ("muon_bf16", ("--schedule", "waves-up")),
               ("state_and_views", ())]
UBSAN_LIB = os.path.join(simbuild.BUILD, "libmuon_adamw_sim_ubsan.so")


def _ubsan_runtime():
    import glob
    found = glob.glob(os.path.join(os.path.dirname(simbuild.CXX), "..", "lib", "clang", "*", "lib", "linux",
                                   "libclang_rt.ubsan_standalone-x86_64.so"))
    return found[0] if found else None


def _run(case, args, ubsan=False):
    cmd = [sys.executable, "-m", "tests.cpu_sim.cases", case, *args]
    env = None
    if ubsan:
        cmd += ["--lib", UBSAN_LIB]
        env = dict(os.environ, LD_PRELOAD=_ubsan_runtime(), UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=1200, env=env)


def _run_gpu_file(path, expr):
    cmd = [sys.executable, "-m", "pytest", path, "-m", "gpu", "-p", "tests.cpu_sim.gpu_plugin", "-q",
           "-p", "no:cacheprovider", "-k", expr]
    return subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=1200)


@pytest.fixture(scope="module")
def case_results():
    """All cases and GPU-file runs start at once, four at a time, once the
    simulator build is current; each test waits for its own."""
    simbuild.build()
    have_ubsan = _ubsan_runtime() is not None
    if have_ubsan:
        simbuild.build(out=UBSAN_LIB, extra=("-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                                             "-shared-libsan"))
    ex = ThreadPoolExecutor(4)
    futs = {("gpu-file", p): ex.submit(_run_gpu_file, p, e) for p, e in GPU_FILES}
    slow_first = sorted(CASES, key=lambda ca: ca[0] not in ("gpt_layer0", "ns_table", "ns_layouts", "ns_schedules"))
    futs.update({(c, a): ex.submit(_run, c, a) for c, a in slow_first})
    if have_ubsan:
        futs.update({("ubsan", c, a): ex.submit(_run, c, a, True) for c, a in UBSAN_CASES})
    yield futs
    ex.shutdown(wait=True)


@pytest.mark.parametrize("path", [p for p, _ in GPU_FILES])
def test_gpu_test_files_pass_on_the_simulator(case_results, path):
    r = case_results[("gpu-file", path)].result()
    assert r.returncode == 0, f"{path}:\n{r.stdout[-4000:]}\n{r.stderr[-2000:]}"
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]


@pytest.mark.parametrize("case,args", CASES, ids=[c + ("-" + "-".join(a[1::2]) if a else "") for c, a in CASES])
def test_kernels_against_the_oracle(case_results, case, args):
    r = case_results[(case, args)].result()
    if r.returncode < 0:
        pytest.fail(f"{case} {args}: killed by signal {-r.returncode} (11: an access hit a guard page)\n{r.stderr}")
    assert r.returncode == 0, f"{case} {args}:\n{r.stdout}\n{r.stderr}"
    assert "ok;" in r.stdout


@pytest.mark.parametrize("case,args", UBSAN_CASES, ids=[c + ("-" + "-".join(a[1::2]) if a else "") for c, a in UBSAN_CASES])
def test_kernels_under_undefined_behaviour_sanitizer(case_results, case, args):
    if ("ubsan", case, args) not in case_results:
        pytest.skip("no UndefinedBehaviorSanitizer runtime next to the compiler")
    r = case_results[("ubsan", case, args)].result()
    assert r.returncode == 0, f"{case} {args} (UBSan):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "ok;" in r.stdout and "runtime error" not in r.stderr
