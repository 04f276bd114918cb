"""pytest plugin: the GPU test files run on the CPU against the simulator build.

    python -m pytest tests/test_gpu_next_rows.py -m gpu -p tests.cpu_sim.gpu_plugin

The binding is pointed at ``tests/cpu_sim/_build/libmuon_adamw_sim.so`` (the
library's own sources compiled for the CPU simulator), and the tests' device
tensors become CPU tensors:
- ``Tensor.is_cuda`` reads true;
- ``.to(device)`` always copies, as a transfer to a GPU does;
- allocations on 'cuda' land on the CPU, with byte buffers 256-byte aligned
  as the library requires of workspaces;
- stream handles are 0 and synchronisation is a no-op (the simulator runs
  every launch to completion before it returns).

A launch fault the simulator reports fails the test that caused it.

Development and test tool only. Nothing under ``muon_adamw_amd`` loads it,
and a run with it is a CPU run of the sources, not a GPU result. It shows
that the GPU test files' own logic and bars hold against the kernels as
written.
"""
import os
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import muon_adamw_amd as ma  # noqa: E402
from tests import cpu_sim  # noqa: E402

_empty = torch.empty
_to = torch.Tensor.to


def _cpu_empty(*size, dtype=None, device=None, **kw):
    if device is not None and "cuda" in str(device):
        device = "cpu"
    if dtype == torch.uint8:
        n = size[0] if len(size) == 1 and not isinstance(size[0], (tuple, list)) else int(torch.tensor(size).prod())
        raw = _empty(n + 256, dtype=torch.uint8, device=device, **kw)
        off = (-raw.data_ptr()) % 256
        return raw[off:off + n]
    return _empty(*size, dtype=dtype, device=device, **kw)


def _copying_to(self, *a, **k):
    out = _to(self, *a, **k)
    return out.clone() if out is self else out


def pytest_configure(config):
    lib = cpu_sim.load()
    ma._lib = lib
    torch.Tensor.is_cuda = property(lambda self: True)
    torch.Tensor.to = _copying_to
    torch.empty = _cpu_empty
    ma._stream_handle = lambda stream, device: 0
    torch.cuda.synchronize = lambda *a, **k: None
    torch.cuda.empty_cache = lambda *a, **k: None
    torch.cuda.current_device = lambda: 0
    import tests.gpu_helpers as gh
    orig = gh.to_gpu
    gh.to_gpu = lambda data, device="cpu": orig(data, device="cpu")


def pytest_collection_modifyitems(session, config, items):
    import tests.gpu_helpers as gh
    for name, mod in list(sys.modules.items()):
        if name.startswith("tests.") or name.startswith(("test_", "wip_")):
            if getattr(mod, "DEV", None) == "cuda":
                mod.DEV = "cpu"
            if hasattr(mod, "to_gpu"):
                mod.to_gpu = gh.to_gpu


def pytest_runtest_teardown(item):
    fault = ma._lib.hipsim_fault()
    if fault:
        ma._lib.hipsim_clear_fault()
        raise AssertionError("simulator fault: " + fault.decode())
