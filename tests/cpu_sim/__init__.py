"""The library's kernels run on the CPU (test infrastructure).

``build.py`` compiles the library's own sources against a CPU stand-in for the
HIP runtime (``include/hip/hip_runtime.h``, ``runtime.cpp``). ``load()`` opens
that build through the same C declarations as the product binding. Buffers
come from ``Arena``: every buffer sits against an inaccessible guard page, so
an access past its end (``"tail"``) or before its start (``"head"``) stops the
process at once. Cases that may fault therefore run in a child process (see
``cases.py``).
"""
from __future__ import annotations

import ctypes
import mmap
import os

import numpy as np


LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "libmuon_adamw_sim.so")
PAGE = mmap.PAGESIZE
_libc = ctypes.CDLL(None, use_errno=True)
_libc.mprotect.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
_libc.mprotect.restype = ctypes.c_int

COUNTERS = {"launches": 0, "blocks": 1, "wave_ops": 2, "barriers": 3, "dma": 4, "mfma": 5, "skipped": 6}


def load(path: str = LIB) -> ctypes.CDLL:
    import muon_adamw_amd as ma
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m tests.cpu_sim.build`")
    lib = ma.declare(ctypes.CDLL(path))
    lib.hipsim_set_workers.argtypes = [ctypes.c_int]
    lib.hipsim_set_workers.restype = ctypes.c_int
    lib.hipsim_set_dma_deferred.argtypes = [ctypes.c_int]
    lib.hipsim_set_dma_deferred.restype = ctypes.c_int
    lib.hipsim_set_xcds.argtypes = [ctypes.c_int]
    lib.hipsim_set_xcds.restype = ctypes.c_int
    lib.hipsim_set_schedule.argtypes = [ctypes.c_int]
    lib.hipsim_set_schedule.restype = ctypes.c_int
    lib.hipsim_fault.argtypes = []
    lib.hipsim_fault.restype = ctypes.c_char_p
    lib.hipsim_clear_fault.argtypes = []
    lib.hipsim_clear_fault.restype = None
    lib.hipsim_counter.argtypes = [ctypes.c_int]
    lib.hipsim_counter.restype = ctypes.c_longlong
    return lib


def counter(lib, name: str) -> int:
    return int(lib.hipsim_counter(COUNTERS[name]))


class Arena:
    """Buffers each placed against a guard page.

    ``mode="tail"``: the buffer ends 0-15 bytes before an inaccessible page
    (the start stays 16-byte aligned, as the kernels' vector accesses need).
    ``mode="head"``: it starts right after one (page-aligned).
    ``poison``: every buffer starts as 0xFF bytes (NaN as fp32 or bf16), so
    workspaces and outputs hold garbage on entry, as callers may pass them;
    inputs are copied over it (``like``)."""

    def __init__(self, mode: str = "tail", poison: bool = False):
        assert mode in ("tail", "head")
        self.mode = mode
        self.poison = poison
        self._maps = []

    def bytes(self, nbytes: int) -> np.ndarray:
        nbytes = max(int(nbytes), 1)
        body = (nbytes + PAGE - 1) // PAGE * PAGE
        total = body + 2 * PAGE
        m = mmap.mmap(-1, total, prot=mmap.PROT_READ | mmap.PROT_WRITE)
        base = ctypes.addressof(ctypes.c_char.from_buffer(m))
        for off in (0, total - PAGE):
            if _libc.mprotect(base + off, PAGE, 0) != 0:
                raise OSError(ctypes.get_errno(), "mprotect failed")
        if self.mode == "head":
            start = PAGE
        else:
            start = (PAGE + body - nbytes) // 16 * 16
        self._maps.append(m)
        out = np.frombuffer(m, dtype=np.uint8, count=nbytes, offset=start)
        if self.poison:
            out[...] = 0xFF      # NaN in fp32 and bf16: a read of anything not written shows
        return out

    def array(self, shape, dtype) -> np.ndarray:
        dt = np.dtype(dtype)
        n = int(np.prod(shape)) if len(shape) else 1
        return self.bytes(n * dt.itemsize).view(dt)[:n].reshape(shape)

    def like(self, a: np.ndarray) -> np.ndarray:
        out = self.array(a.shape, a.dtype)
        out[...] = a
        return out


def addr(a: np.ndarray) -> int:
    return a.ctypes.data
