"""Python binding of libmuon_adamw.so, the MI355X hybrid Muon + AdamW step.

Argument marshalling only: torch tensors are turned into the C descriptors of
``include/muon_adamw.h`` (device pointers, shapes, dtypes) and the current HIP
stream; every step of the update runs in the library's HIP kernels. There is
no fallback: if the library is missing or a tensor is unsupported, the call
raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuon_adamw.so")

MA_F32, MA_BF16 = 0, 1
CAUTIOUS = {"none": 0, "wd_mask": 1, "wrapper": 2}
STATUS = {0: "MA_OK", 1: "MA_E_INVALID", 2: "MA_E_DTYPE", 3: "MA_E_ALIAS", 4: "MA_E_WORKSPACE",
          5: "MA_E_UNSUPPORTED", 6: "MA_E_HIP"}
NS_COEFFS = (3.4445, -4.7750, 2.0315)


class MuonTensorC(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("momentum", ctypes.c_void_p), ("row_v", ctypes.c_void_p),
                ("batch", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("views", ctypes.c_int32), ("param_dtype", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32), ("lr", ctypes.c_float),
                ("weight_decay", ctypes.c_float)]


class MuonHParamsC(ctypes.Structure):
    _fields_ = [("beta", ctypes.c_double), ("normuon_beta2", ctypes.c_double),
                ("ns_a", ctypes.c_float), ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float),
                ("ns_eps", ctypes.c_float), ("muon_plus_eps", ctypes.c_float),
                ("nesterov", ctypes.c_int32), ("ns_steps", ctypes.c_int32),
                ("ns_dtype", ctypes.c_int32), ("normuon", ctypes.c_int32),
                ("muon_plus", ctypes.c_int32), ("cautious", ctypes.c_int32),
                ("pad_", ctypes.c_int32), ("ns_table", ctypes.POINTER(ctypes.c_float)),
                ("clip", ctypes.c_void_p), ("ns_norm_scale", ctypes.c_float), ("pad2_", ctypes.c_int32)]


class AdamWTensorC(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("numel", ctypes.c_int64), ("param_dtype", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32), ("lr", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("moment_dtype", ctypes.c_int32), ("pad_", ctypes.c_int32)]


class AdamWHParamsC(ctypes.Structure):
    _fields_ = [("beta1", ctypes.c_double), ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("step", ctypes.c_int64), ("cautious", ctypes.c_int32), ("pad_", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("clip", ctypes.c_void_p)]


class GradRefC(ctypes.Structure):
    _fields_ = [("grad", ctypes.c_void_p), ("numel", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("pad_", ctypes.c_int32)]


class MatrixInfoC(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int32), ("batch_index", ctypes.c_int32),
                ("view", ctypes.c_int32), ("m", ctypes.c_int32), ("n", ctypes.c_int32),
                ("r", ctypes.c_int32), ("c", ctypes.c_int32), ("rp", ctypes.c_int32),
                ("cp", ctypes.c_int32), ("transposed", ctypes.c_int32),
                ("bucket", ctypes.c_int32), ("scale", ctypes.c_float), ("pad_", ctypes.c_int32),
                ("u_offset", ctypes.c_uint64), ("a_offset", ctypes.c_uint64), ("b_offset", ctypes.c_uint64)]


class KernelTimeC(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


EXPORTS = ("muon_step", "adamw_step", "ma_muon_workspace_bytes", "ma_last_error",
           "ma_newton_schulz", "ma_newton_schulz_workspace_bytes", "ma_muon_plan_counts",
           "ma_muon_matrix_info", "ma_profile_begin", "ma_profile_end", "ma_grad_norm_workspace_bytes",
           "ma_global_grad_norm", "ma_muon_step_status", "ma_muon_queue_info", "ma_mfma_bf16_ceiling")
# bits of ma_muon_step_status
NS_WAIT_TIMEOUT, NS_QUEUE_UNDRAINED = 1, 2

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the built library (``python -m muon_adamw_amd.build`` makes it)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m muon_adamw_amd.build`")
    _lib = declare(ctypes.CDLL(path))
    return _lib


def declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Sets the argument and result types of every function the header declares."""
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.muon_step.argtypes = [ctypes.POINTER(MuonTensorC), I32, ctypes.POINTER(MuonHParamsC), P, SZ, P]
    lib.muon_step.restype = ctypes.c_int
    lib.adamw_step.argtypes = [ctypes.POINTER(AdamWTensorC), I32, ctypes.POINTER(AdamWHParamsC), P]
    lib.adamw_step.restype = ctypes.c_int
    lib.ma_muon_workspace_bytes.argtypes = [ctypes.POINTER(MuonTensorC), I32, ctypes.POINTER(MuonHParamsC)]
    lib.ma_muon_workspace_bytes.restype = SZ
    lib.ma_last_error.argtypes = []
    lib.ma_last_error.restype = ctypes.c_char_p
    lib.ma_newton_schulz.argtypes = [P, P, I64, I64, I64, I32, ctypes.POINTER(MuonHParamsC), P, SZ, P]
    lib.ma_newton_schulz.restype = ctypes.c_int
    lib.ma_newton_schulz_workspace_bytes.argtypes = [I64, I64, I64, I32, ctypes.POINTER(MuonHParamsC)]
    lib.ma_newton_schulz_workspace_bytes.restype = SZ
    lib.ma_muon_plan_counts.argtypes = [ctypes.POINTER(MuonTensorC), I32, ctypes.POINTER(MuonHParamsC),
                                        ctypes.POINTER(I32), ctypes.POINTER(I32)]
    lib.ma_muon_plan_counts.restype = ctypes.c_int
    lib.ma_muon_matrix_info.argtypes = [ctypes.POINTER(MuonTensorC), I32, ctypes.POINTER(MuonHParamsC),
                                        I32, ctypes.POINTER(MatrixInfoC)]
    lib.ma_muon_matrix_info.restype = ctypes.c_int
    lib.ma_profile_begin.argtypes = []
    lib.ma_profile_begin.restype = ctypes.c_int
    lib.ma_profile_end.argtypes = [ctypes.POINTER(KernelTimeC), I32]
    lib.ma_profile_end.restype = I32
    lib.ma_grad_norm_workspace_bytes.argtypes = [ctypes.POINTER(GradRefC), I32]
    lib.ma_grad_norm_workspace_bytes.restype = SZ
    lib.ma_global_grad_norm.argtypes = [ctypes.POINTER(GradRefC), I32, ctypes.c_float, P, P, SZ, P]
    lib.ma_global_grad_norm.restype = ctypes.c_int
    lib.ma_muon_step_status.argtypes = [P, ctypes.POINTER(I32), P]
    lib.ma_muon_step_status.restype = ctypes.c_int
    lib.ma_muon_queue_info.argtypes = [ctypes.POINTER(MuonTensorC), I32, ctypes.POINTER(MuonHParamsC),
                                       ctypes.POINTER(I32), ctypes.POINTER(I32), I32]
    lib.ma_muon_queue_info.restype = ctypes.c_int
    lib.ma_mfma_bf16_ceiling.argtypes = [P, I32, I32, P]
    lib.ma_mfma_bf16_ceiling.restype = ctypes.c_int
    return lib


class MuonAdamWError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(status: int):
    if status != 0:
        raise MuonAdamWError(status, load_library().ma_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MA_F32
    if t.dtype == torch.bfloat16:
        return MA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 and bfloat16 only; complex is rejected)")


def _check_dense(t: torch.Tensor, what: str):
    if t.layout != torch.strided:
        raise TypeError(f"{what}: sparse tensors are not supported (layout {t.layout})")
    if t.is_complex():
        raise TypeError(f"{what}: complex tensors are not supported")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")


def _check_device(t: torch.Tensor, device, what: str):
    """Every pointer of a call must be memory of the one GPU the kernels run
    on: a host or other-device tensor would be dereferenced by the GPU."""
    if t.device != device:
        raise ValueError(f"{what} must be on {device} (got {t.device})")


def _check_clip_state(clip, what: str = "clip"):
    """A clip state is the tensor global_grad_norm returned (or a raw device
    address, passed through unchecked for callers that manage their own)."""
    if clip is None or isinstance(clip, int):
        return
    if not isinstance(clip, torch.Tensor):
        raise TypeError(f"{what} must be the state tensor global_grad_norm returned or a device address")
    if not clip.is_cuda or clip.dtype != torch.float32 or clip.numel() < 4 or not clip.is_contiguous():
        raise ValueError(f"{what} must be a contiguous float32 GPU tensor of 4 entries")


def _stream_handle(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


@dataclass
class MuonParam:
    """One Muon parameter: ``param`` is (rows, cols) or (batch, rows, cols)."""
    param: torch.Tensor
    grad: Optional[torch.Tensor]
    momentum: torch.Tensor
    row_v: Optional[torch.Tensor] = None
    views: int = 1
    lr: float = 0.02
    weight_decay: float = 0.1


@dataclass
class AdamWParam:
    param: torch.Tensor
    grad: Optional[torch.Tensor]
    m: torch.Tensor
    v: torch.Tensor
    lr: float = 3e-4
    weight_decay: float = 0.1


def _ptr(t) -> Optional[int]:
    return None if t is None else (t if isinstance(t, int) else t.data_ptr())


def muon_hparams(beta=0.95, nesterov=True, ns_steps=5, ns_coeffs=NS_COEFFS, ns_eps=1e-7,
                 ns_dtype="bf16", normuon=False, normuon_beta2=0.95, muon_plus=False,
                 muon_plus_eps=1e-8, cautious="none", ns_table=None, ns_norm_scale=1.0,
                 clip=None) -> MuonHParamsC:
    """``ns_table``: one (a, b, c) per iteration (ns_steps rows), or None.
    ``clip``: the device state tensor global_grad_norm wrote, or None."""
    _check_clip_state(clip)
    a, b, c = ns_coeffs
    h = MuonHParamsC()
    h.beta, h.normuon_beta2 = beta, normuon_beta2
    h.ns_a, h.ns_b, h.ns_c, h.ns_eps, h.muon_plus_eps = a, b, c, ns_eps, muon_plus_eps
    h.nesterov, h.ns_steps = int(bool(nesterov)), int(ns_steps)
    h.ns_dtype = MA_BF16 if ns_dtype == "bf16" else MA_F32
    h.normuon, h.muon_plus, h.cautious = int(bool(normuon)), int(bool(muon_plus)), CAUTIOUS[cautious]
    if ns_table is not None:
        rows = [tuple(r) for r in ns_table]
        if len(rows) != ns_steps or any(len(r) != 3 for r in rows):
            raise ValueError("ns_table needs one (a, b, c) row per Newton-Schulz step")
        arr = (ctypes.c_float * (3 * ns_steps))(*[float(x) for r in rows for x in r])
        h._table = arr   # keeps the host array alive as long as the struct
        h.ns_table = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    h.ns_norm_scale = ns_norm_scale
    h.clip = _ptr(clip)
    return h


def _muon_descs(tensors: Sequence[MuonParam], check_device=True):
    arr = (MuonTensorC * max(len(tensors), 1))()
    device = None
    for i, t in enumerate(tensors):
        p = t.param
        _check_dense(p, f"muon[{i}].param")
        if p.dim() == 2:
            batch, rows, cols = 1, p.shape[0], p.shape[1]
        elif p.dim() == 3:
            batch, rows, cols = p.shape
        else:
            raise ValueError(f"muon[{i}].param must be 2-D or 3-D, got {tuple(p.shape)}")
        if check_device:
            if not p.is_cuda:
                raise ValueError(f"muon[{i}].param must be on a GPU")
            device = device or p.device
            if p.device != device:
                raise ValueError("all tensors of one call must be on one device")
        d = arr[i]
        d.param = p.data_ptr()
        d.param_dtype = _dtype_code(p)
        d.batch, d.rows, d.cols, d.views = batch, rows, cols, t.views
        d.lr, d.weight_decay = t.lr, t.weight_decay
        if t.grad is not None:
            _check_dense(t.grad, f"muon[{i}].grad")
            if t.grad.shape != p.shape:
                raise ValueError(f"muon[{i}].grad must match param's shape")
            if check_device:
                _check_device(t.grad, p.device, f"muon[{i}].grad")
            d.grad = t.grad.data_ptr()
            d.grad_dtype = _dtype_code(t.grad)
        else:
            d.grad = None
            d.grad_dtype = d.param_dtype
        m = t.momentum
        _check_dense(m, f"muon[{i}].momentum")
        if m.dtype != torch.float32 or m.numel() != p.numel():
            raise ValueError(f"muon[{i}].momentum must be float32 with param's numel")
        if check_device:
            _check_device(m, p.device, f"muon[{i}].momentum")
        d.momentum = m.data_ptr()
        if t.row_v is not None:
            _check_dense(t.row_v, f"muon[{i}].row_v")
            if t.row_v.dtype != torch.float32 or t.row_v.numel() != batch * rows:
                raise ValueError(f"muon[{i}].row_v must be float32 with batch*rows entries")
            if check_device:
                _check_device(t.row_v, p.device, f"muon[{i}].row_v")
            d.row_v = t.row_v.data_ptr()
        else:
            d.row_v = None
    return arr, device


def muon_workspace_bytes(tensors: Sequence[MuonParam], hp: MuonHParamsC) -> int:
    lib = load_library()
    arr, _ = _muon_descs(tensors, check_device=False)
    _check(lib.ma_muon_plan_counts(arr, len(tensors), ctypes.byref(hp), None, None))
    return lib.ma_muon_workspace_bytes(arr, len(tensors), ctypes.byref(hp))


def muon_step(tensors: Sequence[MuonParam], hp: MuonHParamsC, workspace: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """The Muon half of the hybrid step, in place. Returns the workspace used
    (it holds the orthogonalised updates until the next call)."""
    lib = load_library()
    arr, device = _muon_descs(tensors)
    _check(lib.ma_muon_plan_counts(arr, len(tensors), ctypes.byref(hp), None, None))
    need = lib.ma_muon_workspace_bytes(arr, len(tensors), ctypes.byref(hp))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device or "cuda")
    elif device is not None:
        _check_device(workspace, device, "workspace")
    _check(lib.muon_step(arr, len(tensors), ctypes.byref(hp), ctypes.c_void_p(workspace.data_ptr()),
                         workspace.numel(), ctypes.c_void_p(_stream_handle(stream, workspace.device))))
    return workspace


def muon_step_status(workspace: torch.Tensor, stream=None) -> int:
    """Device status of the last muon_step / newton_schulz that used
    ``workspace``: 0 when it ran to completion, else NS_WAIT_TIMEOUT and/or
    NS_QUEUE_UNDRAINED (its results are then not to be used). Waits for the
    stream."""
    lib = load_library()
    if not workspace.is_cuda:
        raise ValueError("workspace must be on a GPU")
    st = ctypes.c_int32(-1)
    _check(lib.ma_muon_step_status(ctypes.c_void_p(workspace.data_ptr()), ctypes.byref(st),
                                   ctypes.c_void_p(_stream_handle(stream, workspace.device))))
    return int(st.value)


def adamw_step(tensors: Sequence[AdamWParam], beta1=0.9, beta2=0.95, eps=1e-8, step=1, stream=None,
               cautious=False, seed=0, clip=None):
    """The AdamW half. m and v are float32 or bfloat16 (stochastic rounding,
    seeded by ``seed``, the step, the tensor and the moment); ``cautious``:
    the wrapper mask; ``clip``: the device state global_grad_norm wrote."""
    lib = load_library()
    arr = (AdamWTensorC * max(len(tensors), 1))()
    device = None
    for i, t in enumerate(tensors):
        for nm in ("param", "m", "v"):
            _check_dense(getattr(t, nm), f"adamw[{i}].{nm}")
        if not t.param.is_cuda:
            raise ValueError(f"adamw[{i}].param must be on a GPU")
        device = device or t.param.device
        for nm in ("param", "m", "v"):
            _check_device(getattr(t, nm), device, f"adamw[{i}].{nm}")
        n = t.param.numel()
        if t.m.dtype != t.v.dtype or t.m.numel() != n or t.v.numel() != n:
            raise ValueError(f"adamw[{i}]: m and v must share a dtype and have param's numel")
        d = arr[i]
        d.param, d.m, d.v, d.numel = t.param.data_ptr(), t.m.data_ptr(), t.v.data_ptr(), n
        d.moment_dtype = _dtype_code(t.m)
        d.param_dtype = _dtype_code(t.param)
        if t.grad is not None:
            _check_dense(t.grad, f"adamw[{i}].grad")
            if t.grad.numel() != n:
                raise ValueError(f"adamw[{i}].grad must match param's numel")
            _check_device(t.grad, device, f"adamw[{i}].grad")
            d.grad, d.grad_dtype = t.grad.data_ptr(), _dtype_code(t.grad)
        else:
            d.grad, d.grad_dtype = None, d.param_dtype
        d.lr, d.weight_decay = t.lr, t.weight_decay
    _check_clip_state(clip)
    hp = AdamWHParamsC(beta1, beta2, eps, int(step))
    hp.cautious = CAUTIOUS["wrapper"] if cautious else 0
    hp.seed = int(seed) & ((1 << 64) - 1)
    hp.clip = _ptr(clip)
    _check(lib.adamw_step(arr, len(tensors), ctypes.byref(hp),
                          ctypes.c_void_p(_stream_handle(stream, device or torch.device("cuda")))))


def global_grad_norm(grads: Sequence[Optional[torch.Tensor]], max_norm: float = 0.0,
                     state: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Global gradient norm and clip state over ``grads`` (None entries skip).
    Returns the device state: [norm, clip factor, skip flag, 0]."""
    lib = load_library()
    arr = (GradRefC * max(len(grads), 1))()
    device = None
    for i, g in enumerate(grads):
        if g is None:
            continue
        _check_dense(g, f"grads[{i}]")
        if not g.is_cuda:
            raise ValueError(f"grads[{i}] must be on a GPU")
        device = device or g.device
        _check_device(g, device, f"grads[{i}]")
        arr[i].grad, arr[i].numel, arr[i].dtype = g.data_ptr(), g.numel(), _dtype_code(g)
    # with every gradient absent, the current GPU (with its index, as tensors report it)
    device = device or torch.device("cuda", torch.cuda.current_device())
    if state is None:
        state = torch.empty(4, dtype=torch.float32, device=device)
    else:
        _check_clip_state(state, "state")
        _check_device(state, device, "state")
    need = lib.ma_grad_norm_workspace_bytes(arr, len(grads))
    if need == 0:
        raise MuonAdamWError(1, lib.ma_last_error().decode())
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    _check_device(workspace, device, "workspace")
    _check(lib.ma_global_grad_norm(arr, len(grads), float(max_norm), ctypes.c_void_p(state.data_ptr()),
                                   ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                   ctypes.c_void_p(_stream_handle(stream, device))))
    return state


def newton_schulz(x: torch.Tensor, hp: Optional[MuonHParamsC] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Newton-Schulz alone on a (rows, cols) or (batch, rows, cols) tensor."""
    lib = load_library()
    hp = hp or muon_hparams(ns_dtype="bf16" if x.dtype == torch.bfloat16 else "f32")
    _check_dense(x, "x")
    if not x.is_cuda:
        raise ValueError("x must be on a GPU")
    if x.dim() not in (2, 3):
        raise ValueError(f"x must be 2-D or 3-D, got {tuple(x.shape)}")
    batch, rows, cols = (1, *x.shape) if x.dim() == 2 else tuple(x.shape)
    dt = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_dense(out, "out")
        if out.shape != x.shape or out.dtype != x.dtype:
            raise ValueError("out must have x's shape and dtype")
        _check_device(out, x.device, "out")
    need = lib.ma_newton_schulz_workspace_bytes(batch, rows, cols, dt, ctypes.byref(hp))
    if need == 0:
        raise MuonAdamWError(1, lib.ma_last_error().decode())
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check_device(workspace, x.device, "workspace")
    _check(lib.ma_newton_schulz(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()), batch, rows,
                                cols, dt, ctypes.byref(hp), ctypes.c_void_p(workspace.data_ptr()),
                                workspace.numel(), ctypes.c_void_p(_stream_handle(stream, x.device))))
    return out


def plan_counts(tensors: Sequence[MuonParam], hp: MuonHParamsC):
    lib = load_library()
    arr, _ = _muon_descs(tensors, check_device=False)
    nm, nb = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib.ma_muon_plan_counts(arr, len(tensors), ctypes.byref(hp), ctypes.byref(nm), ctypes.byref(nb)))
    return nm.value, nb.value


def matrix_info(tensors: Sequence[MuonParam], hp: MuonHParamsC, k: int) -> dict:
    lib = load_library()
    arr, _ = _muon_descs(tensors, check_device=False)
    info = MatrixInfoC()
    _check(lib.ma_muon_matrix_info(arr, len(tensors), ctypes.byref(hp), k, ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in MatrixInfoC._fields_ if f != "pad_"}


def queue_info(tensors: Sequence[MuonParam], hp: MuonHParamsC):
    """The persistent launch's task queues: a list of 8 lists (one per XCD)
    of (matrix, iteration * 4 + product, first task, tiles required)."""
    lib = load_library()
    arr, _ = _muon_descs(tensors, check_device=False)
    nseg = (ctypes.c_int32 * 8)()
    _check(lib.ma_muon_queue_info(arr, len(tensors), ctypes.byref(hp), nseg, None, 0))
    total = sum(nseg)
    segs = (ctypes.c_int32 * max(4 * total, 1))()
    _check(lib.ma_muon_queue_info(arr, len(tensors), ctypes.byref(hp), nseg, segs, total))
    out, k = [], 0
    for x in range(8):
        out.append([tuple(segs[4 * (k + i): 4 * (k + i) + 4]) for i in range(nseg[x])])
        k += nseg[x]
    return out


def workspace_u(workspace: torch.Tensor, info: dict, ns_dtype: str) -> torch.Tensor:
    """View of matrix ``info``'s final Newton-Schulz output inside a workspace:
    (rp, cp) canonical orientation, zero outside (r, c)."""
    es = 2 if ns_dtype == "bf16" else 4
    nbytes = info["rp"] * info["cp"] * es
    raw = workspace[info["u_offset"]: info["u_offset"] + nbytes]
    dt = torch.bfloat16 if ns_dtype == "bf16" else torch.float32
    return raw.view(dt).view(info["rp"], info["cp"])


def mfma_bf16_ceiling(sink: torch.Tensor, blocks: int, iters: int, stream=None) -> int:
    """Enqueues the MFMA-only loop (blocks x 4 waves x iters x 8 multiplies of
    32768 flops); ``sink`` is a float32 GPU tensor of at least ``blocks``
    entries. Returns the flop count; the caller times the launch."""
    lib = load_library()
    if not sink.is_cuda or sink.dtype != torch.float32 or sink.numel() < blocks or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous float32 GPU tensor of at least `blocks` entries")
    _check(lib.ma_mfma_bf16_ceiling(ctypes.c_void_p(sink.data_ptr()), int(blocks), int(iters),
                                    ctypes.c_void_p(_stream_handle(stream, sink.device))))
    return blocks * 4 * iters * 8 * 32768


def profile_begin():
    """Start bracketing every library kernel launch with HIP events."""
    _check(load_library().ma_profile_begin())


def profile_end() -> dict:
    """Stop; returns {kernel name: (launches, total ms)} from the events."""
    lib = load_library()
    buf = (KernelTimeC * 64)()
    n = lib.ma_profile_end(buf, 64)
    if n < 0:
        raise MuonAdamWError(6, lib.ma_last_error().decode())
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(n)}
