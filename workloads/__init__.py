"""Seeded synthetic workloads for the hybrid Muon + AdamW step.

This module is the one thing the CPU oracle and the HIP path share: it defines
the parameter sets (shapes, storage dtypes, hyperparameters, value
distributions) and draws their seeded random values. It holds none of the
optimizer's arithmetic: no momentum, no Newton-Schulz, no AdamW. Its only
numeric work is drawing normals/uniforms and casting them to the storage dtype.

Draw recipe (one torch.Generator per workload, seeded with ``workload.seed``,
on ``gen_device``): tensors are visited in list order, Muon tensors first, then
AdamW tensors. For each tensor: the gradient is ``randn(shape) * grad_std``;
if ``outlier_frac > 0`` a ``rand(shape)`` draw follows and entries with
``u < outlier_frac`` are multiplied by ``outlier_scale``; then the parameter is
``randn(shape) * param_std`` (or ones for norm weights). Values are drawn in
float32 and cast to the storage dtype with torch's round-to-nearest-even.
Optimizer state (momentum, NorMuon second moment, Adam moments) starts at zero.

Sources of the parameter sets: the Muon/AdamW routing rule of the speedtronic
"v2 optimizers" page ("Hybrid routing" section), the matrix views of packed
gate/up tensors from the "Optimization" chapter of the kimi-k3 pages ("A tensor's
storage shape can be misleading" section), and the expert batch axis of the
dew.training.optim page (``BATCH_AXES``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import torch

NS_COEFFS = (3.4445, -4.7750, 2.0315)


@dataclass(frozen=True)
class MuonTensorSpec:
    """One parameter stepped by Muon: ``batch x rows x cols``, row-major.

    ``rows`` is the output dimension and ``cols`` the input dimension (PyTorch
    layout). ``views`` splits the rows into equal, independent matrices.
    """
    name: str
    batch: int
    rows: int
    cols: int
    views: int = 1
    param_dtype: str = "f32"
    grad_dtype: str = "f32"
    lr: float = 0.02
    wd: float = 0.1
    param_std: float = 0.02
    grad_std: float = 1e-3
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    has_grad: bool = True

    @property
    def shape(self) -> Tuple[int, int, int]:
        return (self.batch, self.rows, self.cols)

    @property
    def numel(self) -> int:
        return self.batch * self.rows * self.cols

    def matrices(self) -> List[Tuple[int, int, int, int]]:
        """(batch index, view index, m, n) of every matrix this tensor holds."""
        m = self.rows // self.views
        return [(b, v, m, self.cols) for b in range(self.batch) for v in range(self.views)]


@dataclass(frozen=True)
class AdamWTensorSpec:
    name: str
    shape: Tuple[int, ...]
    param_dtype: str = "f32"
    grad_dtype: str = "f32"
    lr: float = 3e-4
    wd: float = 0.1
    init: str = "normal"          # "normal" or "ones"
    param_std: float = 0.02
    grad_std: float = 1e-3

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


@dataclass(frozen=True)
class MuonHParams:
    beta: float = 0.95
    nesterov: bool = True
    ns_steps: int = 5
    ns_coeffs: Tuple[float, float, float] = NS_COEFFS
    ns_eps: float = 1e-7
    ns_dtype: str = "bf16"
    normuon: bool = False
    normuon_beta2: float = 0.95
    muon_plus: bool = False
    muon_plus_eps: float = 1e-8
    cautious: str = "none"        # "none", "wd_mask" (flaxchat form), "wrapper" (speedtronic form)


@dataclass(frozen=True)
class AdamWHParams:
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    step: int = 1


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    muon: Tuple[MuonTensorSpec, ...]
    adamw: Tuple[AdamWTensorSpec, ...] = ()
    muon_hp: MuonHParams = field(default_factory=MuonHParams)
    adamw_hp: AdamWHParams = field(default_factory=AdamWHParams)
    gen_device: str = "cpu"       # where values are drawn by default

    def matrices(self):
        """(tensor index, batch index, view index, m, n) over all Muon matrices."""
        out = []
        for i, t in enumerate(self.muon):
            if not t.has_grad:
                continue
            for (b, v, m, n) in t.matrices():
                out.append((i, b, v, m, n))
        return out


# ---------------------------------------------------------------------------
# The five parameter sets
# ---------------------------------------------------------------------------

def single_256x128() -> Workload:
    """One fp32 256x128 (tall) matrix, fp32 Newton-Schulz, seed 0."""
    t = MuonTensorSpec("w", 1, 256, 128, param_dtype="f32", grad_dtype="f32",
                       lr=0.02, wd=0.1, param_std=0.02, grad_std=1.0)
    return Workload("single_256x128_f32", 0, (t,), (), MuonHParams(ns_dtype="f32"))


def gpt_12l_d768() -> Workload:
    """GPT-style 12 layers, d=768: Q,K,V,O 768x768, MLP up 3072x768, down 768x3072
    (72 Muon matrices, fp32 storage, bf16 Newton-Schulz) + AdamW on the tied
    50304x768 embedding/head and 25 RMSNorm weights of 768."""
    mu = []
    for layer in range(12):
        for nm in ("q", "k", "v", "o"):
            mu.append(MuonTensorSpec(f"h{layer}.attn.{nm}", 1, 768, 768))
        mu.append(MuonTensorSpec(f"h{layer}.mlp.up", 1, 3072, 768))
        mu.append(MuonTensorSpec(f"h{layer}.mlp.down", 1, 768, 3072))
    ad = [AdamWTensorSpec("wte", (50304, 768), wd=0.1)]
    for i in range(25):
        ad.append(AdamWTensorSpec(f"norm{i}", (768,), wd=0.0, init="ones"))
    return Workload("gpt_12L_d768", 1, tuple(mu), tuple(ad),
                    MuonHParams(ns_dtype="bf16"), AdamWHParams(0.9, 0.95, 1e-8, 1))


def llama_8l_d4096() -> Workload:
    """Llama-style 8 layers, d=4096 GQA: q,o 4096x4096, k,v 1024x4096, packed
    gate_up 28672x4096 viewed as 2 x (14336x4096), down 4096x14336; bf16
    params and grads, fp32 momentum; 1% gradient outliers x100."""
    mu = []
    kw = dict(param_dtype="bf16", grad_dtype="bf16", grad_std=1e-3,
              outlier_frac=0.01, outlier_scale=100.0)
    for layer in range(8):
        mu.append(MuonTensorSpec(f"l{layer}.q", 1, 4096, 4096, **kw))
        mu.append(MuonTensorSpec(f"l{layer}.k", 1, 1024, 4096, **kw))
        mu.append(MuonTensorSpec(f"l{layer}.v", 1, 1024, 4096, **kw))
        mu.append(MuonTensorSpec(f"l{layer}.o", 1, 4096, 4096, **kw))
        mu.append(MuonTensorSpec(f"l{layer}.gate_up", 1, 28672, 4096, views=2, **kw))
        mu.append(MuonTensorSpec(f"l{layer}.down", 1, 4096, 14336, **kw))
    return Workload("llama_8L_d4096", 2, tuple(mu), (), MuonHParams(ns_dtype="bf16"),
                    gen_device="cuda")


def moe_64x2048() -> Workload:
    """MoE layer: 64 experts, d=2048, ffn=1408; gate_up [64, 2816, 2048] viewed as
    2 x (1408x2048), down [64, 2048, 1408] (192 matrices); NorMuon row second
    moment and the cautious weight-decay mask; router 64x2048 on AdamW."""
    mu = (MuonTensorSpec("experts.gate_up", 64, 2816, 2048, views=2),
          MuonTensorSpec("experts.down", 64, 2048, 1408))
    ad = (AdamWTensorSpec("router", (64, 2048), wd=0.1),)
    hp = MuonHParams(ns_dtype="bf16", normuon=True, normuon_beta2=0.95, cautious="wd_mask")
    return Workload("moe_64x2048", 3, mu, ad, hp, AdamWHParams(0.9, 0.95, 1e-8, 1),
                    gen_device="cuda")


def wide_4l_d8192() -> Workload:
    """4 layers d=8192: attention 8192x8192 x4, MLP up 28672x8192, down
    8192x28672, bf16; Muon+ row_col (eps 1e-8) and the cautious wrapper."""
    mu = []
    kw = dict(param_dtype="bf16", grad_dtype="bf16", param_std=0.01, grad_std=1e-4)
    for layer in range(4):
        for nm in ("q", "k", "v", "o"):
            mu.append(MuonTensorSpec(f"l{layer}.{nm}", 1, 8192, 8192, **kw))
        mu.append(MuonTensorSpec(f"l{layer}.up", 1, 28672, 8192, **kw))
        mu.append(MuonTensorSpec(f"l{layer}.down", 1, 8192, 28672, **kw))
    hp = MuonHParams(ns_dtype="bf16", muon_plus=True, muon_plus_eps=1e-8, cautious="wrapper")
    return Workload("wide_4L_d8192", 4, tuple(mu), (), hp, gen_device="cuda")


WORKLOADS = {
    1: single_256x128,
    2: gpt_12l_d768,
    3: llama_8l_d4096,
    4: moe_64x2048,
    5: wide_4l_d8192,
}


def workload(k: int) -> Workload:
    return WORKLOADS[k]()


# ---------------------------------------------------------------------------
# Value generation
# ---------------------------------------------------------------------------

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class MuonTensorData:
    spec: MuonTensorSpec
    param: torch.Tensor
    grad: Optional[torch.Tensor]
    momentum: torch.Tensor
    row_v: Optional[torch.Tensor]


@dataclass
class AdamWTensorData:
    spec: AdamWTensorSpec
    param: torch.Tensor
    grad: torch.Tensor
    m: torch.Tensor
    v: torch.Tensor


@dataclass
class WorkloadData:
    workload: Workload
    muon: List[MuonTensorData]
    adamw: List[AdamWTensorData]


def _draw_grad(gen, shape, std, frac, scale, dev):
    g = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std
    if frac > 0:
        u = torch.rand(shape, generator=gen, device=dev, dtype=torch.float32)
        g = torch.where(u < frac, g * scale, g)
    return g


def generate(wl: Workload, device: str = "cpu", gen_device: Optional[str] = None,
             only: Optional[Sequence[int]] = None) -> WorkloadData:
    """Draw the workload's tensors on ``gen_device`` and move them to ``device``.

    ``only`` restricts which Muon tensors are kept (all are still drawn in
    order, so the values do not depend on ``only``).
    """
    gdev = gen_device or wl.gen_device
    if gdev == "cuda" and not torch.cuda.is_available():
        gdev = "cpu"
    gen = torch.Generator(device=gdev)
    gen.manual_seed(wl.seed)
    hp = wl.muon_hp
    muon = []
    for i, t in enumerate(wl.muon):
        g = _draw_grad(gen, t.shape, t.grad_std, t.outlier_frac, t.outlier_scale, gdev)
        w = torch.randn(t.shape, generator=gen, device=gdev, dtype=torch.float32) * t.param_std
        if only is not None and i not in only:
            del g, w
            muon.append(None)
            continue
        p = w.to(TORCH_DTYPE[t.param_dtype]).to(device)
        del w
        gr = g.to(TORCH_DTYPE[t.grad_dtype]).to(device) if t.has_grad else None
        del g
        mom = torch.zeros(t.shape, dtype=torch.float32, device=device)
        rv = (torch.zeros((t.batch, t.rows), dtype=torch.float32, device=device)
              if hp.normuon else None)
        muon.append(MuonTensorData(t, p, gr, mom, rv))
    adamw = []
    for t in wl.adamw:
        g = _draw_grad(gen, t.shape, t.grad_std, 0.0, 1.0, gdev)
        if t.init == "ones":
            w = torch.ones(t.shape, device=gdev, dtype=torch.float32)
        else:
            w = torch.randn(t.shape, generator=gen, device=gdev, dtype=torch.float32) * t.param_std
        p = w.to(TORCH_DTYPE[t.param_dtype]).to(device)
        gr = g.to(TORCH_DTYPE[t.grad_dtype]).to(device)
        adamw.append(AdamWTensorData(t, p, gr,
                                     torch.zeros(t.shape, dtype=torch.float32, device=device),
                                     torch.zeros(t.shape, dtype=torch.float32, device=device)))
    return WorkloadData(wl, muon, adamw)


def to_numpy(t: torch.Tensor):
    """Host copy of a tensor's stored values: float32 arrays as float32, bfloat16
    arrays as their raw uint16 bit patterns (the oracle decodes them itself)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16").copy()
    return t.numpy().copy()
