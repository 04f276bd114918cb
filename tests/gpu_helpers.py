"""Glue shared by the GPU parity tests: run the HIP path through the binding,
feed the same stored inputs to the oracle, compare."""
import numpy as np
import torch

import muon_adamw_amd as ma
import workloads
from oracle import storage


def rel(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    d = np.linalg.norm(x - y)
    n = np.linalg.norm(y)
    return d / n if n > 0 else d


def host(t):
    """Stored values of a tensor as float64 (bf16 decoded by the oracle's rule)."""
    a = workloads.to_numpy(t)
    return storage.decode(a, "bf16" if t.dtype == torch.bfloat16 else "f32")


def hp_c(h: workloads.MuonHParams):
    return ma.muon_hparams(h.beta, h.nesterov, h.ns_steps, h.ns_coeffs, h.ns_eps, h.ns_dtype, h.normuon,
                           h.normuon_beta2, h.muon_plus, h.muon_plus_eps, h.cautious)


def hp_dict(h: workloads.MuonHParams):
    return {"beta": h.beta, "nesterov": h.nesterov, "ns_steps": h.ns_steps, "ns_coeffs": h.ns_coeffs,
            "ns_eps": h.ns_eps, "normuon": h.normuon, "normuon_beta2": h.normuon_beta2,
            "muon_plus": h.muon_plus, "muon_plus_eps": h.muon_plus_eps, "cautious": h.cautious}


def muon_params(data: workloads.WorkloadData):
    return [ma.MuonParam(t.param, t.grad, t.momentum, t.row_v, t.spec.views, t.spec.lr, t.spec.wd)
            for t in data.muon if t is not None]


def adamw_params(data: workloads.WorkloadData):
    return [ma.AdamWParam(t.param, t.grad, t.m, t.v, t.spec.lr, t.spec.wd) for t in data.adamw]


def snapshot(t):
    return None if t is None else t.detach().clone()


def to_gpu(data: workloads.WorkloadData, device="cuda"):
    for t in data.muon:
        if t is None:
            continue
        t.param = t.param.to(device)
        t.grad = None if t.grad is None else t.grad.to(device)
        t.momentum = t.momentum.to(device)
        t.row_v = None if t.row_v is None else t.row_v.to(device)
    for t in data.adamw:
        t.param, t.grad, t.m, t.v = (x.to(device) for x in (t.param, t.grad, t.m, t.v))
    return data


def flush(msg):
    print(msg, flush=True)
