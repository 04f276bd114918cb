"""The seeded synthetic inputs, on the host: the recipe (seed k - 1 for set k,
each Muon tensor's gradient drawn before its parameter, state at zero, norm
weights at one, values drawn in fp32 and cast with round-to-nearest-even) and
the determinism both sides of the parity tests rely on."""
import pytest
import torch

import workloads


def test_seeds_follow_the_set_number():
    assert [workloads.workload(k).seed for k in range(1, 6)] == [0, 1, 2, 3, 4]


def test_first_draws_follow_the_recipe():
    wl = workloads.workload(1)
    t = wl.muon[0]
    gen = torch.Generator(device="cpu")
    gen.manual_seed(wl.seed)
    g = torch.randn(t.shape, generator=gen, dtype=torch.float32) * t.grad_std
    w = torch.randn(t.shape, generator=gen, dtype=torch.float32) * t.param_std
    d = workloads.generate(wl, device="cpu")
    assert torch.equal(d.muon[0].grad, g.to(d.muon[0].grad.dtype))
    assert torch.equal(d.muon[0].param, w.to(d.muon[0].param.dtype))
    assert not d.muon[0].momentum.any()


def test_generation_is_deterministic_and_independent_of_the_kept_subset():
    wl = workloads.workload(2)
    a = workloads.generate(wl, device="cpu", only=[0, 3])
    b = workloads.generate(wl, device="cpu", only=[3])
    assert a.muon[1] is None and b.muon[0] is None
    assert torch.equal(a.muon[3].grad, b.muon[3].grad) and torch.equal(a.muon[3].param, b.muon[3].param)
    for t, spec in zip(a.adamw, wl.adamw):
        if spec.init == "ones":
            assert bool((t.param == 1).all())
        assert not t.m.any() and not t.v.any()


@pytest.mark.parametrize("dtype", ["bf16"])
def test_storage_cast_is_round_to_nearest_even(dtype):
    x = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=torch.float32)
    got = x.to(workloads.TORCH_DTYPE[dtype]).view(torch.int16).tolist()
    assert [v & 0xFFFF for v in got] == [0x3F80, 0x3F82, 0xBF80]
