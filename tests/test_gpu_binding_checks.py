"""The binding refuses, before anything is enqueued, tensors that are not on
the call's GPU or do not fit the call (a host pointer would otherwise be
dereferenced by a kernel). Needs a GPU for the device tensors; no kernel runs."""
import pytest
import torch

import muon_adamw_amd as ma

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_muon_state_on_the_host_is_rejected():
    p = torch.zeros(64, 32, device=DEV)
    g = torch.zeros(64, 32, device=DEV)
    with pytest.raises(ValueError, match="momentum"):
        ma.muon_step([ma.MuonParam(p, g, torch.zeros(64, 32))], ma.muon_hparams())
    with pytest.raises(ValueError, match="grad"):
        ma.muon_step([ma.MuonParam(p, torch.zeros(64, 32), torch.zeros(64, 32, device=DEV))], ma.muon_hparams())
    with pytest.raises(ValueError, match="row_v"):
        ma.muon_step([ma.MuonParam(p, g, torch.zeros(64, 32, device=DEV), torch.zeros(64))],
                     ma.muon_hparams(normuon=True))
    with pytest.raises(ValueError, match="workspace"):
        ma.muon_step([ma.MuonParam(p, g, torch.zeros(64, 32, device=DEV))], ma.muon_hparams(),
                     workspace=torch.zeros(1 << 20, dtype=torch.uint8))


def test_adamw_state_on_the_host_is_rejected():
    p = torch.zeros(100, device=DEV)
    with pytest.raises(ValueError, match=r"adamw\[0\]\.m"):
        ma.adamw_step([ma.AdamWParam(p, torch.zeros(100, device=DEV), torch.zeros(100), torch.zeros(100, device=DEV))])
    with pytest.raises(ValueError, match=r"adamw\[0\]\.grad"):
        ma.adamw_step([ma.AdamWParam(p, torch.zeros(100), torch.zeros(100, device=DEV), torch.zeros(100, device=DEV))])
    with pytest.raises(ValueError, match="clip"):
        ma.adamw_step([ma.AdamWParam(p, None, torch.zeros(100, device=DEV), torch.zeros(100, device=DEV))],
                      clip=torch.zeros(4))


def test_grad_norm_state_and_newton_schulz_out_are_checked():
    g = torch.zeros(100, device=DEV)
    with pytest.raises(ValueError, match="state"):
        ma.global_grad_norm([g], 1.0, state=torch.zeros(4))
    x = torch.zeros(64, 32, device=DEV)
    with pytest.raises(ValueError, match="out"):
        ma.newton_schulz(x, out=torch.zeros(32, 64, device=DEV))
    with pytest.raises(ValueError, match="out"):
        ma.newton_schulz(x, out=torch.zeros(64, 32))
    with pytest.raises(ValueError, match="2-D or 3-D"):
        ma.newton_schulz(torch.zeros(8, device=DEV))
    with pytest.raises(ValueError, match="workspace"):
        ma.newton_schulz(x, workspace=torch.zeros(1 << 24, dtype=torch.uint8))


def test_grad_norm_with_every_gradient_absent():
    """No gradient at all is a valid call: the binding defaults to the current
    GPU, and the state reads norm 0, clip factor 1, no skip."""
    state = ma.global_grad_norm([None, None], 1.0)
    torch.cuda.synchronize()
    assert state.device.type == "cuda"
    assert state.cpu().tolist()[:3] == [0.0, 1.0, 0.0]
