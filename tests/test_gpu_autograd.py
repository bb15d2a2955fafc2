"""The torch.autograd binding (gated_deltanet_scan_amd.autograd.frame_scan):
gradients from loss.backward() equal gdn_frame_scan_bwd's for the same loss
gradients, bit for bit, in both the saved-state and the recomputing form."""
import numpy as np
import pytest
import torch

from gated_deltanet_scan_amd import api, autograd, inputs

pytestmark = pytest.mark.gpu


def leaf(t):
    return t.detach().clone().requires_grad_(True)


@pytest.mark.parametrize("recompute", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 5, 100, 64, "bf16", 0.1), (1, 2, 4, 30, 32, "f32", 0.0),
                                   (2, 2, 300, 5, 16, "bf16", 0.1)], ids=lambda s: "B%dH%dF%dN%dD%d_%s" % s[:6])
def test_autograd_matches_the_backward_call(shape, recompute):
    B, H, F, N, D, dtype, s0 = shape
    w = inputs.make(B, H, F, N, D, dtype=dtype, seed=31, s0_std=s0)
    q, k, v, b, a, S0 = inputs.to_torch(w, "cuda")
    dO_h, dS_h = inputs.make_grads(w, seed=31)
    dO = torch.from_numpy(dO_h).cuda().to(q.dtype)
    dS = torch.from_numpy(dS_h).cuda()
    leaves = [leaf(t) for t in (q, k, v, b, a)] + ([leaf(S0)] if S0 is not None else [None])
    o, S_final = autograd.frame_scan(*leaves, recompute=recompute)
    loss = (o.float() * dO.float()).sum() + (S_final * dS).sum()
    loss.backward()
    ref = api.frame_scan_bwd(q, k, v, b, a, dO, S0, dS, return_dS0=S0 is not None)
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dbeta", "dalpha", "dS0")
    for name, x, r in zip(names, leaves, ref):
        if x is None:
            assert r is None
            continue
        assert torch.equal(x.grad, r), name


def test_output_only_loss():
    w = inputs.make(1, 2, 4, 40, 32, dtype="bf16", seed=32, s0_std=0.1)
    q, k, v, b, a, S0 = inputs.to_torch(w, "cuda")
    leaves = [leaf(t) for t in (q, k, v, b, a, S0)]
    o, _ = autograd.frame_scan(*leaves)
    o.float().sum().backward()
    ones = torch.ones_like(q)
    ref = api.frame_scan_bwd(q, k, v, b, a, ones, S0, None)
    torch.cuda.synchronize()
    for x, r in zip(leaves, ref):
        assert torch.equal(x.grad, r)
