"""Closed forms checked directly on the GPU (fp32 I/O), without the oracle."""
import numpy as np
import pytest
import torch

from gated_deltanet_scan_amd import api

pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def rel(a, b):
    return np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b)


@pytest.mark.parametrize("D", [16, 64, 128])
def test_pure_decay(D):
    rng = np.random.default_rng(D)
    B, H, F, N = 2, 3, 5, 37
    q = rng.standard_normal((B, F, N, H, D)).astype(np.float32)
    k = rng.standard_normal((B, F, N, H, D)).astype(np.float32)
    v = rng.standard_normal((B, F, N, H, D)).astype(np.float32)
    alpha = rng.uniform(0.5, 1.0, (B, F, H)).astype(np.float32)
    S0 = rng.standard_normal((B, H, D, D)).astype(np.float32)
    o, S = api.frame_scan_fwd(dev(q), dev(k), dev(v), torch.zeros((B, F, N, H), device="cuda"),
                              dev(alpha), dev(S0))
    cum = np.cumprod(alpha.astype(np.float64), axis=1)
    assert rel(S.cpu().numpy(), cum[:, -1][:, :, None, None] * S0) < 1e-6
    o_exp = np.einsum("bfh,bfnhe,bhae->bfnha", cum, q.astype(np.float64), S0.astype(np.float64))
    assert rel(o.cpu().numpy(), o_exp) < 1e-6


def test_state_invariance_alpha1_beta0():
    rng = np.random.default_rng(1)
    B, H, F, N, D = 1, 2, 4, 20, 64
    q, k, v = (rng.standard_normal((B, F, N, H, D)).astype(np.float32) for _ in range(3))
    S0 = rng.standard_normal((B, H, D, D)).astype(np.float32)
    o, S = api.frame_scan_fwd(dev(q), dev(k), dev(v), torch.zeros((B, F, N, H), device="cuda"),
                              torch.ones((B, F, H), device="cuda"), dev(S0))
    assert np.array_equal(S.cpu().numpy(), S0)
    assert rel(o.cpu().numpy(), np.einsum("bfnhe,bhae->bfnha", q, S0.astype(np.float64))) < 1e-6


@pytest.mark.parametrize("D", [32, 128])
def test_orthonormal_write_back(D):
    """beta = 1 on orthonormal keys: the state maps each key of the frame to its
    value, so reading with q = k returns v (times the raw key scale)."""
    rng = np.random.default_rng(2 + D)
    B, H, F, N = 1, 2, 3, 16
    k = np.zeros((B, F, N, H, D))
    scale = rng.uniform(0.5, 2.0, (B, F, N, H, 1))
    for f in range(F):
        for h in range(H):
            basis = np.linalg.qr(rng.standard_normal((D, D)))[0]
            k[0, f, :, h] = basis[:, :N].T * scale[0, f, :, h]
    v = rng.standard_normal((B, F, N, H, D))
    alpha = rng.uniform(0.3, 0.9, (B, F, H))
    S0 = rng.standard_normal((B, H, D, D))
    o, S = api.frame_scan_fwd(dev(k), dev(k), dev(v), torch.ones((B, F, N, H), device="cuda"),
                              dev(alpha), dev(S0))
    got = o.cpu().numpy().astype(np.float64)
    exp = (scale * v).astype(np.float32).astype(np.float64)
    assert rel(got, exp) < 1e-5
