"""Pins of the fp64 backward oracle (oracle.scan_bwd) against facts that do not
come from its own derivation:

(a) central finite differences of the forward oracle: for a random linear loss
    L = <dO, O> + <dS_F, S_F>, dL/dx must match the difference quotient for
    every input x (q, k, v, beta, alpha, S0), in the default mode, with logit
    gates, with keys used as given, in the reverse direction and at a zero key;
(b) reverse-mode automatic differentiation (torch, float64, CPU) of a plain
    restatement of the forward definition written here with tensor ops.
"""
import numpy as np
import pytest
import torch

import oracle
from test_oracle_pins import rand_case

FIELDS = ("q", "k", "v", "beta", "alpha", "S0")


def loss(args, dO, dS, **kw):
    o, S = oracle.scan(*args, **kw)
    return float((o * dO).sum() + (S * dS).sum())


def fd_check(args, kw, seed, n_idx=5, h=1e-6, tol=2e-6):
    rng = np.random.default_rng(seed)
    o, S = oracle.scan(*args, **kw)
    dO = rng.standard_normal(o.shape)
    dS = rng.standard_normal(S.shape)
    grads = oracle.scan_bwd(*args, dO, dS, **kw)
    for name, x, g in zip(FIELDS, args, grads):
        flat = x.reshape(-1)
        for idx in rng.choice(flat.size, size=min(n_idx, flat.size), replace=False):
            old = flat[idx]
            flat[idx] = old + h
            lp = loss(args, dO, dS, **kw)
            flat[idx] = old - h
            lm = loss(args, dO, dS, **kw)
            flat[idx] = old
            num = (lp - lm) / (2 * h)
            ana = g.reshape(-1)[idx]
            assert abs(num - ana) <= tol * max(1.0, abs(num)), (name, idx, num, ana)


@pytest.mark.parametrize("seed", [0, 1])
def test_finite_differences_default(seed):
    args = list(rand_case(B=1, H=2, F=3, N=4, Dk=5, Dv=4, seed=40 + seed))
    fd_check(args, {}, seed)


def test_finite_differences_logit_gates():
    q, k, v, _, _, S0 = rand_case(B=1, H=2, F=3, N=4, Dk=5, Dv=4, seed=42)
    rng = np.random.default_rng(43)
    bl = rng.standard_normal((1, 3, 4, 2))
    al = rng.standard_normal((1, 3, 2)) + 2.0
    fd_check([q, k, v, bl, al, S0], {"gates_are_logits": True}, 43)


def test_finite_differences_raw_keys_and_reverse():
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=2, F=3, N=4, Dk=5, Dv=4, seed=44)
    k *= 0.4
    fd_check([q, k, v, beta, alpha, S0], {"normalize_keys": False}, 44)
    q, k, v, beta, alpha, S0 = rand_case(B=2, H=1, F=4, N=3, Dk=4, Dv=5, seed=45)
    fd_check([q, k, v, beta, alpha, S0], {"reverse": True}, 45)


def test_finite_differences_at_a_zero_key():
    """A zero key is scaled by 1/eps (the clamp), so its gradient is dk^/eps;
    steps below eps stay on that branch."""
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=1, F=2, N=3, Dk=4, Dv=3, seed=46)
    k[0, 1, 2, 0] = 0.0
    args = [q, k, v, beta, alpha, S0]
    rng = np.random.default_rng(47)
    o, S = oracle.scan(*args)
    dO, dS = rng.standard_normal(o.shape), rng.standard_normal(S.shape)
    dk = oracle.scan_bwd(*args, dO, dS)[1]
    h = 1e-8
    for c in range(4):
        k[0, 1, 2, 0, c] = h
        lp = loss(args, dO, dS)
        k[0, 1, 2, 0, c] = -h
        lm = loss(args, dO, dS)
        k[0, 1, 2, 0, c] = 0.0
        num = (lp - lm) / (2 * h)
        assert abs(num - dk[0, 1, 2, 0, c]) <= 1e-5 * max(1.0, abs(num))


def torch_forward(q, k, v, beta, alpha, S0, eps=1e-6, logits=False):
    """The forward definition restated with tensor operations (frame loop,
    Gram and U products as einsums); independent of the C oracle."""
    B, F, N, H, Dk = q.shape
    Dv = v.shape[-1]
    if logits:
        beta = torch.sigmoid(beta) / N
        alpha = torch.sigmoid(alpha)
    kh = k / torch.clamp(torch.linalg.norm(k, dim=-1, keepdim=True), min=eps)
    S = S0.clone()
    outs = []
    for f in range(F):
        G = torch.einsum("bnh,bnhc,bnhe->bhce", beta[:, f], kh[:, f], kh[:, f])
        U = torch.einsum("bnh,bnha,bnhe->bhae", beta[:, f], v[:, f], kh[:, f])
        eye = torch.eye(Dk, dtype=q.dtype)
        S = alpha[:, f, :, None, None] * (S @ (eye - G)) + U
        outs.append(torch.einsum("bhae,bnhe->bnha", S, q[:, f]))
    return torch.stack(outs, dim=1), S


@pytest.mark.parametrize("logits", [False, True])
def test_matches_autograd_of_a_tensor_restatement(logits):
    args = list(rand_case(B=2, H=2, F=4, N=5, Dk=6, Dv=4, seed=48))
    if logits:
        rng = np.random.default_rng(49)
        args[3] = rng.standard_normal(args[3].shape)
        args[4] = rng.standard_normal(args[4].shape) + 2.0
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in args]
    o, S = torch_forward(*ts, logits=logits)
    rng = np.random.default_rng(50)
    dO = rng.standard_normal(o.shape)
    dS = rng.standard_normal(S.shape)
    ((o * torch.tensor(dO)).sum() + (S * torch.tensor(dS)).sum()).backward()
    grads = oracle.scan_bwd(*args, dO, dS, gates_are_logits=logits)
    for name, t, g in zip(FIELDS, ts, grads):
        ref = t.grad.numpy()
        err = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
        assert err < 1e-12, (name, err)


def test_zero_output_gradient_gives_zero():
    args = list(rand_case(B=1, H=2, F=3, N=4, Dk=5, Dv=4, seed=51))
    o, S = oracle.scan(*args)
    grads = oracle.scan_bwd(*args, np.zeros_like(o), np.zeros_like(S))
    assert all(np.all(g == 0) for g in grads)
