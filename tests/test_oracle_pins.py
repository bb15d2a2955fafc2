"""Pins of the fp64 oracle against facts that do not come from the oracle.

The pages print no worked example of the layer, so the oracle is pinned by
(a) a hand-worked example (tests/golden/worked_2x2.txt), (b) the textbook
token-level gated delta rule, which the frame operator must reduce to at N = 1,
(c) a per-token rank-one route that never forms the Gram matrix, (d) closed
forms (pure decay, exact write-back of orthonormal keys) and (e) invariances
(token permutation, rotation, key scaling, head/batch independence, chaining,
linearity, contraction).  Each is chosen so that a plausible slip in the oracle
(a dropped or sign-flipped correction, decay on the wrong term, output read
from the pre-update state, a transposed state, missing key normalisation, a
wrong gate or layout index) fails at least one of them.
"""
import os

import numpy as np
import pytest

import oracle
from gated_deltanet_scan_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def rel(a, b):
    d = np.linalg.norm(np.asarray(a) - np.asarray(b))
    n = np.linalg.norm(np.asarray(b))
    return d / n if n > 0 else d


def rand_case(B=1, H=2, F=3, N=5, Dk=6, Dv=5, seed=0, s0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, F, N, H, Dk))
    k = rng.standard_normal((B, F, N, H, Dk))
    v = rng.standard_normal((B, F, N, H, Dv))
    beta = rng.uniform(0.05, 0.4, (B, F, N, H)) / N
    alpha = rng.uniform(0.5, 0.99, (B, F, H))
    S0 = rng.standard_normal((B, H, Dv, Dk)) if s0 else None
    return q, k, v, beta, alpha, S0


# ---------------------------------------------------------------- independent routes
def token_rule(q, k, v, beta, alpha, S0, eps=1e-6, normalize=True):
    """Textbook gated delta rule, one token per step (valid when N == 1):
    s <- alpha * (s - beta (s k^) k^T) + beta v k^T ;  o = s q.
    normalize=False takes k^ = k (the keys as given)."""
    B, F, N, H, Dk = q.shape
    assert N == 1
    Dv = v.shape[-1]
    o = np.zeros((B, F, 1, H, Dv))
    Sf = np.zeros((B, H, Dv, Dk))
    for b in range(B):
        for h in range(H):
            s = np.zeros((Dv, Dk)) if S0 is None else S0[b, h].copy()
            for f in range(F):
                kk = k[b, f, 0, h]
                if normalize:
                    kk = kk / max(np.linalg.norm(kk), eps)
                bt, al = beta[b, f, 0, h], alpha[b, f, h]
                s = al * (s - bt * np.outer(s @ kk, kk)) + bt * np.outer(v[b, f, 0, h], kk)
                o[b, f, 0, h] = s @ q[b, f, 0, h]
            Sf[b, h] = s
    return o, Sf


def rank_one_route(q, k, v, beta, alpha, S0, eps=1e-6, normalize=True):
    """Frame update as a sum of per-token rank-one corrections, all read from
    the same frozen state; no Gram matrix is ever formed."""
    B, F, N, H, Dk = q.shape
    Dv = v.shape[-1]
    o = np.zeros((B, F, N, H, Dv))
    Sf = np.zeros((B, H, Dv, Dk))
    for b in range(B):
        for h in range(H):
            s = np.zeros((Dv, Dk)) if S0 is None else S0[b, h].copy()
            for f in range(F):
                corr = np.zeros((Dv, Dk))
                write = np.zeros((Dv, Dk))
                for i in range(N):
                    kk = k[b, f, i, h]
                    if normalize:
                        kk = kk / max(np.linalg.norm(kk), eps)
                    bt = beta[b, f, i, h]
                    corr += bt * np.outer(s @ kk, kk)
                    write += bt * np.outer(v[b, f, i, h], kk)
                s = alpha[b, f, h] * (s - corr) + write
                for i in range(N):
                    o[b, f, i, h] = s @ q[b, f, i, h]
            Sf[b, h] = s
    return o, Sf


def unrolled_route(q, k, v, beta, alpha, S0, eps=1e-6):
    """S_f = S0 prod_{g<=f} A_g + sum_g U_g prod_{g<h<=f} A_h with
    A_g = alpha_g (I - G_g), evaluated as explicit ordered matrix products."""
    B, F, N, H, Dk = q.shape
    Dv = v.shape[-1]
    o = np.zeros((B, F, N, H, Dv))
    Sf = np.zeros((B, H, Dv, Dk))
    for b in range(B):
        for h in range(H):
            A, U = [], []
            for f in range(F):
                kh = k[b, f, :, h]
                kh = kh / np.maximum(np.linalg.norm(kh, axis=1, keepdims=True), eps)
                bt = beta[b, f, :, h]
                G = np.einsum("i,ic,ie->ce", bt, kh, kh)
                A.append(alpha[b, f, h] * (np.eye(Dk) - G))
                U.append(np.einsum("i,ia,ie->ae", bt, v[b, f, :, h], kh))
            s0 = np.zeros((Dv, Dk)) if S0 is None else S0[b, h]
            for f in range(F):
                P = np.eye(Dk)
                for g in range(f + 1):
                    P = P @ A[g]
                s = s0 @ P
                for g in range(f + 1):
                    P = np.eye(Dk)
                    for hh in range(g + 1, f + 1):
                        P = P @ A[hh]
                    s = s + U[g] @ P
                o[b, f, :, h] = q[b, f, :, h] @ s.T
                if f == F - 1:
                    Sf[b, h] = s
    return o, Sf


# ---------------------------------------------------------------- golden example
def _read_golden(path):
    out = {}
    with open(path) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            name, shape, *vals = line.split()
            shape = tuple(int(x) for x in shape.strip("[]").split(","))
            out[name] = np.array([float(x) for x in vals]).reshape(shape)
    return out


def test_golden_worked_2x2():
    g = _read_golden(os.path.join(HERE, "golden", "worked_2x2.txt"))
    # fixture shapes are [F,N,D], [F,N], [F], [D,D]; add B=1 and H=1 axes
    q = g["q"][None, :, :, None, :]
    k = g["k"][None, :, :, None, :]
    v = g["v"][None, :, :, None, :]
    beta = g["beta"][None, :, :, None]
    alpha = g["alpha"][None, :, None]
    S0 = g["S0"][None, None]
    o, S = oracle.scan(q, k, v, beta, alpha, S0)
    np.testing.assert_allclose(o[0, :, :, 0, :], g["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S[0, 0], g["S_final"], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- P1 / route checks
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_token_rule_at_N1(seed):
    q, k, v, beta, alpha, S0 = rand_case(B=2, H=3, F=7, N=1, Dk=5, Dv=4, seed=seed)
    beta = np.random.default_rng(seed + 10).uniform(0.1, 1.5, beta.shape)  # large betas too
    o, S = oracle.scan(q, k, v, beta, alpha, S0)
    o2, S2 = token_rule(q, k, v, beta, alpha, S0)
    assert rel(o, o2) < 1e-12 and rel(S, S2) < 1e-12


@pytest.mark.parametrize("seed", [0, 1])
def test_rank_one_route(seed):
    q, k, v, beta, alpha, S0 = rand_case(B=2, H=2, F=4, N=9, Dk=7, Dv=6, seed=seed)
    o, S = oracle.scan(q, k, v, beta, alpha, S0)
    o2, S2 = rank_one_route(q, k, v, beta, alpha, S0)
    assert rel(o, o2) < 1e-12 and rel(S, S2) < 1e-12


def test_unrolled_product_form():
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=2, F=5, N=6, Dk=5, Dv=4, seed=3)
    o, S = oracle.scan(q, k, v, beta, alpha, S0)
    o2, S2 = unrolled_route(q, k, v, beta, alpha, S0)
    assert rel(o, o2) < 1e-12 and rel(S, S2) < 1e-12


# ---------------------------------------------------------------- keys as given
@pytest.mark.parametrize("seed", [0, 1])
def test_raw_keys_token_rule_and_rank_one(seed):
    """normalize_keys=False: the textbook rule and the rank-one route with the
    raw (non-unit) keys, whose norms here lie well away from 1."""
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=2, F=5, N=1, Dk=5, Dv=4, seed=seed)
    k *= np.random.default_rng(seed + 30).uniform(0.3, 0.6, k.shape[:-1] + (1,))
    o, S = oracle.scan(q, k, v, beta, alpha, S0, normalize_keys=False)
    o2, S2 = token_rule(q, k, v, beta, alpha, S0, normalize=False)
    assert rel(o, o2) < 1e-12 and rel(S, S2) < 1e-12
    o3, S3 = oracle.scan(q, k, v, beta, alpha, S0)
    assert rel(S3, S) > 1e-2                      # the two modes really differ
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=2, F=3, N=6, Dk=5, Dv=4, seed=seed + 5)
    k *= 0.4
    o, S = oracle.scan(q, k, v, beta, alpha, S0, normalize_keys=False)
    o2, S2 = rank_one_route(q, k, v, beta, alpha, S0, normalize=False)
    assert rel(o, o2) < 1e-12 and rel(S, S2) < 1e-12


def test_raw_unit_keys_equal_normalised():
    """With keys of unit norm, using them as given equals normalising them."""
    q, k, v, beta, alpha, S0 = rand_case(B=2, H=2, F=3, N=5, Dk=6, Dv=4, seed=31)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    o, S = oracle.scan(q, k, v, beta, alpha, S0)
    o2, S2 = oracle.scan(q, k, v, beta, alpha, S0, normalize_keys=False)
    assert rel(o2, o) < 1e-14 and rel(S2, S) < 1e-14


# ---------------------------------------------------------------- reverse direction
def test_reverse_is_forward_on_reversed_frames():
    """The reverse scan equals the forward scan of the frames in reverse order
    (outputs reversed back), from the same initial state."""
    q, k, v, beta, alpha, S0 = rand_case(B=2, H=2, F=5, N=4, Dk=5, Dv=4, seed=32)
    o, S = oracle.scan(q, k, v, beta, alpha, S0, reverse=True)
    fl = lambda x: np.ascontiguousarray(x[:, ::-1])
    o2, S2 = oracle.scan(fl(q), fl(k), fl(v), fl(beta), fl(alpha), S0)
    assert rel(o, fl(o2)) < 1e-14 and rel(S, S2) < 1e-14
    o3, S3 = oracle.scan(q, k, v, beta, alpha, S0)
    assert rel(S3, S) > 1e-3                      # the directions really differ


def test_reverse_token_rule_at_N1():
    """At N = 1 the reverse scan is the textbook rule walked from the last frame."""
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=2, F=6, N=1, Dk=4, Dv=3, seed=33)
    o, S = oracle.scan(q, k, v, beta, alpha, S0, reverse=True)
    for b in range(1):
        for h in range(2):
            s = S0[b, h].copy()
            for f in range(5, -1, -1):
                kk = k[b, f, 0, h] / np.linalg.norm(k[b, f, 0, h])
                bt, al = beta[b, f, 0, h], alpha[b, f, h]
                s = al * (s - bt * np.outer(s @ kk, kk)) + bt * np.outer(v[b, f, 0, h], kk)
                np.testing.assert_allclose(o[b, f, 0, h], s @ q[b, f, 0, h], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(S[b, h], s, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- closed forms
def test_pure_decay_closed_form():
    q, k, v, beta, alpha, S0 = rand_case(B=2, H=2, F=6, N=4, Dk=5, Dv=3, seed=4)
    beta = np.zeros_like(beta)
    o, S = oracle.scan(q, k, v, beta, alpha, S0)
    cum = np.cumprod(alpha, axis=1)                     # [B,F,H]
    S_exp = cum[:, -1][:, :, None, None] * S0
    o_exp = np.einsum("bfh,bfnhe,bhae->bfnha", cum, q, S0)
    assert rel(S, S_exp) < 1e-14 and rel(o, o_exp) < 1e-14


def test_invariance_alpha1_beta0():
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=3, F=5, N=3, Dk=4, Dv=4, seed=5)
    o, S = oracle.scan(q, k, v, np.zeros_like(beta), np.ones_like(alpha), S0)
    assert np.array_equal(S, S0)
    np.testing.assert_allclose(o, np.einsum("bfnhe,bhae->bfnha", q, S0), rtol=1e-14, atol=1e-14)


def test_single_unit_key_write():
    Dk = Dv = 8
    rng = np.random.default_rng(6)
    kk = rng.standard_normal(Dk)
    kk /= np.linalg.norm(kk)
    vv = rng.standard_normal(Dv)
    shp = (1, 1, 1, 1)
    o, S = oracle.scan(kk.reshape(shp + (Dk,)), kk.reshape(shp + (Dk,)), vv.reshape(shp + (Dv,)),
                       np.ones(shp), np.ones((1, 1, 1)), None)
    np.testing.assert_allclose(S[0, 0], np.outer(vv, kk), atol=1e-15)
    np.testing.assert_allclose(S[0, 0] @ kk, vv, atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 0, 0], vv, atol=1e-14)   # q = k reads the new value


@pytest.mark.parametrize("seed", [0, 1])
def test_orthonormal_write_back(seed):
    """beta = 1 on orthonormal keys: S_f k_j = v_j for every key of the frame,
    S_f x = alpha S_{f-1} x on the orthogonal complement, and q = k reads v."""
    rng = np.random.default_rng(seed)
    Dk, Dv, N, F = 8, 6, 3, 4
    basis = np.linalg.qr(rng.standard_normal((Dk, Dk)))[0]
    k = np.zeros((1, F, N, 1, Dk))
    scale = rng.uniform(0.5, 3.0, (1, F, N, 1, 1))      # raw key scale: normalised away
    for f in range(F):
        perm = rng.permutation(Dk)[:N]
        k[0, f, :, 0] = basis[:, perm].T * scale[0, f, :, 0]
    v = rng.standard_normal((1, F, N, 1, Dv))
    alpha = rng.uniform(0.3, 0.9, (1, F, 1))
    S0 = rng.standard_normal((1, 1, Dv, Dk))
    beta = np.ones((1, F, N, 1))
    o, _ = oracle.scan(k, k, v, beta, alpha, S0)
    np.testing.assert_allclose(o, scale * v, atol=1e-12)      # q = k reads back (scaled) v
    # state after each frame: run prefixes and check both properties
    prev = S0[0, 0]
    for f in range(F):
        _, S = oracle.scan(k[:, :f + 1], k[:, :f + 1], v[:, :f + 1], beta[:, :f + 1],
                           alpha[:, :f + 1], S0)
        S = S[0, 0]
        kh = k[0, f, :, 0] / np.linalg.norm(k[0, f, :, 0], axis=1, keepdims=True)
        np.testing.assert_allclose(S @ kh.T, v[0, f, :, 0].T, atol=1e-12)
        proj = np.eye(Dk) - kh.T @ kh
        x = proj @ rng.standard_normal(Dk)
        np.testing.assert_allclose(S @ x, alpha[0, f, 0] * (prev @ x), atol=1e-12)
        prev = S


# ---------------------------------------------------------------- invariances
def test_token_permutation_within_frame():
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=2, F=3, N=7, Dk=5, Dv=4, seed=7)
    o, S = oracle.scan(q, k, v, beta, alpha, S0)
    perm = np.random.default_rng(8).permutation(7)
    o2, S2 = oracle.scan(q[:, :, perm], k[:, :, perm], v[:, :, perm], beta[:, :, perm], alpha, S0)
    assert rel(S2, S) < 1e-14
    assert rel(o2, o[:, :, perm]) < 1e-14


def test_chaining_split_and_steps():
    q, k, v, beta, alpha, S0 = rand_case(B=2, H=2, F=6, N=4, Dk=5, Dv=5, seed=9)
    o, S = oracle.scan(q, k, v, beta, alpha, S0)
    m = 2
    oa, Sa = oracle.scan(q[:, :m], k[:, :m], v[:, :m], beta[:, :m], alpha[:, :m], S0)
    ob, Sb = oracle.scan(q[:, m:], k[:, m:], v[:, m:], beta[:, m:], alpha[:, m:], Sa)
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o) and np.array_equal(Sb, S)
    s = S0
    for f in range(6):
        of, s = oracle.scan(q[:, f:f + 1], k[:, f:f + 1], v[:, f:f + 1], beta[:, f:f + 1],
                            alpha[:, f:f + 1], s)
        assert np.array_equal(of[:, 0], o[:, f])
    assert np.array_equal(s, S)


def test_linearity_in_values_and_state():
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=2, F=4, N=5, Dk=4, Dv=3, seed=10)
    _, _, v2, _, _, S02 = rand_case(B=1, H=2, F=4, N=5, Dk=4, Dv=3, seed=11)
    c = -1.7
    o1, S1 = oracle.scan(q, k, v, beta, alpha, S0)
    o2, S2 = oracle.scan(q, k, v2, beta, alpha, S02)
    o3, S3 = oracle.scan(q, k, v + c * v2, beta, alpha, S0 + c * S02)
    assert rel(o3, o1 + c * o2) < 1e-13 and rel(S3, S1 + c * S2) < 1e-13


def test_contraction_without_values():
    rng = np.random.default_rng(12)
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=1, F=8, N=6, Dk=5, Dv=4, seed=12)
    beta = rng.uniform(0, 2.0 / 6, beta.shape)      # sum of betas per frame <= 2
    v = np.zeros_like(v)
    prev = S0
    for f in range(8):
        _, s = oracle.scan(q[:, f:f + 1], k[:, f:f + 1], v[:, f:f + 1], beta[:, f:f + 1],
                           alpha[:, f:f + 1], prev)
        assert np.linalg.norm(s) <= alpha[0, f, 0] * np.linalg.norm(prev) * (1 + 1e-12)
        prev = s


def test_rotation_equivariance():
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=2, F=3, N=5, Dk=6, Dv=4, seed=13)
    R = np.linalg.qr(np.random.default_rng(14).standard_normal((6, 6)))[0]
    o, S = oracle.scan(q, k, v, beta, alpha, S0)
    o2, S2 = oracle.scan(q @ R, k @ R, v, beta, alpha, S0 @ R)
    assert rel(S2, S @ R) < 1e-13 and rel(o2, o) < 1e-13


def test_key_scale_invariance():
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=2, F=3, N=5, Dk=6, Dv=4, seed=15)
    c = np.random.default_rng(16).uniform(0.01, 100.0, k.shape[:-1] + (1,))
    o, S = oracle.scan(q, k, v, beta, alpha, S0)
    o2, S2 = oracle.scan(q, k * c, v, beta, alpha, S0)
    assert rel(S2, S) < 1e-13 and rel(o2, o) < 1e-13


def test_heads_and_batches_independent():
    """Fill every (b, h) with its own distribution and check that the joint
    run equals one run per (b, h): pins the [B,F,N,H,D] / [B,F,H] layouts."""
    B, H = 2, 3
    q, k, v, beta, alpha, S0 = rand_case(B=B, H=H, F=3, N=4, Dk=4, Dv=3, seed=17)
    for b in range(B):
        for h in range(H):
            v[b, :, :, h] += 10 * b + h
            q[b, :, :, h] *= 1 + h
            beta[b, :, :, h] *= 1 + 0.5 * b
    o, S = oracle.scan(q, k, v, beta, alpha, S0)
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(None), slice(None), slice(h, h + 1))
            ob, Sb = oracle.scan(q[sl], k[sl], v[sl], beta[sl], alpha[b:b + 1, :, h:h + 1],
                                 S0[b:b + 1, h:h + 1])
            assert np.array_equal(ob[0, :, :, 0], o[b, :, :, h])
            assert np.array_equal(Sb[0, 0], S[b, h])


# ---------------------------------------------------------------- gates, eps, empty
def test_logit_gates():
    q, k, v, _, _, S0 = rand_case(B=1, H=2, F=3, N=4, Dk=4, Dv=4, seed=18)
    rng = np.random.default_rng(19)
    bl = rng.standard_normal((1, 3, 4, 2))
    al = rng.standard_normal((1, 3, 2)) + 3
    o, S = oracle.scan(q, k, v, bl, al, S0, gates_are_logits=True)
    sig = lambda x: 1 / (1 + np.exp(-x))
    o2, S2 = oracle.scan(q, k, v, sig(bl) / 4, sig(al), S0)
    assert rel(o, o2) < 1e-15 and rel(S, S2) < 1e-15


def test_zero_key_contributes_nothing():
    q, k, v, beta, alpha, S0 = rand_case(B=1, H=1, F=2, N=5, Dk=4, Dv=4, seed=20)
    k[0, 1, 2, 0] = 0.0
    o, S = oracle.scan(q, k, v, beta, alpha, S0)
    keep = [0, 1, 3, 4]
    # dropping the token from frame 1 must give the same state
    _, Sa = oracle.scan(q[:, :1], k[:, :1], v[:, :1], beta[:, :1], alpha[:, :1], S0)
    _, Sb = oracle.scan(q[:, 1:, keep], k[:, 1:, keep], v[:, 1:, keep], beta[:, 1:, keep],
                        alpha[:, 1:], Sa)
    assert rel(S, Sb) < 1e-14


def test_empty_tokens_and_frames():
    rng = np.random.default_rng(21)
    B, H, F, D = 1, 2, 3, 4
    S0 = rng.standard_normal((B, H, D, D))
    alpha = rng.uniform(0.5, 1.0, (B, F, H))
    z = np.zeros((B, F, 0, H, D))
    o, S = oracle.scan(z, z, z, np.zeros((B, F, 0, H)), alpha, S0)
    assert o.shape == (B, F, 0, H, D)
    np.testing.assert_allclose(S, np.prod(alpha, axis=1)[:, :, None, None] * S0, rtol=1e-15)
    z0 = np.zeros((B, 0, 5, H, D))
    o, S = oracle.scan(z0, z0, z0, np.zeros((B, 0, 5, H)), np.zeros((B, 0, H)), S0)
    assert np.array_equal(S, S0) and o.shape == (B, 0, 5, H, D)


def test_threads_do_not_change_bits():
    """Thread count must not change a single bit (checked in a subprocess)."""
    import subprocess
    import sys
    code = (
        "import numpy as np, sys; sys.path.insert(0, %r); import oracle;"
        "from tests.test_oracle_pins import rand_case;"
        "a = rand_case(B=1, H=2, F=3, N=33, Dk=24, Dv=20, seed=22);"
        "o, S = oracle.scan(*a); sys.stdout.write(o.tobytes().hex()[:4000] + S.tobytes().hex())"
    ) % os.path.dirname(HERE)
    outs = []
    for nt in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=nt)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, check=True,
                                   capture_output=True, text=True, cwd=os.path.dirname(HERE)).stdout)
    assert outs[0] == outs[1] and len(outs[0]) > 100


# ---------------------------------------------------------------- the synthetic recipe
def test_bf16_inputs_are_exact_for_oracle():
    w = inputs.make(1, 2, 2, 16, 32, dtype="bf16", seed=0)
    import torch
    for x in (w.q, w.k, w.v):
        t = torch.from_numpy(x)
        assert torch.equal(t.to(torch.bfloat16).to(torch.float32), t)
