"""Pins of the block-projection oracle (oracle/block.py) against values fixed
independently of its code: selection weights that copy known columns, a
closed-form frame mean, brute-force dot products on tiny inputs and
linearity.  A transposed weight, a wrong q/k/v or beta/alpha column block, a
sum instead of a mean or a wrong flattening order of the heads each fails one
of them.
"""
import math

import numpy as np

from oracle import block


def selection_weights(C, H, D):
    """w_qkv copies x columns j*H*D + h*D + e into (j, h, e); w_gate copies
    column 3*H*D + j*H + h into gate (j, h)."""
    w_qkv = np.zeros((3, H, D, C))
    w_gate = np.zeros((2, H, C))
    for j in range(3):
        for h in range(H):
            for e in range(D):
                w_qkv[j, h, e, j * H * D + h * D + e] = 1.0
    for j in range(2):
        for h in range(H):
            w_gate[j, h, 3 * H * D + j * H + h] = 1.0
    return w_qkv, w_gate


def test_selection_weights_copy_columns():
    B, F, N, H, D = 2, 3, 4, 2, 3
    C = 3 * H * D + 2 * H + 1
    rng = np.random.default_rng(0)
    x = rng.standard_normal((B, F, N, C))
    w_qkv, w_gate = selection_weights(C, H, D)
    q, k, v, bl, al = block.block_in_proj(x, w_qkv, w_gate)
    for j, t in enumerate((q, k, v)):
        for h in range(H):
            for e in range(D):
                np.testing.assert_array_equal(t[:, :, :, h, e], x[:, :, :, j * H * D + h * D + e])
    for h in range(H):
        np.testing.assert_array_equal(bl[:, :, :, h], x[:, :, :, 3 * H * D + h])


def test_alpha_is_the_frame_mean_closed_form():
    # the alpha column holds c0 + c1*n for token n: the mean over N tokens is
    # c0 + c1*(N-1)/2; the beta column holds a constant per frame
    B, F, N, H, D = 1, 3, 7, 2, 2
    C = 3 * H * D + 2 * H
    x = np.zeros((B, F, N, C))
    w_qkv, w_gate = selection_weights(C, H, D)
    for f in range(F):
        for h in range(H):
            c0, c1 = 1.5 * f - h, 0.25 * (h + 1)
            x[0, f, :, 3 * H * D + H + h] = c0 + c1 * np.arange(N)
            x[0, f, :, 3 * H * D + h] = 10.0 + f
    _, _, _, bl, al = block.block_in_proj(x, w_qkv, w_gate)
    for f in range(F):
        for h in range(H):
            c0, c1 = 1.5 * f - h, 0.25 * (h + 1)
            assert abs(al[0, f, h] - (c0 + c1 * (N - 1) / 2)) < 1e-12
            assert np.all(bl[0, f, :, h] == 10.0 + f)


def test_brute_force_tiny():
    # every output element as its own dot product, summed exactly with fsum
    B, F, N, C, H, D = 1, 2, 3, 5, 2, 3
    rng = np.random.default_rng(1)
    x = rng.standard_normal((B, F, N, C))
    w_qkv = rng.standard_normal((3, H, D, C))
    w_gate = rng.standard_normal((2, H, C))
    w_out = rng.standard_normal((C, H * D))
    q, k, v, bl, al = block.block_in_proj(x, w_qkv, w_gate)
    outs = (q, k, v)
    for f in range(F):
        for h in range(H):
            terms = []
            for n in range(N):
                for j in range(3):
                    for e in range(D):
                        ref = math.fsum(x[0, f, n, c] * w_qkv[j, h, e, c] for c in range(C))
                        assert abs(outs[j][0, f, n, h, e] - ref) < 1e-12
                ref = math.fsum(x[0, f, n, c] * w_gate[0, h, c] for c in range(C))
                assert abs(bl[0, f, n, h] - ref) < 1e-12
                terms.append(math.fsum(x[0, f, n, c] * w_gate[1, h, c] for c in range(C)))
            assert abs(al[0, f, h] - math.fsum(terms) / N) < 1e-12
    o = rng.standard_normal((B, F, N, H, D))
    y = block.block_out_proj(o, w_out)
    for f in range(F):
        for n in range(N):
            for c in range(C):
                ref = math.fsum(o[0, f, n, h, e] * w_out[c, h * D + e] for h in range(H) for e in range(D))
                assert abs(y[0, f, n, c] - ref) < 1e-12


def test_out_proj_permutation_weights():
    # output c picks entry perm[c] of the flattened (h, e) axis, h major
    B, F, N, H, D = 1, 2, 3, 3, 4
    C = H * D
    perm = np.random.default_rng(2).permutation(H * D)
    w_out = np.zeros((C, H * D))
    w_out[np.arange(C), perm] = 1.0
    o = np.random.default_rng(3).standard_normal((B, F, N, H, D))
    y = block.block_out_proj(o, w_out)
    for c in range(C):
        h, e = divmod(int(perm[c]), D)
        np.testing.assert_array_equal(y[..., c], o[..., h, e])


def test_linearity():
    B, F, N, C, H, D = 2, 2, 5, 8, 2, 4
    rng = np.random.default_rng(4)
    x1, x2 = rng.standard_normal((2, B, F, N, C))
    w_qkv = rng.standard_normal((3, H, D, C))
    w_gate = rng.standard_normal((2, H, C))
    a = 0.75
    mix = block.block_in_proj(a * x1 + x2, w_qkv, w_gate)
    one = block.block_in_proj(x1, w_qkv, w_gate)
    two = block.block_in_proj(x2, w_qkv, w_gate)
    for m, p, r in zip(mix, one, two):
        np.testing.assert_allclose(m, a * p + r, rtol=0, atol=1e-12)


def test_no_tokens():
    H, D, C = 2, 4, 16
    x = np.zeros((1, 3, 0, C))
    q, k, v, bl, al = block.block_in_proj(x, np.ones((3, H, D, C)), np.ones((2, H, C)))
    assert q.shape == (1, 3, 0, H, D) and bl.shape == (1, 3, 0, H)
    np.testing.assert_array_equal(al, np.zeros((1, 3, H)))
