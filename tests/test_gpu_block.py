"""Block projections on the GPU (gdn_block_in_proj, gdn_block_out_proj) against
the fp64 oracle (oracle/block.py) on the same seeded bf16 inputs.

Tolerances.  q, k, v and y are fp32 sums rounded once to bf16, so each element
is within 2^-9 of the exact value relative to itself from the rounding, plus
the fp32 summation error, at most about C * 2^-24 times sum_c |x_c w_c| (C the
contraction length); the bar is 2^-8 |ref| + 2^-24 * C * sum_c |x_c w_c|.  The
logits are fp32 outputs: bar 2^-24 * C * sum_c |x_c w_c| (+ the same bound for
the N-term frame sum of the alpha terms).  The chain in_proj -> scan (gate
logits) -> out_proj is compared as one relative Frobenius error against the
oracle chain: the scan's own bf16 bar, 5e-3, plus one bf16 rounding
(2^-9 / sqrt(3) = 1.1e-3 rms) for each of q, k, v, o and y gives 1e-2.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import block as oblock
from gated_deltanet_scan_amd import api, inputs

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(torch.bfloat16).contiguous()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def abs_in_proj(w):
    """sum_c |x_c w_c| for every output of the input projections."""
    return oblock.block_in_proj(np.abs(w.x), np.abs(w.w_qkv), np.abs(w.w_gate))


def check_bf16(got, ref, absref, K, name):
    bar = 2.0 ** -8 * np.abs(ref) + U32 * K * absref
    err = np.abs(got - ref)
    worst = float(np.max(err - bar)) if err.size else -1.0
    print("%s: max err %.3e, worst margin %.3e" % (name, float(err.max()) if err.size else 0.0, worst))
    assert np.all(err <= bar), name


def check_f32(got, ref, bar, name):
    err = np.abs(got - ref)
    print("%s: max err %.3e (bar min %.3e)" % (name, float(err.max()) if err.size else 0.0,
                                                float(bar.min()) if bar.size else 0.0))
    assert np.all(err <= bar), name


def run_in(w):
    return api.block_in_proj(bf(w.x), bf(w.w_qkv), bf(w.w_gate), H=w.H, D=w.D)


def compare_in(w, got):
    ref = oblock.block_in_proj(w.x, w.w_qkv, w.w_gate)
    absr = abs_in_proj(w)
    C, N = w.C, w.N
    for name, g, r, a in zip(("q", "k", "v"), got[:3], ref[:3], absr[:3]):
        check_bf16(host(g), r, a, C, name)
    check_f32(host(got[3]), ref[3], U32 * C * absr[3] + 1e-30, "beta_logit")
    # each per-token term is within U32*C*sum|x w| and the N-term sum adds N*U32 of the same size
    alpha_bar = U32 * (C + N + 1) * absr[4] + 1e-30
    check_f32(host(got[4]), ref[4], alpha_bar, "alpha_logit")


SHAPES = [
    # (B, F, N, C, H, D): ragged token counts, several column tiles, small and large widths
    (1, 3, 50, 256, 2, 64),
    (2, 2, 37, 128, 4, 32),
    (1, 4, 100, 512, 4, 128),
    (1, 2, 1, 64, 1, 16),
    (2, 5, 23, 2048, 16, 128),
    (1, 2, 130, 200, 24, 16),      # C not a multiple of 128; 48 gate rows (one 64-row slab)
    (1, 2, 65, 72, 40, 8),         # C < 128; 80 gate rows (two slabs)
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dF%dN%dC%dH%dD%d" % s)
def test_in_proj(shape):
    B, F, N, C, H, D = shape
    w = inputs.make_block(B, F, N, C, H, D, seed=1)
    got = run_in(w)
    torch.cuda.synchronize()
    compare_in(w, got)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dF%dN%dC%dH%dD%d" % s)
def test_out_proj(shape):
    B, F, N, C, H, D = shape
    w = inputs.make_block(B, F, N, C, H, D, seed=2)
    rng = np.random.default_rng((2, 4))
    o = inputs.round_bf16(rng.standard_normal((B, F, N, H, D), dtype=np.float32))
    y = api.block_out_proj(bf(o), bf(w.w_out))
    torch.cuda.synchronize()
    ref = oblock.block_out_proj(o, w.w_out)
    check_bf16(host(y), ref, oblock.block_out_proj(np.abs(o), np.abs(w.w_out)), H * D, "y")


def test_no_tokens_and_no_frames():
    w = inputs.make_block(1, 3, 0, 64, 2, 16, seed=3)
    q, k, v, bl, al = run_in(w)
    torch.cuda.synchronize()
    assert q.shape == (1, 3, 0, 2, 16) and bl.shape == (1, 3, 0, 2)
    np.testing.assert_array_equal(host(al), np.zeros((1, 3, 2)))
    w = inputs.make_block(1, 0, 5, 64, 2, 16, seed=3)
    q, k, v, bl, al = run_in(w)
    torch.cuda.synchronize()
    assert q.numel() == 0 and al.numel() == 0


def test_chain_through_the_scan():
    """in_proj -> frame_scan_fwd (gate logits, key normalisation) -> out_proj."""
    B, F, N, C, H, D = 1, 6, 70, 512, 4, 64
    w = inputs.make_block(B, F, N, C, H, D, seed=5)
    q, k, v, bl, al = run_in(w)
    o, _ = api.frame_scan_fwd(q, k, v, bl, al, None, gates_are_logits=True)
    y = api.block_out_proj(o, bf(w.w_out))
    torch.cuda.synchronize()
    rq, rk, rv, rb, ra = oblock.block_in_proj(w.x, w.w_qkv, w.w_gate)
    ro, _ = oracle.scan(rq, rk, rv, rb, ra, None, gates_are_logits=True)
    ry = oblock.block_out_proj(ro, w.w_out)
    e = np.linalg.norm(host(y) - ry) / np.linalg.norm(ry)
    print("chain rel err %.3e" % e)
    assert e <= 1e-2


def test_full_minute_every_element():
    """The full-minute shape (B1 F121 N880, H16 D128) at model width C = 2048:
    one in_proj call and one out_proj call at full size, every output element
    compared with the oracle (in chunks of frames, to bound host memory)."""
    B, F, N, C, H, D = 1, 121, 880, 2048, 16, 128
    w = inputs.make_block(B, F, N, C, H, D, seed=0)
    got = run_in(w)
    rng = np.random.default_rng((0, 4))
    o = inputs.round_bf16(rng.standard_normal((B, F, N, H, D), dtype=np.float32))
    y = api.block_out_proj(bf(o), bf(w.w_out))
    torch.cuda.synchronize()
    for f0 in range(0, F, 11):
        sl = slice(f0, min(F, f0 + 11))
        sub = inputs.BlockWorkload(1, sl.stop - sl.start, N, C, H, D, w.x[:, sl], w.w_qkv, w.w_gate, w.w_out)
        compare_in(sub, [t[:, sl] for t in got])
        ref = oblock.block_out_proj(o[:, sl], w.w_out)
        check_bf16(host(y[:, sl]), ref, oblock.block_out_proj(np.abs(o[:, sl]), np.abs(w.w_out)), H * D, "y")
