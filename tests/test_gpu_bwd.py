"""Backward pass on the GPU (gdn_frame_scan_bwd) against the fp64 oracle's
scan_bwd on the same seeded inputs and loss gradients.

Tolerances, per gradient tensor (dq, dk, dv, dbeta, dalpha, dS0), relative
Frobenius error ||err|| / ||ref||: the forward pass's bars, 5e-3 for bf16 I/O
and 1e-5 for fp32 I/O.  For bf16 the error budget is the bf16 rounding of the
outputs dq, dk, dv (about 1.1e-3 relative rms) plus the error the recomputed
states carry from the forward pass (about 2e-3 at the largest shapes,
dominated by the bf16 operands of U), which reaches every gradient through
X_f and S_f; every matrix operand of the backward products (S_f, X_f and
M + M^T) enters as a high and a low bf16 part, so the products add no more.
Measured worst cases: 2.7e-3 (dalpha) in bf16 and 8e-7 in fp32.
Cases span several 64-token blocks with ragged tails, every supported D, both
directions, gate logits, unnormalised keys, a zero key (the eps branch of the
key normalisation), no tokens, one frame, more than one launch chunk and
every unit of the full-minute workload.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_scan_amd import api, inputs

pytestmark = pytest.mark.gpu

TOL_BF16_REL = 5e-3
TOL_F32_REL = 1e-5
NAMES = ("dq", "dk", "dv", "dbeta", "dalpha", "dS0")


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    n = np.linalg.norm(ref)
    d = np.linalg.norm(got - ref)
    return float(d / n) if n > 0 else float(d)


def dev(x, dt=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(dt).contiguous()


def run_bwd(w, dO, dS, *, logits=False, raw_keys=False, reverse=False, beta=None, alpha=None, k=None,
            return_dS0=True):
    q, kk, v, b, a, s0 = inputs.to_torch(w, "cuda")
    io = q.dtype
    if k is not None:
        kk = dev(k, io)
    if beta is not None:
        b = dev(beta)
    if alpha is not None:
        a = dev(alpha)
    grads = api.frame_scan_bwd(q, kk, v, b, a, dev(dO, io), s0, None if dS is None else dev(dS),
                               gates_are_logits=logits, normalize_keys=not raw_keys, reverse=reverse,
                               return_dS0=return_dS0)
    torch.cuda.synchronize()
    return [None if g is None else g.float().cpu().numpy() for g in grads]


def ref_bwd(w, dO, dS, *, logits=False, raw_keys=False, reverse=False, beta=None, alpha=None, k=None):
    return oracle.scan_bwd(w.q, w.k if k is None else k, w.v, w.beta if beta is None else beta,
                           w.alpha if alpha is None else alpha, w.S0, dO, dS, gates_are_logits=logits,
                           normalize_keys=not raw_keys, reverse=reverse)


def compare(got, ref, dtype, tag=""):
    tol = TOL_BF16_REL if dtype == "bf16" else TOL_F32_REL
    bad = []
    for name, g, r in zip(NAMES, got, ref):
        if g is None:
            continue
        e = rel_err(g, r)
        print("%s %s: rel %.3e" % (tag, name, e))
        if not (e <= tol):
            bad.append((name, e))
    assert not bad, (tag, bad)


def logit_gates(w, seed):
    rng = np.random.default_rng((seed, 2))
    bl = rng.standard_normal(w.beta.shape).astype(np.float32)
    al = (rng.standard_normal(w.alpha.shape) + 3.0).astype(np.float32)
    return bl, al


SMALL = [
    # (B, H, F, N, D, dtype, s0_std): ragged tails past 64-token blocks, every D
    (1, 2, 5, 100, 128, "bf16", 0.1),
    (2, 2, 4, 70, 64, "bf16", 0.1),
    (1, 3, 6, 130, 32, "bf16", 0.0),
    (2, 1, 7, 300, 16, "bf16", 0.1),
    (1, 2, 3, 40, 128, "f32", 0.1),
    (1, 2, 4, 33, 64, "f32", 0.0),
    (1, 2, 5, 20, 32, "f32", 0.1),
    (1, 2, 8, 12, 16, "f32", 0.1),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dH%dF%dN%dD%d_%s" % s[:6])
@pytest.mark.parametrize("mode", ["plain", "logits", "raw", "reverse"])
def test_small(shape, mode):
    B, H, F, N, D, dtype, s0 = shape
    w = inputs.make(B, H, F, N, D, dtype=dtype, seed=3, s0_std=s0, normalise_k=(mode != "raw"))
    if mode == "raw":          # unnormalised keys need small betas to stay contractive
        w.beta = (w.beta / D).astype(np.float32)
    dO, dS = inputs.make_grads(w, seed=3)
    kw = {}
    if mode == "logits":
        bl, al = logit_gates(w, 3)
        kw = dict(logits=True, beta=bl, alpha=al)
    elif mode == "raw":
        kw = dict(raw_keys=True)
    elif mode == "reverse":
        kw = dict(reverse=True)
    got = run_bwd(w, dO, dS, **kw)
    ref = ref_bwd(w, dO, dS, **kw)
    compare(got, ref, dtype, "%s %s" % (shape, mode))


def test_zero_key_uses_eps_branch():
    w = inputs.make(1, 2, 3, 50, 64, dtype="bf16", seed=5, s0_std=0.1)
    k = w.k.copy()
    k[0, 1, 7, 1, :] = 0.0                 # one key of norm 0 <= eps
    dO, dS = inputs.make_grads(w, seed=5)
    got = run_bwd(w, dO, dS, k=k)
    ref = ref_bwd(w, dO, dS, k=k)
    compare(got, ref, "bf16", "zero key")


def test_unnormalised_keys_not_unit():
    # keys used as given with norms far from one: the normalisation branch must be off
    w = inputs.make(1, 2, 4, 64, 32, dtype="f32", seed=6, normalise_k=False)
    w.beta = (w.beta / 32).astype(np.float32)
    dO, dS = inputs.make_grads(w, seed=6)
    compare(run_bwd(w, dO, dS, raw_keys=True), ref_bwd(w, dO, dS, raw_keys=True), "f32", "raw")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_more_than_one_chunk(dtype):
    # 300 frames: two launch chunks of at most 256 frames, the state entering
    # the second chunk and the gradient leaving it carried between launches
    w = inputs.make(1, 2, 300, 5, 16, dtype=dtype, seed=7, s0_std=0.1)
    dO, dS = inputs.make_grads(w, seed=7)
    for rev in (False, True):
        compare(run_bwd(w, dO, dS, reverse=rev), ref_bwd(w, dO, dS, reverse=rev), dtype,
                "chunks reverse=%s" % rev)


def test_one_frame_and_no_dS_final():
    w = inputs.make(2, 2, 1, 90, 64, dtype="bf16", seed=8, s0_std=0.1)
    dO, _ = inputs.make_grads(w, seed=8)
    compare(run_bwd(w, dO, None), ref_bwd(w, dO, None), "bf16", "F1")


def test_no_tokens():
    # N = 0: S_f = alpha_f S_{f-1}; only dalpha and dS0 are nonzero
    w = inputs.make(1, 2, 4, 0, 32, dtype="f32", seed=9, s0_std=0.1)
    dO, dS = inputs.make_grads(w, seed=9)
    got = run_bwd(w, dO, dS)
    ref = ref_bwd(w, dO, dS)
    compare(got, ref, "f32", "N0")


def test_no_frames_copies_dS_final():
    w = inputs.make(1, 2, 0, 10, 16, dtype="f32", seed=10, s0_std=0.1)
    dO, dS = inputs.make_grads(w, seed=10)
    got = run_bwd(w, dO, dS)
    np.testing.assert_array_equal(got[5], dS)


def test_dS0_not_requested():
    w = inputs.make(1, 2, 3, 40, 32, dtype="bf16", seed=11, s0_std=0.1)
    dO, dS = inputs.make_grads(w, seed=11)
    got = run_bwd(w, dO, dS, return_dS0=False)
    assert got[5] is None
    compare(got, ref_bwd(w, dO, dS), "bf16", "no dS0")


def test_bitwise_reproducible():
    w = inputs.make(1, 4, 6, 200, 128, dtype="bf16", seed=12, s0_std=0.1)
    dO, dS = inputs.make_grads(w, seed=12)
    a = run_bwd(w, dO, dS)
    b = run_bwd(w, dO, dS)
    for name, x, y in zip(NAMES, a, b):
        assert np.array_equal(x, y), name


def test_full_minute_every_unit():
    """The full-minute workload (B1 H16 F121 N880 d128 bf16) in one launch, every
    gradient of every (b, h) unit against the oracle (each unit must meet the
    bar on its own, so that a wrong unit mapping cannot hide in a whole-tensor
    norm)."""
    w = inputs.make_config("full_minute", seed=0)
    dO, dS = inputs.make_grads(w, seed=0)
    got = run_bwd(w, dO, dS)
    ref = oracle.scan_bwd(w.q, w.k, w.v, w.beta, w.alpha, None, dO, dS)
    compare(got, ref, "bf16", "full_minute")
    for h in range(w.H):
        sl = (slice(0, 1), slice(None), slice(None), slice(h, h + 1))
        mine = [got[0][sl], got[1][sl], got[2][sl], got[3][sl], got[4][:, :, h:h + 1], got[5][:, h:h + 1]]
        theirs = [ref[0][sl], ref[1][sl], ref[2][sl], ref[3][sl], ref[4][:, :, h:h + 1], ref[5][:, h:h + 1]]
        compare(mine, theirs, "bf16", "full_minute unit h=%d" % h)
