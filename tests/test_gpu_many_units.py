"""Scans with many (b, h) units: more recurrence workgroups (one per 16-row
slab of a state) than the GPU has CUs, so the slabs of several heads share
each XCD, and the Gram and output passes walk many items per workgroup.

Against the oracle in both directions, bf16 and fp32, the forward and the
backward (whose adjoint recurrence is the same kernel); and bit for bit
across unit counts: heads 0..15 of a B1 H17 d128 scan equal a B1 H16 d128
scan of the same heads, since each unit's arithmetic does not depend on how
many units share the launch.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_scan_amd import api, inputs
from test_gpu_bwd import compare, ref_bwd, run_bwd
from test_gpu_parity import check, check_every_unit, oracle_ref

pytestmark = pytest.mark.gpu


def run(w, **kw):
    q, k, v, b, a, s0 = inputs.to_torch(w, "cuda")
    o, S = api.frame_scan_fwd(q, k, v, b, a, s0, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy()


FWD = [  # B, H, F, N, D, dtype, reverse; every one has more than 128 slab workgroups
    (2, 12, 4, 40, 128, "bf16", False),
    (2, 12, 3, 70, 128, "bf16", True),
    (3, 30, 3, 30, 64, "bf16", False),
    (1, 70, 3, 20, 32, "bf16", True),
    (1, 20, 3, 24, 128, "f32", False),
    (2, 36, 2, 17, 64, "f32", True),
]


@pytest.mark.parametrize("shape", FWD, ids=lambda s: "B%dH%dF%dN%dD%d_%s_%s" % (s[:6] + ("rev" if s[6] else "fwd",)))
def test_forward_against_oracle(shape):
    B, H, F, N, D, dtype, reverse = shape
    assert B * H * D // 16 > 128
    w = inputs.make(B, H, F, N, D, dtype=dtype, seed=81, s0_std=0.05)
    o, S = run(w, reverse=reverse)
    ro, rS = oracle_ref(w, reverse=reverse)
    check(o, ro, dtype, "O")
    check(S, rS, dtype, "S_F")


@pytest.mark.parametrize("shape", [(2, 12, 3, 40, 128, "bf16"), (2, 40, 3, 20, 64, "bf16"), (1, 80, 2, 12, 32, "f32")],
                         ids=lambda s: "B%dH%dF%dN%dD%d_%s" % s)
@pytest.mark.parametrize("reverse", [False, True])
def test_backward_against_oracle(shape, reverse):
    B, H, F, N, D, dtype = shape
    w = inputs.make(B, H, F, N, D, dtype=dtype, seed=82, s0_std=0.05)
    dO, dS = inputs.make_grads(w, seed=82)
    got = run_bwd(w, dO, dS, reverse=reverse)
    ref = ref_bwd(w, dO, dS, reverse=reverse)
    compare(got, ref, dtype, "B%dH%dD%d" % (B, H, D))


def test_units_do_not_depend_on_the_unit_count():
    w17 = inputs.make(1, 17, 5, 100, 128, dtype="bf16", seed=83, s0_std=0.05)
    sl = lambda x: np.ascontiguousarray(x[..., :16, :]) if x.ndim == 5 else x
    w16 = inputs.make(1, 16, 5, 100, 128, dtype="bf16", seed=83, s0_std=0.05)
    w16.q, w16.k, w16.v = sl(w17.q), sl(w17.k), sl(w17.v)
    w16.beta = np.ascontiguousarray(w17.beta[..., :16])
    w16.alpha = np.ascontiguousarray(w17.alpha[..., :16])
    w16.S0 = np.ascontiguousarray(w17.S0[:, :16])
    o17, S17 = run(w17)
    o16, S16 = run(w16)
    assert np.array_equal(o17[..., :16, :], o16) and np.array_equal(S17[:, :16], S16)
    ro, rS = oracle_ref(w17)
    check(o17, ro, "bf16", "O H17")
    check(S17, rS, "bf16", "S_F H17")


@pytest.mark.slow
@pytest.mark.parametrize("D", [128, 64])
def test_many_units_of_whole_frames(D):
    """128 (b, h) units of 880-token frames (B4 H32 F16): several recurrence
    workgroups share each CU.  The workspace starts as all-ones bytes (NaN in
    bf16, so any value read before it is written shows), and every unit must
    meet the tolerances.  At this shape the state planes once came back with
    one or two corrupted values per call: a buffer store's data registers were
    rewritten by the next instruction (now padded; see store_b128)."""
    w = inputs.make(4, 32, 16, 880, D, dtype="bf16", seed=84, s0_std=0.02)
    q, k, v, b, a, s0 = inputs.to_torch(w, "cuda")
    desc = api.make_desc(w.B, w.H, w.F, w.N, w.Dk, q.dtype)
    ws = api.alloc_workspace(desc, q.device)
    for rep in range(2):
        ws.fill_(255)
        o, S = api.frame_scan_fwd(q, k, v, b, a, s0, workspace=ws)
        torch.cuda.synchronize()
        o, S = o.float().cpu().numpy(), S.cpu().numpy()
        if rep == 0:
            ro, rS = oracle_ref(w)
        check_every_unit(w, o, S, ro, rS)


@pytest.mark.parametrize("N", [127, 128])
def test_both_sides_of_the_intermediate_precision_threshold(N):
    """d 64 with 127 tokens per frame keeps U in fp32 and the state planes with
    remainder codes; with 128 the forward scan hands both on in bf16.  Both
    meet the oracle's tolerance, in both directions."""
    w = inputs.make(2, 3, 6, N, 64, dtype="bf16", seed=85, s0_std=0.05)
    for reverse in (False, True):
        o, S = run(w, reverse=reverse)
        ro, rS = oracle_ref(w, reverse=reverse)
        check(o, ro, "bf16", "O N%d" % N)
        check(S, rS, "bf16", "S_F N%d" % N)


def test_bf16_intermediates_with_every_option():
    """The bf16-intermediate regime (d 64, 150 tokens per frame) with gate
    logits (beta = sigmoid / N summing to ~0.6 per frame), 300 frames (two
    launch chunks, the state carried between them) and the state updated in
    place, forward and reverse, against the oracle."""
    w = inputs.make(1, 4, 300, 150, 64, dtype="bf16", seed=86, s0_std=0.05)
    rng = np.random.default_rng(87)
    beta_logit = rng.standard_normal(w.beta.shape).astype(np.float32) + 0.6
    alpha_logit = (rng.standard_normal(w.alpha.shape) + 3.0).astype(np.float32)
    q, k, v, _, _, s0 = inputs.to_torch(w, "cuda")
    b = torch.from_numpy(beta_logit).cuda()
    a = torch.from_numpy(alpha_logit).cuda()
    for reverse in (False, True):
        carry = s0.clone()
        o, S = api.frame_scan_fwd(q, k, v, b, a, carry, S_final=carry, gates_are_logits=True, reverse=reverse)
        torch.cuda.synchronize()
        assert S.data_ptr() == carry.data_ptr()
        ro, rS = oracle_ref(w, logits=True, beta=beta_logit, alpha=alpha_logit, reverse=reverse)
        check(o.float().cpu().numpy(), ro, "bf16", "O rev=%d" % reverse)
        check(S.cpu().numpy(), rS, "bf16", "S_F rev=%d" % reverse)
