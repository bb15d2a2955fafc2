"""HIP path vs the fp64 oracle on seeded synthetic inputs.

Tolerances: bf16 I/O with fp32 state: max |err| <= 2e-2 and
||err||_F / ||ref||_F <= 5e-3, each on O and on S_final; fp32 I/O:
||err||_F / ||ref||_F <= 1e-5.  The oracle's O is unrounded fp64, so the bf16
rounding of O (about 1.7e-3 relative) is part of the measured error.

Every case, small or full-size, runs the whole tensor through the oracle.  The
full-size workloads run exactly the launch the benchmark times; besides the
whole-tensor errors, every (b, h) unit must meet the tolerances on its own, so
that a wrong mapping of any one unit (the persistent item walk of the Gram
pass, the head rotation of the output pass, the XCD placement of the
recurrence) cannot hide in a whole-tensor norm.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_scan_amd import api, inputs

pytestmark = pytest.mark.gpu

TOL_BF16_MAXABS = 2e-2
TOL_BF16_REL = 5e-3
TOL_F32_REL = 1e-5


def errs(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    n = np.linalg.norm(ref)
    rel = np.linalg.norm(d) / n if n > 0 else np.linalg.norm(d)
    return (float(np.abs(d).max()) if d.size else 0.0), float(rel)


def check(got, ref, dtype, what):
    mx, rel = errs(got, ref)
    print("%s: max|err| %.3e  rel %.3e" % (what, mx, rel))
    if dtype == "bf16":
        assert mx <= TOL_BF16_MAXABS and rel <= TOL_BF16_REL, (what, mx, rel)
    else:
        assert rel <= TOL_F32_REL, (what, mx, rel)


def run_gpu(w, *, logits=False, S0="auto", beta=None, alpha=None, raw_keys=False, reverse=False):
    q, k, v, b, a, s0 = inputs.to_torch(w, "cuda")
    if beta is not None:
        b = torch.from_numpy(np.ascontiguousarray(beta, dtype=np.float32)).cuda()
    if alpha is not None:
        a = torch.from_numpy(np.ascontiguousarray(alpha, dtype=np.float32)).cuda()
    if S0 is not None and not isinstance(S0, str):
        s0 = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda()
    o, S = api.frame_scan_fwd(q, k, v, b, a, s0, gates_are_logits=logits,
                              normalize_keys=not raw_keys, reverse=reverse)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy()


def oracle_ref(w, *, logits=False, units=None, beta=None, alpha=None, S0="auto", raw_keys=False,
               reverse=False):
    beta = w.beta if beta is None else beta
    alpha = w.alpha if alpha is None else alpha
    S0 = w.S0 if isinstance(S0, str) else S0
    if units is None:
        return oracle.scan(w.q, w.k, w.v, beta, alpha, S0, gates_are_logits=logits,
                           normalize_keys=not raw_keys, reverse=reverse)
    outs = []
    for b, h in units:
        sl = (slice(b, b + 1), slice(None), slice(None), slice(h, h + 1))
        s0 = None if S0 is None else S0[b:b + 1, h:h + 1]
        outs.append(oracle.scan(w.q[sl], w.k[sl], w.v[sl], beta[sl], alpha[b:b + 1, :, h:h + 1],
                                s0, gates_are_logits=logits))
    return outs


# ------------------------------------------------------------------ small, whole tensor
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_fp32_config(seed):
    w = inputs.make_config("tiny_fp32", seed=seed)
    o, S = run_gpu(w)
    ro, rS = oracle_ref(w)
    check(o, ro, "f32", "O")
    check(S, rS, "f32", "S_F")


SMALL = [  # B, H, F, N, D, s0_std
    (1, 1, 1, 1, 16, 0.0),
    (2, 3, 3, 17, 16, 0.1),
    (1, 2, 4, 100, 32, 0.1),
    (2, 2, 3, 130, 64, 0.05),      # ragged over one 128-token stage
    (1, 3, 2, 257, 128, 0.02),     # two full stages and a 1-token tail
    (1, 2, 5, 880, 128, 0.02),     # the clip's frame size, 6 full stages + 112
    (3, 5, 2, 48, 64, 0.0),        # odd unit count for the XCD mapping
]


@pytest.mark.parametrize("B,H,F,N,D,s0", SMALL)
def test_bf16_small(B, H, F, N, D, s0):
    w = inputs.make(B, H, F, N, D, dtype="bf16", seed=B * 1000 + N, s0_std=s0)
    o, S = run_gpu(w)
    ro, rS = oracle_ref(w)
    check(o, ro, "bf16", "O")
    check(S, rS, "bf16", "S_F")


@pytest.mark.parametrize("B,H,F,N,D,s0", [
    (1, 2, 3, 13, 16, 0.1), (2, 2, 3, 70, 32, 0.1), (1, 3, 2, 65, 64, 0.05), (1, 2, 3, 200, 128, 0.02)])
def test_fp32_small(B, H, F, N, D, s0):
    w = inputs.make(B, H, F, N, D, dtype="f32", seed=7 + N, s0_std=s0)
    o, S = run_gpu(w)
    ro, rS = oracle_ref(w)
    check(o, ro, "f32", "O")
    check(S, rS, "f32", "S_F")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_logit_gates(dtype):
    w = inputs.make(2, 3, 4, 96, 64, dtype=dtype, seed=31, s0_std=0.05)
    bl, al = w.meta["beta_logit"], w.meta["alpha_logit"]
    o, S = run_gpu(w, logits=True, beta=bl, alpha=al)
    ro, rS = oracle_ref(w, logits=True, beta=bl, alpha=al)
    check(o, ro, dtype, "O")
    check(S, rS, dtype, "S_F")


def test_large_betas_and_unnormalised_keys():
    """Sum of betas per frame near 1.8 (inside the contraction domain) and keys
    of arbitrary norm: exercises the hi/lo state split and the normaliser."""
    w = inputs.make(1, 2, 6, 64, 128, dtype="bf16", seed=41, s0_std=0.1, normalise_k=False)
    beta = np.full_like(w.beta, 1.8 / 64)
    o, S = run_gpu(w, beta=beta)
    ro, rS = oracle_ref(w, beta=beta)
    check(o, ro, "bf16", "O")
    check(S, rS, "bf16", "S_F")


def test_zero_key_contributes_nothing():
    w = inputs.make(1, 2, 3, 40, 64, dtype="bf16", seed=43, s0_std=0.05)
    w.k[0, 1, 7, 1] = 0.0
    w.k[0, 2, 0, 0] = 0.0
    o, S = run_gpu(w)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    ro, rS = oracle_ref(w)
    check(o, ro, "bf16", "O")
    check(S, rS, "bf16", "S_F")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_more_frames_than_one_launch_chunk(dtype):
    """300 frames run as two launch chunks (256 + 44 frames) with the state
    carried between them, also in place (S_final is S0)."""
    w = inputs.make(1, 2, 300, 24, 32, dtype=dtype, seed=47, s0_std=0.05)
    o, S = run_gpu(w)
    ro, rS = oracle_ref(w)
    check(o, ro, dtype, "O")
    check(S, rS, dtype, "S_F")
    q, k, v, b, a, s0 = inputs.to_torch(w, "cuda")
    carry = s0.clone()
    o2, _ = api.frame_scan_fwd(q, k, v, b, a, carry, S_final=carry)
    torch.cuda.synchronize()
    check(o2.float().cpu().numpy(), ro, dtype, "O (in place)")
    check(carry.cpu().numpy(), rS, dtype, "S_F (in place)")


def test_more_units_than_cus():
    """320 (b, h) units: more recurrence and output workgroups than stay
    resident, and (b, h) indices past every XCD round."""
    w = inputs.make(4, 80, 3, 20, 16, dtype="bf16", seed=48, s0_std=0.05)
    o, S = run_gpu(w)
    ro, rS = oracle_ref(w)
    check(o, ro, "bf16", "O")
    check(S, rS, "bf16", "S_F")


def test_empty_token_frames_decay_only():
    w = inputs.make(2, 3, 4, 0, 32, dtype="bf16", seed=44, s0_std=0.1)
    o, S = run_gpu(w)
    assert o.shape == (2, 4, 0, 3, 32)
    exp = np.prod(w.alpha.astype(np.float64), axis=1)[:, :, None, None] * w.S0
    check(S, exp, "f32", "S_F")


def test_empty_scan_copies_state():
    w = inputs.make(2, 3, 0, 5, 32, dtype="bf16", seed=45, s0_std=0.1)
    o, S = run_gpu(w)
    assert np.array_equal(S, w.S0)
    w2 = inputs.make(2, 3, 0, 5, 32, dtype="bf16", seed=45)
    o, S = run_gpu(w2)                       # S0 = None -> zeros
    assert np.array_equal(S, np.zeros_like(S))


def test_in_place_state_and_determinism():
    w = inputs.make(2, 4, 3, 150, 128, dtype="bf16", seed=46, s0_std=0.05)
    q, k, v, b, a, s0 = inputs.to_torch(w, "cuda")
    o1, S1 = api.frame_scan_fwd(q, k, v, b, a, s0)
    o2, S2 = api.frame_scan_fwd(q, k, v, b, a, s0)
    carry = s0.clone()
    o3, S3 = api.frame_scan_fwd(q, k, v, b, a, carry, S_final=carry)   # S_final is S0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert torch.equal(o1, o3) and torch.equal(S1, carry) and S3.data_ptr() == carry.data_ptr()


# ------------------------------------------------------------------ keys as given
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 16), ("f32", 64)])
def test_raw_keys(dtype, D):
    """GDN_FLAG_NO_KEY_NORM: keys of norm 0.3-0.6 used as given."""
    w = inputs.make(2, 3, 4, 150, D, dtype=dtype, seed=51 + D, s0_std=0.05)
    scale = np.random.default_rng(52).uniform(0.3, 0.6, w.k.shape[:-1] + (1,)).astype(np.float32)
    w.k = w.k * scale
    if dtype == "bf16":
        w.k = inputs.round_bf16(w.k)
    o, S = run_gpu(w, raw_keys=True)
    ro, rS = oracle_ref(w, raw_keys=True)
    check(o, ro, dtype, "O")
    check(S, rS, dtype, "S_F")


# ------------------------------------------------------------------ reverse direction
@pytest.mark.parametrize("B,H,F,N,D,dtype", [
    (1, 2, 7, 33, 16, "bf16"), (2, 3, 5, 130, 64, "bf16"), (1, 2, 6, 257, 128, "bf16"),
    (1, 2, 4, 50, 32, "f32"), (2, 2, 3, 70, 128, "f32")])
def test_reverse_scan(B, H, F, N, D, dtype):
    w = inputs.make(B, H, F, N, D, dtype=dtype, seed=71 + F + D, s0_std=0.05)
    o, S = run_gpu(w, reverse=True)
    ro, rS = oracle_ref(w, reverse=True)
    check(o, ro, dtype, "O")
    check(S, rS, dtype, "S_F")


def test_reverse_scan_over_launch_chunks_and_in_place():
    """300 frames in reverse: two launch chunks visited last-first, the state
    carried between them, also in place (S_final is S0)."""
    w = inputs.make(1, 2, 300, 24, 32, dtype="bf16", seed=73, s0_std=0.05)
    o, S = run_gpu(w, reverse=True)
    ro, rS = oracle_ref(w, reverse=True)
    check(o, ro, "bf16", "O")
    check(S, rS, "bf16", "S_F")
    q, k, v, b, a, s0 = inputs.to_torch(w, "cuda")
    carry = s0.clone()
    o2, _ = api.frame_scan_fwd(q, k, v, b, a, carry, S_final=carry, reverse=True)
    torch.cuda.synchronize()
    assert torch.equal(o2.float().cpu(), torch.from_numpy(o)) and np.array_equal(carry.cpu().numpy(), S)


def test_reverse_short_clip_every_unit():
    w = inputs.make_config("short_clip", seed=0)
    o, S = run_gpu(w, reverse=True)
    ro, rS = oracle_ref(w, reverse=True)
    check_every_unit(w, o, S, ro, rS)


def test_reverse_of_one_frame_is_the_forward_step():
    w = inputs.make(2, 3, 1, 100, 64, dtype="bf16", seed=74, s0_std=0.05)
    o1, S1 = run_gpu(w)
    o2, S2 = run_gpu(w, reverse=True)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


# ------------------------------------------------------------------ full-size workloads
def check_every_unit(w, o, S, ro, rS):
    """Whole-tensor tolerances, then each (b, h) unit on its own."""
    check(o, ro, w.dtype, "O")
    check(S, rS, w.dtype, "S_F")
    worst_o, worst_s = (0.0, 0.0, None), (0.0, 0.0, None)
    for b in range(w.B):
        for h in range(w.H):
            mo, ro_ = errs(o[b, :, :, h], ro[b, :, :, h])
            ms, rs_ = errs(S[b, h], rS[b, h])
            if ro_ > worst_o[1]:
                worst_o = (mo, ro_, (b, h))
            if rs_ > worst_s[1]:
                worst_s = (ms, rs_, (b, h))
            ok = (mo <= TOL_BF16_MAXABS and ro_ <= TOL_BF16_REL and ms <= TOL_BF16_MAXABS
                  and rs_ <= TOL_BF16_REL)
            assert ok, ("unit", b, h, mo, ro_, ms, rs_)
    print("worst unit O: max %.3e rel %.3e at %s; S_F: max %.3e rel %.3e at %s"
          % (worst_o + worst_s))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_short_clip_every_unit(seed):
    w = inputs.make_config("short_clip", seed=seed)
    o, S = run_gpu(w)
    ro, rS = oracle_ref(w)
    check_every_unit(w, o, S, ro, rS)


@pytest.mark.slow
@pytest.mark.parametrize("seed", [0, 1])
def test_full_minute_every_unit(seed):
    w = inputs.make_config("full_minute", seed=seed)
    o, S = run_gpu(w)
    ro, rS = oracle_ref(w)
    check_every_unit(w, o, S, ro, rS)


@pytest.mark.slow
def test_guidance_every_unit():
    w = inputs.make_config("guidance", seed=0)
    o, S = run_gpu(w)
    ro, rS = oracle_ref(w)
    check_every_unit(w, o, S, ro, rS)


@pytest.mark.slow
def test_full_minute_twice_bitwise_and_guard_bands():
    """Two runs of the full-minute scan give the same bits, and the bytes just
    before and after O, S_final and the workspace keep their canary values."""
    w = inputs.make_config("full_minute", seed=0)
    q, k, v, b, a, _ = inputs.to_torch(w, "cuda")
    desc = api.make_desc(w.B, w.H, w.F, w.N, w.Dk, q.dtype)
    need = api.workspace_size(desc)
    G = 1 << 16                                       # guard elements on each side
    n_o = q.numel()
    o_buf = torch.full((n_o + 2 * G,), -7.25, dtype=q.dtype, device="cuda")
    s_buf = torch.full((w.B * w.H * w.Dv * w.Dk + 2 * G,), 3.5, dtype=torch.float32, device="cuda")
    ws_buf = torch.full((need + 2 * (G * 4),), 0xA5, dtype=torch.uint8, device="cuda")
    o = o_buf[G:G + n_o].view(q.shape)
    S = s_buf[G:G + w.B * w.H * w.Dv * w.Dk].view(w.B, w.H, w.Dv, w.Dk)
    ws = ws_buf[G * 4:G * 4 + need]
    api.frame_scan_fwd(q, k, v, b, a, None, o=o, S_final=S, workspace=ws)
    o1, S1 = o.clone(), S.clone()
    o.fill_(0.0)
    S.fill_(0.0)
    api.frame_scan_fwd(q, k, v, b, a, None, o=o, S_final=S, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(S, S1)
    for buf, val, g in ((o_buf, -7.25, G), (s_buf, 3.5, G)):
        assert torch.all(buf[:g] == val) and torch.all(buf[-g:] == val)
    assert torch.all(ws_buf[:G * 4] == 0xA5) and torch.all(ws_buf[-G * 4:] == 0xA5)


def test_nan_stays_in_its_unit():
    """A NaN key in one (b, h) at frame f poisons that unit from frame f on and
    nothing else: every other unit, and that unit's earlier frames, keep the
    bits of the clean run."""
    w = inputs.make(2, 4, 6, 300, 128, dtype="bf16", seed=53, s0_std=0.05)
    o0, S0 = run_gpu(w)
    w.k[1, 3, 17, 2, 5] = np.nan                   # b = 1, frame 3, token 17, head 2
    o1, S1 = run_gpu(w)
    for b in range(w.B):
        for h in range(w.H):
            if (b, h) == (1, 2):
                assert np.array_equal(o1[b, :3, :, h], o0[b, :3, :, h])
                assert np.isnan(o1[b, 3:, :, h]).any() and np.isnan(S1[b, h]).any()
            else:
                assert np.array_equal(o1[b, :, :, h], o0[b, :, :, h]), (b, h)
                assert np.array_equal(S1[b, h], S0[b, h]), (b, h)


def test_explicit_side_stream():
    """Called with a stream that is not the current one: outputs and the
    internal workspace are allocated on that stream, and the results match the
    oracle after the stream is synchronised."""
    w = inputs.make(2, 4, 5, 300, 128, dtype="bf16", seed=54, s0_std=0.05)
    q, k, v, b, a, s0 = inputs.to_torch(w, "cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, S = api.frame_scan_fwd(q, k, v, b, a, s0, stream=side)
    junk = [torch.full((1 << 24,), 1.0, device="cuda") for _ in range(4)]  # current-stream churn
    side.synchronize()
    del junk
    ro, rS = oracle_ref(w)
    check(o.float().cpu().numpy(), ro, "bf16", "O")
    check(S.cpu().numpy(), rS, "bf16", "S_F")


def test_api_rejects_bad_buffers():
    w = inputs.make(1, 2, 1, 40, 64, dtype="bf16", seed=55)
    q, k, v, b, a, s0 = inputs.to_torch(w, "cuda")
    with pytest.raises(ValueError):          # a 4-D frame with a 5-D output of the wrong shape
        api.frame_step(q[:, 0], k[:, 0], v[:, 0], b[:, 0], a[:, 0], None,
                       o=torch.empty((1, 1, 1, 40, 2, 64), dtype=q.dtype, device="cuda"))
    with pytest.raises(ValueError):          # output too small
        api.frame_step(q[:, 0], k[:, 0], v[:, 0], b[:, 0], a[:, 0], None,
                       o=torch.empty((1, 20, 2, 64), dtype=q.dtype, device="cuda"))
    with pytest.raises(TypeError):
        api.frame_step(q[:, 0], k[:, 0], v[:, 0], b[:, 0], a[:, 0], None,
                       o=torch.empty((1, 40, 2, 64), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):          # workspace in host memory
        api.frame_scan_fwd(q, k, v, b, a, None, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):          # workspace of the wrong dtype
        api.frame_scan_fwd(q, k, v, b, a, None,
                           workspace=torch.empty(1 << 18, dtype=torch.float32, device="cuda"))


@pytest.mark.slow
@pytest.mark.parametrize("carry", ["in_place", "two_buffers"])
def test_streaming_steps_match_scan_and_oracle(carry):
    """64 calls of the single-frame step carrying fp32 state, against one
    64-frame scan of the same frames and against the oracle on every (b, h)
    unit.  The step runs its own kernels (in place: token-range partials summed
    in fp32, the state update fused into the output pass; in two alternating
    buffers: one launch that forms each frame's G and U itself), so it matches
    the scan to rounding, not bit for bit; both must meet the oracle's
    tolerance."""
    w = inputs.make_config("streaming", seed=0)
    q, k, v, b, a, _ = inputs.to_torch(w, "cuda")
    o_scan, S_scan = api.frame_scan_fwd(q, k, v, b, a, None)
    bufs = [torch.zeros_like(S_scan)] + ([torch.full_like(S_scan, float("nan"))] if carry == "two_buffers" else [])
    o_steps = torch.empty_like(o_scan)
    desc = api.make_desc(w.B, w.H, 1, w.N, w.Dk, q.dtype)
    ws = api.alloc_workspace(desc, q.device)
    for f in range(w.F):
        # each streamed frame arrives as its own tensor
        S_in, S_out = bufs[f % len(bufs)], bufs[(f + 1) % len(bufs)]
        of, _ = api.frame_step(q[:, f].contiguous(), k[:, f].contiguous(), v[:, f].contiguous(),
                               b[:, f].contiguous(), a[:, f].contiguous(), S_in, S_out=S_out,
                               workspace=ws)
        o_steps[:, f] = of
    torch.cuda.synchronize()
    S = bufs[w.F % len(bufs)]
    diff = (o_steps.float() - o_scan.float()).abs().max().item()
    print("max |step - scan| on O: %g, on S: %g" % (diff, (S - S_scan).abs().max().item()))
    check(o_steps.float().cpu().numpy(), o_scan.float().cpu().numpy(), "bf16", "O steps vs scan")
    check(S.cpu().numpy(), S_scan.cpu().numpy(), "bf16", "S steps vs scan")
    ro, rS = oracle_ref(w)
    check_every_unit(w, o_steps.float().cpu().numpy(), S.cpu().numpy(), ro, rS)
    check_every_unit(w, o_scan.float().cpu().numpy(), S_scan.cpu().numpy(), ro, rS)
