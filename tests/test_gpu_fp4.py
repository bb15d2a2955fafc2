"""Block-scaled FP4 inputs on the GPU (gdn_frame_scan_fwd_fp4).

q, k and v are encoded in the OCP MXFP4 layout (E2M1 values two per byte, one
E8M0 scale per 32 features; gated_deltanet_scan_amd.inputs.to_mxfp4).  The
oracle runs on the dequantised values, unchanged; the bar is the bf16 mode's
(max |err| <= 2e-2, relative Frobenius error <= 5e-3 on o and on S_final):
the kernels widen every loaded value to bf16 exactly (two significant bits
times a power of two), so the path is the bf16 path on those values.  That is
also checked directly: the result equals gdn_frame_scan_fwd's on bf16 tensors
holding the dequantised values bit for bit, which also fixes the nibble order
(a swapped pair of features changes the keys and so the output).
"""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_scan_amd import api, inputs

pytestmark = pytest.mark.gpu

TOL_MAXABS = 2e-2
TOL_REL = 5e-3


def errs(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    n = np.linalg.norm(ref)
    return (float(np.abs(d).max()) if d.size else 0.0), (float(np.linalg.norm(d) / n) if n > 0 else 0.0)


def check(got, ref, what):
    mx, rel = errs(got, ref)
    print("%s: max|err| %.3e  rel %.3e" % (what, mx, rel))
    assert mx <= TOL_MAXABS and rel <= TOL_REL, (what, mx, rel)


def dev(x, dt=torch.uint8):
    if dt == torch.float32:
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_fp4(enc, w, *, beta=None, alpha=None, **kw):
    (qc, qs), (kc, ks), (vc, vs) = enc
    b = dev(w.beta if beta is None else beta, torch.float32)
    a = dev(w.alpha if alpha is None else alpha, torch.float32)
    s0 = None if w.S0 is None else dev(w.S0, torch.float32)
    o, S = api.frame_scan_fwd_fp4(dev(qc), dev(qs), dev(kc), dev(ks), dev(vc), dev(vs), b, a, s0, **kw)
    torch.cuda.synchronize()
    return o, S


def ref(deq, *, beta=None, alpha=None, logits=False, raw=False, reverse=False):
    return oracle.scan(deq.q, deq.k, deq.v, deq.beta if beta is None else beta,
                       deq.alpha if alpha is None else alpha, deq.S0, gates_are_logits=logits,
                       normalize_keys=not raw, reverse=reverse)


def bf16_path(deq, **kw):
    q, k, v, b, a, s0 = inputs.to_torch(deq, "cuda")
    o, S = api.frame_scan_fwd(q, k, v, b, a, s0, **kw)
    torch.cuda.synchronize()
    return o, S


SHAPES = [(1, 2, 5, 100, 128, 0.1), (2, 2, 4, 70, 64, 0.0), (1, 3, 6, 130, 32, 0.1), (1, 2, 1, 90, 64, 0.1)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dF%dN%dD%d" % s[:5])
@pytest.mark.parametrize("mode", ["plain", "logits", "raw", "reverse"])
def test_matches_oracle_on_dequantised_values(shape, mode):
    B, H, F, N, D, s0 = shape
    w = inputs.make(B, H, F, N, D, dtype="f32", seed=31, s0_std=s0, normalise_k=(mode != "raw"))
    if mode == "raw":
        w.beta = (w.beta / D).astype(np.float32)
    enc, deq = inputs.make_fp4(w)
    kw, rk = {}, {}
    if mode == "logits":
        rng = np.random.default_rng(32)
        bl = rng.standard_normal(w.beta.shape).astype(np.float32)
        al = (rng.standard_normal(w.alpha.shape) + 3.0).astype(np.float32)
        kw = dict(beta=bl, alpha=al, gates_are_logits=True)
        rk = dict(beta=bl, alpha=al, logits=True)
    elif mode == "raw":
        kw, rk = dict(normalize_keys=False), dict(raw=True)
    elif mode == "reverse":
        kw, rk = dict(reverse=True), dict(reverse=True)
    o, S = run_fp4(enc, w, **kw)
    o_ref, S_ref = ref(deq, **rk)
    check(o.float().cpu().numpy(), o_ref, "o %s %s" % (shape, mode))
    check(S.cpu().numpy(), S_ref, "S %s %s" % (shape, mode))


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("reverse", [False, True])
def test_equals_bf16_path_on_dequantised_values(D, reverse):
    w = inputs.make(2, 2, 4, 150, D, dtype="f32", seed=33, s0_std=0.1)
    enc, deq = inputs.make_fp4(w)
    o4, S4 = run_fp4(enc, w, reverse=reverse)
    o16, S16 = bf16_path(deq, reverse=reverse)
    assert torch.equal(o4, o16) and torch.equal(S4, S16)


def test_nibble_order_single_feature():
    """Two nonzero features per token, 1 at feature j and -0.5 at j + 1 (both
    exact in E2M1 under any block scale), q = k = v, with j odd or even at
    random: a decoder that swapped the two features of a byte would put the
    values on other features and change o and S_final far beyond the bar."""
    B, H, F, N, D = 1, 1, 2, 64, 64
    rng = np.random.default_rng(34)
    x = np.zeros((B, F, N, H, D), np.float32)
    for f in range(F):
        for n in range(N):
            j = int(rng.integers(0, D - 1))
            x[0, f, n, 0, j] = 1.0
            x[0, f, n, 0, j + 1] = -0.5
    w = inputs.make(B, H, F, N, D, dtype="f32", seed=35, s0_std=0.0, normalise_k=False)
    w.q, w.k, w.v = x.copy(), x.copy(), x.copy()
    w.beta = np.full(w.beta.shape, 0.25, np.float32)
    enc, deq = inputs.make_fp4(w)
    np.testing.assert_array_equal(deq.q, x)          # the values are exact in E2M1
    o, S = run_fp4(enc, w, normalize_keys=False)
    o_ref, S_ref = ref(deq, raw=True)
    check(o.float().cpu().numpy(), o_ref, "o one-hot")
    check(S.cpu().numpy(), S_ref, "S one-hot")


def test_more_than_one_chunk():
    w = inputs.make(1, 2, 300, 5, 32, dtype="f32", seed=36, s0_std=0.1)
    enc, deq = inputs.make_fp4(w)
    o, S = run_fp4(enc, w)
    o_ref, S_ref = ref(deq)
    check(o.float().cpu().numpy(), o_ref, "o chunks")
    check(S.cpu().numpy(), S_ref, "S chunks")


def test_device_encoder_matches_host_encoder():
    w = inputs.make(1, 2, 3, 97, 128, dtype="f32", seed=37, s0_std=0.0)
    for x in (w.q, w.k, w.v):
        c, s, _ = inputs.to_mxfp4(x)
        dc, ds = inputs.to_mxfp4_device(torch.from_numpy(x).cuda())
        np.testing.assert_array_equal(dc.cpu().numpy(), c)
        np.testing.assert_array_equal(ds.cpu().numpy(), s)


def test_full_minute_units_and_bitwise_bf16():
    """The full-minute workload (B1 H16 F121 N880 d128) in MXFP4: three (b, h)
    units against the oracle, and the whole output against the bf16 path on
    the dequantised values, bit for bit."""
    w = inputs.make_config("full_minute", seed=0)
    enc, deq = inputs.make_fp4(w)
    o4, S4 = run_fp4(enc, w)
    for h in (0, 9, 15):
        sl = (slice(0, 1), slice(None), slice(None), slice(h, h + 1))
        o_ref, S_ref = oracle.scan(deq.q[sl], deq.k[sl], deq.v[sl], deq.beta[sl], deq.alpha[:, :, h:h + 1], None)
        check(o4[sl].float().cpu().numpy(), o_ref, "o unit %d" % h)
        check(S4[:, h:h + 1].cpu().numpy(), S_ref, "S unit %d" % h)
    o16, S16 = bf16_path(deq)
    assert torch.equal(o4, o16) and torch.equal(S4, S16)


def run_fp8(enc, w):
    (qc, qs), (kc, ks), (vc, vs) = enc
    f8 = lambda x: dev(x).view(torch.float8_e4m3fn)
    s0 = None if w.S0 is None else dev(w.S0, torch.float32)
    o, S = api.frame_scan_fwd_fp8(f8(qc), dev(qs), f8(kc), dev(ks), f8(vc), dev(vs), dev(w.beta, torch.float32),
                                  dev(w.alpha, torch.float32), s0)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
@pytest.mark.parametrize("F,N", [(3, 0), (0, 40), (1, 0)])
def test_empty_frames_or_tokens(fmt, F, N):
    """No tokens: the state only decays, S_final = (prod alpha) S0 and o is
    empty; no frames: S_final = S0.  Both MX entry points, against the oracle."""
    w = inputs.make(2, 3, F, N, 64, dtype="f32", seed=38, s0_std=0.1)
    enc, deq = (inputs.make_fp8 if fmt == "fp8" else inputs.make_fp4)(w)
    o, S = (run_fp8 if fmt == "fp8" else run_fp4)(enc, w)
    o_ref, S_ref = ref(deq)
    assert o.shape == (2, F, N, 3, 64) and o.numel() == 0
    check(S.cpu().numpy(), S_ref, "S %s F%d N%d" % (fmt, F, N))
    if F == 0:
        assert np.array_equal(S.cpu().numpy(), w.S0)
