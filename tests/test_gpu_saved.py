"""Training with saved states (gdn_frame_scan_fwd_save, gdn_frame_scan_bwd_saved).

The saved forward runs the scan's own kernels into the caller's buffer, so for
F > 1 its o and S_final must equal gdn_frame_scan_fwd's bit for bit where the
plain forward keeps full-precision intermediates (below d 64 or 128 tokens per
frame; a one-frame gdn_frame_scan_fwd call takes the streaming step's kernels,
so F == 1 is compared with the oracle at the forward's bar instead).  At larger
shapes the plain forward hands U and the state planes between its kernels in
bf16 while the saved forward keeps the full forms the backward reads, so there
the two forwards agree to rounding and both are checked against the oracle.  The
backward from saved states reads exactly the operands the recomputing
backward rebuilds with the same kernels, so its gradients must equal
gdn_frame_scan_bwd's bit for bit; that path is itself checked against the
fp64 oracle in test_gpu_bwd.py, and one case here checks the saved path
against the oracle directly.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_scan_amd import api, inputs

pytestmark = pytest.mark.gpu


def dev(x, dt=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(dt).contiguous()


def setup(shape, mode, seed):
    B, H, F, N, D, dtype, s0 = shape
    w = inputs.make(B, H, F, N, D, dtype=dtype, seed=seed, s0_std=s0, normalise_k=(mode != "raw"))
    if mode == "raw":
        w.beta = (w.beta / D).astype(np.float32)
    kw = {}
    q, k, v, b, a, S0 = inputs.to_torch(w, "cuda")
    if mode == "logits":
        rng = np.random.default_rng((seed, 2))
        b = dev(rng.standard_normal(w.beta.shape))
        a = dev(rng.standard_normal(w.alpha.shape) + 3.0)
        kw = dict(gates_are_logits=True)
    elif mode == "raw":
        kw = dict(normalize_keys=False)
    elif mode == "reverse":
        kw = dict(reverse=True)
    dO, dS = inputs.make_grads(w, seed=seed)
    return w, (q, k, v, b, a, S0), dev(dO, q.dtype), (None if dS is None else dev(dS)), kw


def same(x, y, what):
    if x is None or y is None:
        assert x is None and y is None, what
        return
    assert torch.equal(x, y), "%s differs (max %g)" % (what, (x.float() - y.float()).abs().max().item())


SHAPES = [
    (1, 2, 5, 100, 128, "bf16", 0.1),
    (2, 2, 4, 70, 64, "bf16", 0.0),
    (1, 3, 6, 130, 32, "bf16", 0.1),
    (1, 2, 5, 20, 32, "f32", 0.1),
    (1, 2, 8, 12, 16, "f32", 0.0),
    (1, 2, 300, 5, 16, "bf16", 0.1),     # two launch chunks
    (1, 2, 300, 5, 16, "f32", 0.1),
    (1, 2, 4, 0, 32, "f32", 0.1),        # no tokens
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dF%dN%dD%d_%s" % s[:6])
@pytest.mark.parametrize("mode", ["plain", "logits", "raw", "reverse"])
def test_saved_equals_recompute(shape, mode):
    w, (q, k, v, b, a, S0), dO, dS, kw = setup(shape, mode, 21)
    o_ref, S_ref = api.frame_scan_fwd(q, k, v, b, a, S0, **kw)
    o, S, saved = api.frame_scan_fwd_save(q, k, v, b, a, S0, **kw)
    g_ref = api.frame_scan_bwd(q, k, v, b, a, dO, S0, dS, **kw)
    g = api.frame_scan_bwd(q, k, v, b, a, dO, None, dS, saved=saved, **kw)
    torch.cuda.synchronize()
    same(o, o_ref, "o")
    same(S, S_ref, "S_final")
    for name, x, y in zip(("dq", "dk", "dv", "dbeta", "dalpha", "dS0"), g, g_ref):
        same(x, y, name)


def test_one_frame_against_oracle():
    # F == 1: the saved forward runs the scan kernels, the plain call the step's
    shape = (2, 2, 1, 90, 64, "bf16", 0.1)
    w, (q, k, v, b, a, S0), dO, dS, kw = setup(shape, "plain", 22)
    o, S, saved = api.frame_scan_fwd_save(q, k, v, b, a, S0)
    g = api.frame_scan_bwd(q, k, v, b, a, dO, None, dS, saved=saved)
    g_ref = api.frame_scan_bwd(q, k, v, b, a, dO, S0, dS)
    torch.cuda.synchronize()
    ro, rS = oracle.scan(w.q, w.k, w.v, w.beta, w.alpha, w.S0)
    for got, ref in ((o, ro), (S, rS)):
        got = got.float().cpu().numpy().astype(np.float64)
        assert np.abs(got - ref).max() <= 2e-2
        assert np.linalg.norm(got - ref) <= 5e-3 * np.linalg.norm(ref)
    for name, x, y in zip(("dq", "dk", "dv", "dbeta", "dalpha", "dS0"), g, g_ref):
        same(x, y, name)


def test_in_place_state_keeps_S0_for_backward():
    # S_final written over S0: the saved buffer keeps the state entering the walk
    shape = (1, 2, 5, 60, 64, "bf16", 0.1)
    w, (q, k, v, b, a, S0), dO, dS, kw = setup(shape, "plain", 23)
    S0_copy = S0.clone()
    g_ref = api.frame_scan_bwd(q, k, v, b, a, dO, S0_copy, dS)
    o, S, saved = api.frame_scan_fwd_save(q, k, v, b, a, S0, S_final=S0)
    g = api.frame_scan_bwd(q, k, v, b, a, dO, None, dS, saved=saved)
    torch.cuda.synchronize()
    assert S.data_ptr() == S0.data_ptr()
    for name, x, y in zip(("dq", "dk", "dv", "dbeta", "dalpha", "dS0"), g, g_ref):
        same(x, y, name)


def test_saved_path_against_oracle():
    shape = (1, 2, 6, 80, 64, "bf16", 0.1)
    w, (q, k, v, b, a, S0), dO, dS, kw = setup(shape, "plain", 24)
    _, _, saved = api.frame_scan_fwd_save(q, k, v, b, a, S0)
    g = api.frame_scan_bwd(q, k, v, b, a, dO, None, dS, saved=saved)
    torch.cuda.synchronize()
    dO_h = dO.float().cpu().numpy()
    ref = oracle.scan_bwd(w.q, w.k, w.v, w.beta, w.alpha, w.S0, dO_h, None if dS is None else dS.cpu().numpy())
    for name, x, r in zip(("dq", "dk", "dv", "dbeta", "dalpha", "dS0"), g, ref):
        got = x.float().cpu().numpy().astype(np.float64)
        e = np.linalg.norm(got - r) / np.linalg.norm(r)
        print("%s rel %.3e" % (name, e))
        assert e <= 5e-3, name


def test_full_minute_saved_equals_recompute():
    w = inputs.make_config("full_minute", seed=0)
    q, k, v, b, a, S0 = inputs.to_torch(w, "cuda")
    dO_h, dS_h = inputs.make_grads(w, seed=0)
    dO, dS = dev(dO_h, q.dtype), dev(dS_h)
    o_ref, S_ref = api.frame_scan_fwd(q, k, v, b, a, S0)
    o, S, saved = api.frame_scan_fwd_save(q, k, v, b, a, S0)
    torch.cuda.synchronize()
    # the plain forward's bf16 intermediates against the saved forward's full
    # ones, and the saved forward against the oracle
    ro, rS = oracle.scan(w.q, w.k, w.v, w.beta, w.alpha, w.S0)
    for got, ref, what in ((o, ro, "o"), (S, rS, "S_final"), (o_ref, ro, "o (plain)"), (S_ref, rS, "S_final (plain)")):
        got = got.float().cpu().numpy().astype(np.float64)
        mx, rel = np.abs(got - ref).max(), np.linalg.norm(got - ref) / np.linalg.norm(ref)
        print("%s: max %.3e rel %.3e" % (what, mx, rel))
        assert mx <= 2e-2 and rel <= 5e-3, what
    del o_ref, S_ref, ro, rS
    g = api.frame_scan_bwd(q, k, v, b, a, dO, None, dS, saved=saved)
    g_ref = api.frame_scan_bwd(q, k, v, b, a, dO, S0, dS)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv", "dbeta", "dalpha", "dS0"), g, g_ref):
        same(x, y, name)
