"""The one-frame path (gdn_frame_step, and gdn_frame_scan_fwd with F == 1)
against the fp64 oracle.

That path runs its own kernels: frame_gram splits each (b, h) into token
ranges and writes fp32 partial G and U, and frame_step sums them, forms S_1
and the output in one launch.  These cases cover every head size and I/O
dtype, ragged and tiny token counts (one range, many ranges, a last range of
one token), no tokens at all, a NULL initial state, logit gates and the
in-place carry S_out == S_in.  Tolerances are those of test_gpu_parity.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_scan_amd import api, inputs
from test_gpu_parity import check, oracle_ref

pytestmark = pytest.mark.gpu


def step_gpu(w, *, logits=False, in_place=False, s0=True, beta=None, alpha=None, raw_keys=False):
    q, k, v, b, a, S0 = inputs.to_torch(w, "cuda")
    if beta is not None:
        b = torch.from_numpy(np.ascontiguousarray(beta, dtype=np.float32)).cuda()
    if alpha is not None:
        a = torch.from_numpy(np.ascontiguousarray(alpha, dtype=np.float32)).cuda()
    S_in = S0 if s0 else None
    if in_place:
        S_out = S_in
    else:
        S_out = torch.full((w.B, w.H, w.Dv, w.Dk), float("nan"), dtype=torch.float32, device="cuda")
    o, S = api.frame_step(q[:, 0], k[:, 0], v[:, 0], b[:, 0], a[:, 0], S_in, S_out=S_out,
                          gates_are_logits=logits, normalize_keys=not raw_keys)
    torch.cuda.synchronize()
    assert S.data_ptr() == S_out.data_ptr()
    return o.float().cpu().numpy()[:, None], S.cpu().numpy()


CASES = [  # B, H, N, D, dtype
    (1, 1, 1, 16, "bf16"),
    (2, 3, 17, 16, "f32"),
    (1, 2, 100, 32, "bf16"),
    (3, 5, 513, 32, "f32"),
    (4, 8, 880, 64, "bf16"),
    (2, 2, 257, 64, "f32"),
    (1, 1, 880, 128, "bf16"),      # one unit: many token ranges
    (1, 3, 129, 128, "bf16"),      # a last range of one token
    (2, 4, 200, 128, "f32"),
    (4, 80, 40, 16, "bf16"),       # 320 units: several items per frame_gram workgroup
]


@pytest.mark.parametrize("B,H,N,D,dtype", CASES)
def test_step_matches_oracle(B, H, N, D, dtype):
    w = inputs.make(B, H, 1, N, D, dtype=dtype, seed=300 + N + D, s0_std=0.05)
    o, S = step_gpu(w)
    ro, rS = oracle_ref(w)
    check(o, ro, dtype, "O")
    check(S, rS, dtype, "S_out")


@pytest.mark.parametrize("D", [16, 64, 128])
def test_step_in_place_and_null_state(D):
    w = inputs.make(2, 3, 1, 150, D, dtype="bf16", seed=400 + D, s0_std=0.05)
    o, S = step_gpu(w, in_place=True)                  # S_out is S_in
    ro, rS = oracle_ref(w)
    check(o, ro, "bf16", "O in place")
    check(S, rS, "bf16", "S_out in place")
    o0, S0 = step_gpu(w, s0=False)                     # S_in NULL -> zeros
    ro0, rS0 = oracle_ref(w, S0=None)
    check(o0, ro0, "bf16", "O from zero state")
    check(S0, rS0, "bf16", "S_out from zero state")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_logit_gates(dtype):
    w = inputs.make(2, 3, 1, 96, 64, dtype=dtype, seed=431, s0_std=0.05)
    bl, al = w.meta["beta_logit"], w.meta["alpha_logit"]
    o, S = step_gpu(w, logits=True, beta=bl, alpha=al)
    ro, rS = oracle_ref(w, logits=True, beta=bl, alpha=al)
    check(o, ro, dtype, "O")
    check(S, rS, dtype, "S_out")


def test_step_without_tokens_decays_only():
    w = inputs.make(2, 3, 1, 0, 32, dtype="bf16", seed=444, s0_std=0.1)
    o, S = step_gpu(w)
    assert o.shape == (2, 1, 0, 3, 32)
    exp = w.alpha.astype(np.float64)[:, 0, :, None, None] * w.S0
    check(S, exp, "f32", "S_out")


def test_scan_of_one_frame_uses_the_same_path():
    w = inputs.make(2, 4, 1, 300, 64, dtype="bf16", seed=450, s0_std=0.05)
    q, k, v, b, a, S0 = inputs.to_torch(w, "cuda")
    o1, S1 = api.frame_scan_fwd(q, k, v, b, a, S0)
    o2, S2 = api.frame_step(q[:, 0], k[:, 0], v[:, 0], b[:, 0], a[:, 0], S0)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, 0], o2) and torch.equal(S1, S2)
    ro, rS = oracle_ref(w)
    check(o1.float().cpu().numpy(), ro, "bf16", "O")
    check(S1.cpu().numpy(), rS, "bf16", "S_F")


@pytest.mark.parametrize("D,in_place", [(64, False), (64, True), (128, False)])
def test_step_raw_keys(D, in_place):
    """Keys used as given, on the one-launch path (D = 64, two buffers) and on
    the two-launch path (in place, and D = 128)."""
    w = inputs.make(2, 3, 1, 200, D, dtype="bf16", seed=460 + D, s0_std=0.05)
    scale = np.random.default_rng(461).uniform(0.3, 0.6, w.k.shape[:-1] + (1,)).astype(np.float32)
    w.k = inputs.round_bf16(w.k * scale)
    o, S = step_gpu(w, in_place=in_place, raw_keys=True)
    ro, rS = oracle_ref(w, raw_keys=True)
    check(o, ro, "bf16", "O")
    check(S, rS, "bf16", "S_out")
