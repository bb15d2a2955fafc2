"""The seeded synthetic recipe: deterministic, right shapes and distributions."""
import numpy as np

from gated_deltanet_scan_amd import inputs


def test_deterministic_and_seed_sensitive():
    a = inputs.make(1, 2, 3, 10, 16, dtype="bf16", seed=0)
    b = inputs.make(1, 2, 3, 10, 16, dtype="bf16", seed=0)
    c = inputs.make(1, 2, 3, 10, 16, dtype="bf16", seed=1)
    for x in ("q", "k", "v", "beta", "alpha"):
        assert np.array_equal(getattr(a, x), getattr(b, x))
        assert not np.array_equal(getattr(a, x), getattr(c, x))


def test_shapes_and_distributions():
    w = inputs.make(2, 3, 5, 200, 32, dtype="bf16", seed=3, s0_std=0.02)
    assert w.q.shape == (2, 5, 200, 3, 32) and w.v.shape == (2, 5, 200, 3, 32)
    assert w.beta.shape == (2, 5, 200, 3) and w.alpha.shape == (2, 5, 3)
    assert w.S0.shape == (2, 3, 32, 32) and abs(w.S0.std() - 0.02) < 0.002
    n = np.linalg.norm(w.k.astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)                 # unit keys up to bf16 rounding
    assert np.all(w.beta > 0) and np.all(w.beta < 1.0 / 200)
    assert abs(w.beta.mean() * 200 - 0.5) < 0.02        # E[sigmoid(N(0,1))] = 0.5
    assert np.all((w.alpha > 0) & (w.alpha < 1)) and 0.85 < w.alpha.mean() < 0.97
    assert abs(w.q.std() - 1) < 0.05


def test_named_configs():
    t = inputs.make_config("tiny_fp32")
    assert (t.B, t.H, t.F, t.N, t.Dk, t.dtype, t.S0) == (1, 2, 8, 12, 16, "f32", None)
    assert inputs.CONFIGS["full_minute"] == dict(B=1, H=16, D=128, F=121, N=880, dtype="bf16",
                                                 s0_std=0.0)
    assert inputs.CONFIGS["guidance"]["B"] == 2 and inputs.CONFIGS["guidance"]["s0_std"] == 0.02
    assert inputs.CONFIGS["streaming"]["D"] == 64 and inputs.CONFIGS["streaming"]["H"] == 32
