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


# ---------------------------------------------------------------- MXFP8 encoding
def _e4m3_value(code):
    """OCP FP8 E4M3 from its bit fields: sign, 4 exponent bits (bias 7), 3
    mantissa bits; exponent 0 is subnormal; 0x7F and 0xFF are NaN."""
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def test_e4m3_decoding_matches_the_format_definition():
    import torch
    codes = torch.arange(256, dtype=torch.uint8)
    dec = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = np.array([_e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(dec), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(dec[fin], want[fin])
    assert want[0x7E] == 448.0 and want[0x01] == 2.0 ** -9 and want[0x38] == 1.0


def test_mxfp8_blocks_scales_and_rounding():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((3, 7, 128)) * np.exp2(rng.integers(-20, 20, (3, 7, 1)))).astype(np.float32)
    x[0, 0, :32] = 0.0                                  # an all-zero block
    codes, scales, deq = inputs.to_mxfp8(x)
    assert codes.shape == x.shape and scales.shape == (3, 7, 4) and codes.dtype == np.uint8
    vals = np.array([_e4m3_value(c) for c in range(256)])[codes]
    e = scales.astype(np.int64) - 127
    np.testing.assert_array_equal(deq, (vals * np.exp2(np.repeat(e, 32, axis=-1))).astype(np.float32))
    blk = np.abs(x.reshape(3, 7, 4, 32)).max(-1)
    nz = blk > 0
    np.testing.assert_array_equal(e[nz], np.floor(np.log2(blk[nz])) - 8)
    vmax = np.abs(vals.reshape(3, 7, 4, 32)).max(-1)
    assert np.all(vmax[nz] >= 256) and np.all(vmax[nz] <= 448)
    assert np.all(deq[0, 0, :32] == 0)
    # round to nearest: within half a step of the E4M3 grid at each value's
    # binade, except above 464 (half a step past 448), which saturates to 448
    sc = np.exp2(np.repeat(e, 32, axis=-1))
    t = np.abs(x / sc)
    step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(t, 2.0 ** -6))), -6) - 3)
    err = np.abs(x / sc - deq / sc)
    assert np.all(err[t <= 464] <= step[t <= 464] / 2 + 1e-12)
    assert np.all(np.abs(deq / sc)[t > 464] == 448)
    # values already on the grid come back exactly
    c2, s2, d2 = inputs.to_mxfp8(deq)
    np.testing.assert_array_equal(d2, deq)


# ------------------------------------------------------------------ MXFP4 (E2M1)
def e2m1_value(code):
    """An E2M1 code's value from its bit fields (sign, 2 exponent bits with
    bias 1, 1 mantissa bit; exponent 0 is subnormal)."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m / 2.0) if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def unpack4(packed):
    return np.stack([packed & 15, packed >> 4], axis=-1).reshape(packed.shape[:-1] + (2 * packed.shape[-1],))


def test_mxfp4_decode_matches_the_bit_fields():
    # every representable magnitude times a block scale encodes to itself
    vals = np.array([e2m1_value(c) for c in range(16)])
    assert sorted(set(np.abs(vals))) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    x = np.zeros((1, 32), np.float32)
    x[0, :16] = vals * 4.0
    x[0, 16:] = 6.0 * 4.0                       # amax 24 -> e = floor(log2 24) - 2 = 2
    packed, sc, deq = inputs.to_mxfp4(x)
    assert sc[0, 0] == 127 + 2
    codes = unpack4(packed)
    np.testing.assert_array_equal(deq, x)
    for c in range(16):
        if vals[c] != 0.0 or c == 0:
            assert codes[0, c] == c, (c, codes[0, c])


def test_mxfp4_rounding_ties_even_and_saturation():
    # with amax = 6 (scale 2^0): midpoints go to the even code, values past 6 saturate
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    x = np.zeros((1, 32), np.float32)
    x[0, :7] = mids
    x[0, 7:14] = [-m for m in mids]
    x[0, 14] = 6.0
    x[0, 15] = 7.9                              # amax < 8 keeps e = 0, saturates to 6
    x[0, 16] = 0.26                             # just past a midpoint: rounds up
    _, sc, deq = inputs.to_mxfp4(x)
    assert sc[0, 0] == 127
    np.testing.assert_array_equal(deq[0, :7], want)
    np.testing.assert_array_equal(deq[0, 7:14], [-w for w in want])
    assert deq[0, 14] == 6.0 and deq[0, 15] == 6.0 and deq[0, 16] == 0.5


def test_mxfp4_scale_rule_and_error_bound():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 128)) * np.exp2(rng.integers(-6, 6, (64, 1)))).astype(np.float32)
    packed, sc, deq = inputs.to_mxfp4(x)
    assert packed.shape == (64, 64) and sc.shape == (64, 4)
    blk = np.abs(x.reshape(64, 4, 32)).max(-1)
    e = sc.astype(np.int64) - 127
    # amax lies in [4, 8) * 2^e, so every value fits below the saturation point 6 * 2^e except the top ones
    assert np.all(blk >= 4.0 * np.exp2(e)) and np.all(blk < 8.0 * np.exp2(e))
    # below saturation the error is at most half the local spacing (1 * 2^e above 4, 0.25 * 2^e below 0.5 ...)
    err = np.abs(deq - x).reshape(64, 4, 32)
    sat = np.abs(x.reshape(64, 4, 32)) > 6.0 * np.exp2(e)[..., None]
    assert np.all(err[~sat] <= np.exp2(e)[..., None].repeat(32, -1)[~sat] + 1e-30)


def test_mxfp4_device_recipe_equals_host_recipe():
    # the torch encoder (run here on CPU tensors, in small pieces) against the
    # numpy one, over scales from 2^-20 to 2^20 and an all-zero block
    import torch
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((3, 5, 7, 64)) * np.exp2(rng.integers(-20, 20, (3, 5, 7, 1)))).astype(np.float32)
    x[0, 0, 0, :32] = 0.0
    c, s, _ = inputs.to_mxfp4(x)
    for chunk in (7, 1 << 22):
        dc, ds = inputs.to_mxfp4_device(torch.from_numpy(x), chunk_blocks=chunk)
        np.testing.assert_array_equal(dc.numpy(), c)
        np.testing.assert_array_equal(ds.numpy(), s)
