"""Seeded synthetic inputs for the frame-wise GDN scan.

This module is shared by the tests, the benchmark and the oracle checks.  It
draws inputs only: it holds none of the scan's arithmetic and imports neither
the HIP binding nor the oracle.

Shapes follow the workload on the pages: a 60 s clip at 16 fps is 960 raw
frames; an 8x temporal stride with one extra frame gives 121 latent frames, and
a 1280x704 frame at the tokenizer's spatial stride gives a 22x40 = 880-token
latent grid ("NVIDIA's New 2.6B World Model Generates Minute-Scale 720p Video on
a Single GPU", opening section and "Camera Control: Two Branches at Two Rates";
the WorldFoundry "SANA-WM" page, section "Runtime contract" and its first
paragraph, for 1280x704 and 8k+1 windows).  Real Q/K/V come from trained
projections that are not available, so seeded Gaussians stand in for them.

Recipe (numpy PCG64, ``default_rng(seed)``), drawn in this order, each a
float32 standard normal in C order over the listed layout:
  q [B,F,N,H,Dk], k [B,F,N,H,Dk], v [B,F,N,H,Dv], beta-logit [B,F,N,H],
  alpha-logit [B,F,H] (the draw plus 3), then S0 [B,H,Dv,Dk] when it is random.
k is L2-normalised per token in float64.  beta = sigmoid(logit) / N and
alpha = sigmoid(logit), both computed in float64 and rounded once to float32.
For bf16 workloads q, k and v are rounded to bfloat16 (round to nearest even);
the returned float32 arrays hold exactly the values the GPU receives.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Named workloads.  "streaming" is run one frame per call for 64 calls.
CONFIGS = {
    "tiny_fp32": dict(B=1, H=2, D=16, F=8, N=12, dtype="f32", s0_std=0.0),
    "short_clip": dict(B=1, H=16, D=128, F=21, N=880, dtype="bf16", s0_std=0.0),
    "full_minute": dict(B=1, H=16, D=128, F=121, N=880, dtype="bf16", s0_std=0.0),
    "guidance": dict(B=2, H=16, D=128, F=121, N=880, dtype="bf16", s0_std=0.02),
    "streaming": dict(B=4, H=32, D=64, F=64, N=880, dtype="bf16", s0_std=0.0),
}


@dataclass
class Workload:
    B: int
    H: int
    F: int
    N: int
    Dk: int
    Dv: int
    dtype: str                      # "bf16" or "f32": type of q, k, v and o
    q: np.ndarray                   # float32 arrays holding the exact values
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    alpha: np.ndarray
    S0: Optional[np.ndarray]        # float32 [B,H,Dv,Dk] or None (zeros)
    seed: int = 0
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.B * self.F * self.N


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even); return them as float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _sigmoid64(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def _normalise_rows(k: np.ndarray) -> np.ndarray:
    out = np.empty_like(k, dtype=np.float32)
    flat_in = k.reshape(-1, k.shape[-1])
    flat_out = out.reshape(-1, k.shape[-1])
    step = 1 << 20
    for s in range(0, flat_in.shape[0], step):
        blk = flat_in[s:s + step].astype(np.float64)
        nrm = np.sqrt((blk * blk).sum(axis=1, keepdims=True))
        nrm[nrm == 0.0] = 1.0
        flat_out[s:s + step] = (blk / nrm).astype(np.float32)
    return out


def make(B: int, H: int, F: int, N: int, Dk: int, Dv: Optional[int] = None, *,
         dtype: str = "bf16", seed: int = 0, s0_std: float = 0.0,
         normalise_k: bool = True, beta_logit_mean: float = 0.0,
         alpha_logit_mean: float = 3.0, name: str = "") -> Workload:
    """Draw one workload with the recipe in the module docstring."""
    if dtype not in ("bf16", "f32"):
        raise ValueError("dtype must be 'bf16' or 'f32'")
    Dv = Dk if Dv is None else Dv
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, F, N, H, Dk), dtype=np.float32)
    k = rng.standard_normal((B, F, N, H, Dk), dtype=np.float32)
    v = rng.standard_normal((B, F, N, H, Dv), dtype=np.float32)
    bl = rng.standard_normal((B, F, N, H), dtype=np.float32) + np.float32(beta_logit_mean)
    al = rng.standard_normal((B, F, H), dtype=np.float32) + np.float32(alpha_logit_mean)
    S0 = None
    if s0_std > 0.0:
        S0 = (rng.standard_normal((B, H, Dv, Dk), dtype=np.float32)
              * np.float32(s0_std)).astype(np.float32)
    if normalise_k:
        k = _normalise_rows(k)
    beta = (_sigmoid64(bl) / max(N, 1)).astype(np.float32)
    alpha = _sigmoid64(al).astype(np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return Workload(B=B, H=H, F=F, N=N, Dk=Dk, Dv=Dv, dtype=dtype, q=q, k=k, v=v,
                    beta=beta, alpha=alpha, S0=S0, seed=seed, name=name,
                    meta=dict(beta_logit=bl, alpha_logit=al))


def make_grads(w: Workload, seed: int = 0, *, ds_std: float = 1.0):
    """Seeded loss gradients for the backward pass: (dO [B,F,N,H,Dv], dS_final
    [B,H,Dv,Dk]), float32 standard normals from ``default_rng((seed, 1))`` in
    that order, dS_final scaled by ds_std (0: None); dO is rounded to bfloat16
    for bf16 workloads."""
    rng = np.random.default_rng((seed, 1))
    dO = rng.standard_normal((w.B, w.F, w.N, w.H, w.Dv), dtype=np.float32)
    dS = rng.standard_normal((w.B, w.H, w.Dv, w.Dk), dtype=np.float32) * np.float32(ds_std)
    if w.dtype == "bf16":
        dO = round_bf16(dO)
    return dO, (dS.astype(np.float32) if ds_std > 0.0 else None)


def to_mxfp8(x: np.ndarray):
    """Encode x ([..., D], D a multiple of 32) in the OCP microscaling MXFP8
    layout: per block of 32 consecutive values of the last axis one E8M0 scale
    2^e with e = floor(log2(max |x|)) - 8 (8 is the largest exponent of an
    E4M3 value; all-zero blocks take e = 0), and per value the E4M3 code of
    x / 2^e rounded to nearest even, clamped to +-448.  Returns (codes uint8
    [..., D], scale bytes e + 127 uint8 [..., D/32], the dequantised values
    code * 2^e as float32)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    lead, D = x.shape[:-1], x.shape[-1]
    if D % 32:
        raise ValueError("the last axis must be a multiple of 32")
    blk = x.reshape(lead + (D // 32, 32)).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    e = np.floor(np.log2(np.where(amax > 0, amax, 256.0))) - 8
    e = np.clip(e, -127, 127)
    scaled = np.clip(blk / np.exp2(e)[..., None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(scaled).to(torch.float8_e4m3fn)
    deq = codes.to(torch.float64).numpy() * np.exp2(e)[..., None]
    return (codes.view(torch.uint8).numpy().reshape(x.shape), (e + 127).astype(np.uint8),
            deq.reshape(x.shape).astype(np.float32))


def to_mxfp8_device(x):
    """to_mxfp8 on a device tensor (the same recipe, in torch): returns (codes
    torch.float8_e4m3fn, scale bytes torch.uint8) on x's device."""
    import torch
    lead, D = x.shape[:-1], x.shape[-1]
    blk = x.float().reshape(*lead, D // 32, 32)
    amax = blk.abs().amax(dim=-1)
    e = torch.floor(torch.log2(torch.where(amax > 0, amax, torch.full_like(amax, 256.0)))) - 8
    e = e.clamp(-127, 127)
    scaled = (blk / torch.exp2(e).unsqueeze(-1)).clamp(-448.0, 448.0)
    return scaled.to(torch.float8_e4m3fn).reshape(x.shape), (e + 127).to(torch.uint8)


def make_fp8(w: Workload):
    """MXFP8 encodings of a workload's q, k and v, and a copy of the workload
    holding their dequantised values (what the scan computes on).  Returns
    (((q codes, q scales), (k ...), (v ...)), dequantised workload)."""
    from dataclasses import replace
    enc = [to_mxfp8(x) for x in (w.q, w.k, w.v)]
    deq = replace(w, q=enc[0][2], k=enc[1][2], v=enc[2][2], dtype="bf16")
    return tuple((c, s) for c, s, _ in enc), deq


# E2M1 magnitudes by code (bit 3 is the sign), the midpoints between
# neighbouring magnitudes, and the midpoints where a tie goes up to the even
# code (ties between codes 2i+1 and 2i+2)
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MID = (_E2M1[1:] + _E2M1[:-1]) / 2
_E2M1_TIE_UP = _E2M1_MID[1::2]


def to_mxfp4(x: np.ndarray):
    """Encode x ([..., D], D a multiple of 32) in the OCP microscaling MXFP4
    layout: per block of 32 consecutive values of the last axis one E8M0 scale
    2^e with e = floor(log2(max |x|)) - 2 (2 is the largest exponent of an
    E2M1 value; all-zero blocks take e = 0), and per value the E2M1 code of
    x / 2^e rounded to the nearest representable magnitude (ties to the even
    code), saturated at +-6.  Two codes per byte, value 2j in the lower four
    bits of byte j.  Returns (packed uint8 [..., D/2], scale bytes e + 127
    uint8 [..., D/32], the dequantised values as float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lead, D = x.shape[:-1], x.shape[-1]
    if D % 32:
        raise ValueError("the last axis must be a multiple of 32")
    blk = x.reshape(lead + (D // 32, 32))
    amax = np.abs(blk).max(axis=-1).astype(np.float64)
    e = np.floor(np.log2(np.where(amax > 0, amax, 4.0))) - 2
    e = np.clip(e, -127, 127)
    sc = np.exp2(e).astype(np.float32)                 # 2^-127 .. 2^127, exact in float32
    y = blk / sc[..., None]                            # exact: |y| < 8 and a power-of-two divisor
    a = np.abs(y)
    code = np.zeros(a.shape, np.uint8)
    for m in _E2M1_MID.astype(np.float32):             # count the midpoints below a ...
        code += a > m
    for m in _E2M1_TIE_UP.astype(np.float32):          # ... and ties go to the even code
        code += a == m
    code |= (np.signbit(y) & (code > 0)).astype(np.uint8) << 3            # -0 encodes as +0
    signed = np.concatenate([_E2M1, -_E2M1]).astype(np.float32)
    deq = signed[code] * sc[..., None]
    code = code.reshape(x.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8), deq.reshape(x.shape).astype(np.float32)


def to_mxfp4_device(x, chunk_blocks: int = 1 << 24):
    """to_mxfp4 on a device tensor (the same recipe, in torch, in pieces of
    chunk_blocks scale blocks to bound the float64 temporaries): returns
    (packed codes torch.uint8 [..., D/2], scale bytes torch.uint8) on x's
    device."""
    import torch
    lead, D = x.shape[:-1], x.shape[-1]
    blk = x.reshape(-1, 32)
    codes = torch.empty((blk.shape[0], 16), dtype=torch.uint8, device=x.device)
    scales = torch.empty((blk.shape[0],), dtype=torch.uint8, device=x.device)
    mid = torch.tensor(_E2M1_MID, dtype=torch.float64, device=x.device)
    up = torch.tensor(_E2M1_TIE_UP, dtype=torch.float64, device=x.device)
    for i in range(0, blk.shape[0], chunk_blocks):
        b = blk[i:i + chunk_blocks].float()
        amax = b.abs().amax(dim=-1)
        e = torch.floor(torch.log2(torch.where(amax > 0, amax, torch.full_like(amax, 4.0)))) - 2
        e = e.clamp(-127, 127)
        y = b.double() / torch.exp2(e.double()).unsqueeze(-1)          # exact: a power-of-two scale
        a = y.abs()
        code = torch.bucketize(a, mid, right=False).to(torch.uint8)    # midpoints below a
        code += torch.isin(a, up).to(torch.uint8)                      # ties go to the even code
        code = code | ((y < 0) & (code > 0)).to(torch.uint8) << 3
        codes[i:i + chunk_blocks] = code[:, 0::2] | (code[:, 1::2] << 4)
        scales[i:i + chunk_blocks] = (e + 127).to(torch.uint8)
    return codes.reshape(*lead, D // 2), scales.reshape(*lead, D // 32)


def make_fp4(w: Workload):
    """MXFP4 encodings of a workload's q, k and v, and a copy of the workload
    holding their dequantised values.  Returns (((q codes, q scales), ...),
    dequantised workload)."""
    from dataclasses import replace
    enc = [to_mxfp4(x) for x in (w.q, w.k, w.v)]
    deq = replace(w, q=enc[0][2], k=enc[1][2], v=enc[2][2], dtype="bf16")
    return tuple((c, s) for c, s, _ in enc), deq


def make_config(name: str, seed: int = 0, **overrides) -> Workload:
    """Draw one of the named workloads in CONFIGS (fields may be overridden)."""
    c = dict(CONFIGS[name])
    c.update(overrides)
    return make(c["B"], c["H"], c["F"], c["N"], c["D"], c["D"], dtype=c["dtype"],
                seed=seed, s0_std=c["s0_std"], name=name)


def to_torch(w: Workload, device="cuda", *, with_s0: bool = True):
    """Device tensors in the library's layouts: (q, k, v, beta, alpha, S0-or-None)."""
    import torch
    io = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def dev(x, dt):
        return torch.from_numpy(np.ascontiguousarray(x)).to(device=device).to(dt).contiguous()

    S0 = dev(w.S0, torch.float32) if (with_s0 and w.S0 is not None) else None
    return (dev(w.q, io), dev(w.k, io), dev(w.v, io), dev(w.beta, torch.float32),
            dev(w.alpha, torch.float32), S0)


@dataclass
class BlockWorkload:
    """Hidden states and projection weights of one GDN block (all float32
    arrays holding bfloat16 values exactly)."""
    B: int
    F: int
    N: int
    C: int
    H: int
    D: int
    x: np.ndarray        # [B,F,N,C]
    w_qkv: np.ndarray    # [3,H,D,C]  (weights output-major: one row of inputs per output)
    w_gate: np.ndarray   # [2,H,C]    (beta rows, then alpha rows)
    w_out: np.ndarray    # [C,H*D]


def make_block(B: int, F: int, N: int, C: int, H: int, D: int, *, seed: int = 0,
               frame_share: float = 1.0) -> BlockWorkload:
    """Seeded hidden states and weights for the block projections.

    Recipe (``default_rng((seed, 3))``, float32 standard normals in C order,
    drawn in this order): a per-frame component s [B,F,1,C], token noise
    [B,F,N,C], w_qkv [3,H,D,C], w_gate [2,H,C], w_out [C,H*D].
    x = frame_share * s + noise (tokens of one latent frame share content, so
    the frame-mean decay logits are not all near zero); the weights are scaled
    by 1/sqrt(fan-in) (C, or H*D for w_out).  Everything is rounded to bf16.
    """
    rng = np.random.default_rng((seed, 3))
    s = rng.standard_normal((B, F, 1, C), dtype=np.float32)
    noise = rng.standard_normal((B, F, N, C), dtype=np.float32)
    x = noise + np.float32(frame_share) * s
    w_qkv = rng.standard_normal((3, H, D, C), dtype=np.float32) * np.float32(1.0 / np.sqrt(C))
    w_gate = rng.standard_normal((2, H, C), dtype=np.float32) * np.float32(1.0 / np.sqrt(C))
    w_out = rng.standard_normal((C, H * D), dtype=np.float32) * np.float32(1.0 / np.sqrt(H * D))
    return BlockWorkload(B, F, N, C, H, D, round_bf16(x), round_bf16(w_qkv), round_bf16(w_gate),
                         round_bf16(w_out))
