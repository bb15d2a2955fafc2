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
