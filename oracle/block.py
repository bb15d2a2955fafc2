"""fp64 CPU oracle of the projections either side of the scan in a GDN block.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg call it.

"NVIDIA's New 2.6B World Model Generates Minute-Scale 720p Video on a Single
GPU" (section "The Architecture: Replacing Softmax Attention at Scale") places
the frame-wise GDN layer inside the transformer blocks of a hybrid backbone but
does not give the block's projections.  This follows the plain reading of a
linear attention block: bias-free linear maps from the hidden states to q, k,
v and the gate logits, one beta logit per token and one decay logit per frame
(the decay gate is per frame in the scan), the latter taken from the mean of
the frame's tokens; and a linear map from the scan's output back to the model
width.  Parity unpinned beyond the matrix products themselves: the pages fix
no weights, biases, activations or normalisations of this block, so the pins
check the products and the pooling, not the block's design.

numpy's matmul in float64 does the products; nothing is blocked or fused.
"""
from __future__ import annotations

import numpy as np


def block_in_proj(x, w_qkv, w_gate):
    """x [B,F,N,C], w_qkv [3,H,D,C], w_gate [2,H,C] (weights stored output-major,
    one row of C inputs per output) -> (q, k, v [B,F,N,H,D], beta_logit
    [B,F,N,H], alpha_logit [B,F,H]), float64."""
    x = np.asarray(x, dtype=np.float64)
    w_qkv = np.asarray(w_qkv, dtype=np.float64)
    w_gate = np.asarray(w_gate, dtype=np.float64)
    B, F, N, C = x.shape
    if w_qkv.ndim != 4 or w_qkv.shape[0] != 3 or w_qkv.shape[3] != C or w_gate.shape[0] != 2 \
            or w_gate.shape[2] != C:
        raise ValueError("weight shapes disagree with x")
    H, D = w_qkv.shape[1], w_qkv.shape[2]
    if w_gate.shape[1] != H:
        raise ValueError("w_gate head count disagrees with w_qkv")
    rows = x.reshape(B * F * N, C)
    qkv = (rows @ w_qkv.reshape(3 * H * D, C).T).reshape(B, F, N, 3, H, D)
    gates = (rows @ w_gate.reshape(2 * H, C).T).reshape(B, F, N, 2, H)
    beta_logit = gates[:, :, :, 0, :]
    if N > 0:
        alpha_logit = gates[:, :, :, 1, :].mean(axis=2)
    else:
        alpha_logit = np.zeros((B, F, H))
    return qkv[:, :, :, 0], qkv[:, :, :, 1], qkv[:, :, :, 2], beta_logit, alpha_logit


def block_out_proj(o, w_out):
    """o [B,F,N,H,D], w_out [C,H*D] (output-major) -> y [B,F,N,C], float64."""
    o = np.asarray(o, dtype=np.float64)
    w_out = np.asarray(w_out, dtype=np.float64)
    B, F, N, H, D = o.shape
    if w_out.ndim != 2 or w_out.shape[1] != H * D:
        raise ValueError("w_out columns must equal H*D")
    return (o.reshape(B * F * N, H * D) @ w_out.T).reshape(B, F, N, w_out.shape[0])
