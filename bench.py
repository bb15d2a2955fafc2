#!/usr/bin/env python3
"""Benchmark of the frame-wise GDN forward scan on one MI355X.

One step is one gdn_frame_scan_fwd call over the whole workload (every frame,
head and batch item), with inputs already resident in HBM.  Prints one JSON
line: throughput in tokens/s from a clean timed region of K steps, the
roofline of the dominant kernel (HIP events recorded by the library around
every launch in a second timed region of K steps), and the fp64 CPU oracle
timed on a bounded sample of the same workload; also the per-step GPU time of
gdn_frame_step at the streaming workload's shape and the backward pass
(gdn_frame_scan_bwd) and of the block-scaled input modes
(gdn_frame_scan_fwd_fp8, gdn_frame_scan_fwd_fp4) on the same workload.

    python bench.py [--steps K] [--warmup W] [--workload full_minute]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN scan tokens/s (121 frames×880 tok, 16h×d128, bf16) + % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, published
# the sources of the forward kernels and their launches (the backward-only
# kernel in gdn_bwd.hpp does not change what the forward's counters measured)
CSRC = ["gated_deltanet_scan_amd/csrc/gdn_kernels.hpp", "gated_deltanet_scan_amd/csrc/gdn_api.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in CSRC:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic(w):
    """Algorithmic bytes and flops of the whole scan and of each kernel.

    Bytes: read q, k, v, beta, alpha and S0 once, write o and S_final once.
    Per kernel, the same bytes split by which kernel must move them:
    frame_gram k, v, beta, alpha; frame_output q, o; state_scan S0, S_final.
    Flops (Gram form, per (b, h, f)): 6*N*Dk*Dv + 2*Dv*Dk^2.
    """
    esz = 2 if w.dtype == "bf16" else 4
    units = w.B * w.H * w.F
    tok = w.B * w.F * w.N * w.H
    qkvo = tok * w.Dk * esz
    state = w.B * w.H * w.Dv * w.Dk * 4
    per = {
        "frame_gram": 2 * qkvo + tok * 4 + w.B * w.F * w.H * 4,
        "frame_output": 2 * qkvo,
        "state_scan": 2 * state,
    }
    flops = units * (6 * w.N * w.Dk * w.Dv + 2 * w.Dv * w.Dk * w.Dk)
    flops_kernel = {
        "frame_gram": units * 4 * w.N * w.Dk * w.Dv,
        "frame_output": units * 2 * w.N * w.Dk * w.Dv,
        "state_scan": units * 2 * w.Dv * w.Dk * w.Dk,
    }
    return sum(per.values()), per, flops, flops_kernel


def load_traffic(kernel: str, workload: str, src_hash: str, launches_per_step: int):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    the counters were taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "counters_%s_%s.json" % (kernel, workload))
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        c = json.load(fh)
    if c.get("src_hash") != src_hash:
        return None
    return c.get("hbm_bytes_per_launch")


def oracle_timing(w, budget_s: float):
    """The fp64 oracle on the first F_s frames of every (b, h) of workload w,
    F_s chosen so the run takes about budget_s seconds: (tokens/s, F_s, s)."""
    import numpy as np
    import oracle
    sl = lambda x, n: np.ascontiguousarray(x[:, :n])
    # calibrate on one frame, then take as many frames as fit the budget
    t = time.perf_counter()
    oracle.scan(sl(w.q, 1), sl(w.k, 1), sl(w.v, 1), sl(w.beta, 1), sl(w.alpha, 1), w.S0)
    t1 = max(time.perf_counter() - t, 1e-6)
    fs = int(max(1, min(w.F, budget_s / t1)))
    args = (sl(w.q, fs), sl(w.k, fs), sl(w.v, fs), sl(w.beta, fs), sl(w.alpha, fs), w.S0)
    t = time.perf_counter()
    oracle.scan(*args)
    dt = time.perf_counter() - t
    return w.B * fs * w.N / dt, fs, dt


def cpu_model() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return "unknown"


def single_thread_runs(budget_s: float):
    """The oracle on one thread (a child process with OMP_NUM_THREADS=1) on the
    tiny fp32 workload (whole) and on a bounded sample of the short clip."""
    code = ("import json, sys; sys.path.insert(0, %r); import bench, oracle;"
            "from gated_deltanet_scan_amd import inputs; out = {};"
            "[out.__setitem__(n, bench.oracle_timing(inputs.make_config(n), %r))"
            " for n in ('tiny_fp32', 'short_clip')];"
            "out['threads'] = oracle.max_threads(); print(json.dumps(out))") % (ROOT, budget_s)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    if r.returncode != 0:
        return {"error": r.stderr[-300:]}
    res = json.loads(r.stdout.strip().splitlines()[-1])
    out = {"threads": res.pop("threads")}
    for name, (tps, fs, dt) in res.items():
        out[name] = {"tokens_per_s": round(tps, 1), "frames": fs, "seconds": round(dt, 3)}
    return out


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle on the first F_s frames of every (b, h) of the workload,
    on every host core, plus one-thread runs of the two small workloads."""
    import oracle
    tps, fs, dt = oracle_timing(w, budget_s)
    return {"value": tps, "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": "first %d of %d frames, all %d (b,h) units, %d tokens/frame: %.2f s"
                      % (fs, w.F, w.B * w.H, w.N, dt),
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "single_thread": single_thread_runs(min(budget_s, 5.0))}


def measured_peaks():
    """What this GPU reaches on plain work, as a second yardstick next to the
    published peaks: a 1 GiB device-to-device copy (torch copy_, bytes read
    plus written per second) and a 8192^3 bf16 matrix product (torch.matmul,
    hipBLASLt).  Run after the timed regions: the products draw enough power
    to slow a scan timed right after them."""
    import torch
    n = 1 << 28
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)

    def best(fn, reps):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)

    t_copy = best(lambda: y.copy_(x), 20)
    t_mm = best(lambda: torch.matmul(a, b), 10)
    del x, y, a, b
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * 4 * n / t_copy / 1e9, 1),
            "gemm_bf16_tfs": round(2 * 8192 ** 3 / t_mm / 1e12, 1),
            "how": "best of 20 copies of 1 GiB (read + write bytes) and of 10 bf16 8192^3 "
                   "torch.matmul, HIP events"}


def streaming_step(frames: int, reps: int = 40, warm: int = 10):
    """gdn_frame_step at the streaming workload's shape (B4 H32 d64 N880, bf16,
    fp32 state): `frames` consecutive steps captured in one HIP graph and
    replayed, so the figure is GPU time per step without the Python call
    overhead.  Timed twice: with the state alternating between two buffers
    (S_out of one step is S_in of the next; the one-launch path) and carried
    in place in one buffer (S_out == S_in; the two-launch path).  Inputs are
    seeded Gaussians drawn on the device in the workload's distributions
    (timing does not depend on the values)."""
    import torch
    from gated_deltanet_scan_amd import api
    B, H, N, D = 4, 32, 880, 64
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    mk = lambda *sh: torch.randn(*sh, device="cuda", generator=g)
    q = [mk(B, N, H, D).bfloat16() for _ in range(frames)]
    k = []
    for _ in range(frames):
        kk = mk(B, N, H, D)
        k.append((kk / kk.norm(dim=-1, keepdim=True)).bfloat16())
    v = [mk(B, N, H, D).bfloat16() for _ in range(frames)]
    beta = [torch.sigmoid(mk(B, N, H)) / N for _ in range(frames)]
    alpha = [torch.sigmoid(mk(B, H) + 3.0) for _ in range(frames)]
    o = [torch.empty_like(q[0]) for _ in range(frames)]
    S = [torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda") for _ in range(2)]
    desc = api.make_desc(B, H, 1, N, D, torch.bfloat16)
    ws = api.alloc_workspace(desc, q[0].device)
    cs = torch.cuda.Stream()

    def timed(nbuf: int) -> float:
        def run():
            for f in range(frames):
                api.frame_step(q[f], k[f], v[f], beta[f], alpha[f], S[f % nbuf], o=o[f],
                               S_out=S[(f + 1) % nbuf], workspace=ws, stream=cs)
        with torch.cuda.stream(cs):
            run()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=cs):
                run()
        torch.cuda.synchronize()
        for _ in range(warm):
            graph.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * frames) * 1e3

    us = timed(2)
    us_in_place = timed(1)
    # q, k, v read and o written (bf16), beta and alpha read, S read and written
    nbytes = B * N * H * D * 2 * 4 + B * N * H * 4 + B * H * 4 + 2 * B * H * D * D * 4
    return {"workload": "streaming (B4 H32 d64 N880, one frame per gdn_frame_step)", "us_per_step": round(us, 2),
            "us_per_step_in_place": round(us_in_place, 2),
            "frames_timed": frames * reps, "alg_bytes_per_step": nbytes,
            "hbm_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "timing": "HIP graph of %d consecutive steps, replayed %d times after %d; state in two "
                      "alternating buffers (in place: one buffer)" % (frames, reps, warm)}


def backward(w, q, k, v, beta, alpha, S0, steps: int, warmup: int, flush_buf):
    """gdn_frame_scan_bwd on the workload: one step is one call (forward
    states recomputed, all six gradients written), inputs resident in HBM.
    Algorithmic bytes: read q, k, v, dO, beta, alpha, S0 and dS_final once,
    write dq, dk, dv, dbeta, dalpha and dS0 once."""
    import torch
    from gated_deltanet_scan_amd import api, inputs
    dO_np, dS_np = inputs.make_grads(w, seed=0)
    io = q.dtype
    dO = torch.from_numpy(dO_np).cuda().to(io)
    dS = torch.from_numpy(dS_np).cuda()
    desc = api.make_desc(w.B, w.H, w.F, w.N, w.Dk, io)
    ws = torch.empty(api.workspace_size_bwd(desc), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        return api.frame_scan_bwd(q, k, v, beta, alpha, dO, S0, dS, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    def timed(profiled):
        if profiled:
            api.profile_begin()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps if flush_buf is not None else 1)]
        torch.cuda.synchronize()
        if flush_buf is not None:
            for e0, e1 in ev:
                flush_buf.fill_(1.0)
                e0.record(stream)
                step()
                e1.record(stream)
        else:
            ev[0][0].record(stream)
            for _ in range(steps):
                step()
            ev[0][1].record(stream)
        torch.cuda.synchronize()
        kern = api.profile_end() if profiled else None
        return sum(e0.elapsed_time(e1) for e0, e1 in ev), kern

    gpu_ms, _ = timed(False)
    _, kern = timed(True)
    ms = gpu_ms / steps
    esz = 2 if w.dtype == "bf16" else 4
    tok = w.B * w.F * w.N * w.H
    state = w.B * w.H * w.Dv * w.Dk * 4
    nbytes = 7 * tok * w.Dk * esz + 2 * tok * 4 + 2 * w.B * w.F * w.H * 4 + 3 * state
    kernels = {name: {"avg_ms": round(t / n, 5), "launches_per_step": n / steps}
               for name, (t, n) in kern.items() if n > 0}
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"workload": "the same workload, gdn_frame_scan_bwd", "ms_per_step": round(ms, 5),
           "tokens_per_s": round(w.B * w.F * w.N / (ms * 1e-3), 1),
           "alg_bytes_per_step": nbytes, "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
           "kernels": kernels, "steps": steps, "warmup": warmup,
           "timing": "HIP events around %d calls (per-kernel figures from a second region with "
                     "per-launch events)" % steps}
    del ws
    out["saved_states"] = saved_states(w, q, k, v, beta, alpha, S0, dO, dS, steps, warmup, ms)
    return out


def saved_states(w, q, k, v, beta, alpha, S0, dO, dS, steps: int, warmup: int, recompute_ms: float):
    """The training pair with saved states: gdn_frame_scan_fwd_save (the
    forward that keeps every frame's operands) and gdn_frame_scan_bwd_saved
    (the backward that reads them), each timed by HIP events over `steps`
    calls, beside the recomputing backward's time."""
    import torch
    from gated_deltanet_scan_amd import api
    desc = api.make_desc(w.B, w.H, w.F, w.N, w.Dk, q.dtype)
    saved = torch.empty(api.saved_size(desc), dtype=torch.uint8, device="cuda")
    ws = torch.empty(api.workspace_size_bwd_saved(desc), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    S_final = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def fwd():
        api.frame_scan_fwd_save(q, k, v, beta, alpha, S0, o=o, S_final=S_final, saved=saved, stream=stream)

    def bwd():
        api.frame_scan_bwd(q, k, v, beta, alpha, dO, None, dS, saved=saved, workspace=ws, stream=stream)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    fwd_ms = timed(fwd)
    fwd()
    bwd_ms = timed(bwd)
    return {"fwd_save_ms": round(fwd_ms, 5), "bwd_saved_ms": round(bwd_ms, 5),
            "bwd_speedup_vs_recompute": round(recompute_ms / bwd_ms, 3),
            "saved_bytes": int(saved.numel()), "bwd_workspace_bytes": int(ws.numel()),
            "timing": "HIP events around %d calls of each" % steps}


def mx_inputs(fmt: str, w, q, k, v, beta, alpha, S0, steps: int, warmup: int, flush_buf, bf16_ms: float):
    """gdn_frame_scan_fwd_fp8 (fmt "fp8") or gdn_frame_scan_fwd_fp4 (fmt
    "fp4") on the workload with q, k and v encoded on the device in the OCP
    microscaling layout (E4M3 or E2M1 values, one E8M0 scale per 32
    features); o in bf16.  Algorithmic bytes: q, k, v at one byte (fp8) or
    half a byte (fp4) per value plus their scales, beta, alpha and S0 read
    once, o (bf16) and S_final written once."""
    import torch
    from gated_deltanet_scan_amd import api, inputs
    enc = [(inputs.to_mxfp8_device if fmt == "fp8" else inputs.to_mxfp4_device)(x) for x in (q, k, v)]
    fn = api.frame_scan_fwd_fp8 if fmt == "fp8" else api.frame_scan_fwd_fp4
    o = torch.empty((w.B, w.F, w.N, w.H, w.Dv), dtype=torch.bfloat16, device="cuda")
    S_final = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device="cuda")
    desc = api.make_desc(w.B, w.H, w.F, w.N, w.Dk, torch.bfloat16)
    ws = api.alloc_workspace(desc, q.device)          # the same size in every input format
    stream = torch.cuda.current_stream()

    def step():
        fn(enc[0][0], enc[0][1], enc[1][0], enc[1][1], enc[2][0], enc[2][1], beta, alpha, S0,
           o=o, S_final=S_final, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    def timed(profiled):
        if profiled:
            api.profile_begin()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps if flush_buf is not None else 1)]
        torch.cuda.synchronize()
        if flush_buf is not None:
            for e0, e1 in ev:
                flush_buf.fill_(1.0)
                e0.record(stream)
                step()
                e1.record(stream)
        else:
            ev[0][0].record(stream)
            for _ in range(steps):
                step()
            ev[0][1].record(stream)
        torch.cuda.synchronize()
        kern = api.profile_end() if profiled else None
        return sum(e0.elapsed_time(e1) for e0, e1 in ev), kern

    gpu_ms, _ = timed(False)
    _, kern = timed(True)
    ms = gpu_ms / steps
    tok = w.B * w.F * w.N * w.H
    state = w.B * w.H * w.Dv * w.Dk * 4
    code_bytes = 3 * tok * w.Dk if fmt == "fp8" else 3 * tok * w.Dk // 2
    nbytes = code_bytes + 3 * tok * (w.Dk // 32) + tok * w.Dv * 2 + tok * 4 + w.B * w.F * w.H * 4 + 2 * state
    gbs = nbytes / (ms * 1e-3) / 1e9
    kernels = {name: {"avg_ms": round(t / n, 5), "launches_per_step": n / steps}
               for name, (t, n) in kern.items() if n > 0}
    name = "MXFP8 (E4M3" if fmt == "fp8" else "MXFP4 (E2M1, two per byte"
    return {"workload": "the same workload, q/k/v as %s, E8M0 scale per 32 features), o bf16" % name,
            "ms_per_step": round(ms, 5), "tokens_per_s": round(w.B * w.F * w.N / (ms * 1e-3), 1),
            "speedup_vs_bf16": round(bf16_ms / ms, 3), "alg_bytes_per_step": nbytes,
            "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "kernels": kernels,
            "steps": steps, "warmup": warmup}


def block_projections(w, steps: int, warmup: int, C: int, seed: int):
    """The GDN block around the scan on the same (B, F, N, H, D): input
    projections from hidden states of width C (gdn_block_in_proj), the scan on
    the gate logits they produce, and the output projection
    (gdn_block_out_proj).  Hidden states and weights are seeded device
    Gaussians (weights scaled by 1/sqrt(fan-in)) rounded to bf16.  Each part is
    timed by its own HIP events over `steps` calls; the GEMM rates are the
    algorithmic 2*M*N*K flops over those times."""
    import torch
    from gated_deltanet_scan_amd import api
    g = torch.Generator(device="cuda").manual_seed(seed)
    B, F, N, H, D = w.B, w.F, w.N, w.H, w.Dk
    dev = dict(device="cuda", dtype=torch.float32, generator=g)
    x = (torch.randn((B, F, 1, C), **dev) + torch.randn((B, F, N, C), **dev)).to(torch.bfloat16)
    w_qkv = (torch.randn((3, H, D, C), **dev) / C ** 0.5).to(torch.bfloat16)
    w_gate = (torch.randn((2, H, C), **dev) / C ** 0.5).to(torch.bfloat16)
    w_out = (torch.randn((C, H * D), **dev) / (H * D) ** 0.5).to(torch.bfloat16)
    q, k, v = [torch.empty((B, F, N, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    bl = torch.empty((B, F, N, H), dtype=torch.float32, device="cuda")
    al = torch.empty((B, F, H), dtype=torch.float32, device="cuda")
    o = torch.empty_like(q)
    y = torch.empty((B, F, N, C), dtype=torch.bfloat16, device="cuda")
    bws = torch.empty(api.block_workspace_size(B, H, F, N, D, C), dtype=torch.uint8, device="cuda")
    desc = api.make_desc(B, H, F, N, D, torch.bfloat16, gates_are_logits=True)
    sws = api.alloc_workspace(desc, q.device)
    stream = torch.cuda.current_stream()
    parts = {
        "in_proj": lambda: api.block_in_proj(x, w_qkv, w_gate, H=H, D=D, q=q, k=k, v=v, beta_logit=bl,
                                             alpha_logit=al, workspace=bws, stream=stream),
        "scan": lambda: api.frame_scan_fwd(q, k, v, bl, al, None, gates_are_logits=True, o=o, workspace=sws,
                                           return_state=False, stream=stream),
        "out_proj": lambda: api.block_out_proj(o, w_out, y=y, workspace=bws, stream=stream),
    }
    for _ in range(warmup):
        for fn in parts.values():
            fn()
    torch.cuda.synchronize()
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
          for n in parts}
    for i in range(steps):
        for n, fn in parts.items():
            ev[n][i][0].record(stream)
            fn()
            ev[n][i][1].record(stream)
    torch.cuda.synchronize()
    ms = {n: sum(a.elapsed_time(b) for a, b in ev[n]) / steps for n in parts}
    M = B * F * N
    flops = {"in_proj": 2 * M * C * (3 * H * D + 2 * H), "out_proj": 2 * M * H * D * C}
    total = sum(ms.values())
    out = {"workload": "the same (B, F, N, H, D) at model width C = %d: q/k/v and output projections as bf16 "
                       "GEMMs with fp32 accumulation (hipBLASLt), gate logits and frame means in the library's "
                       "own kernels, the scan on the gate logits" % C,
           "C": C, "ms_per_step": round(total, 5), "tokens_per_s": round(M / (total * 1e-3), 1),
           "steps": steps, "warmup": warmup}
    for n in parts:
        out[n] = {"ms": round(ms[n], 5)}
        if n in flops:
            tfs = flops[n] / (ms[n] * 1e-3) / 1e12
            out[n].update({"alg_flops": flops[n], "tflops": round(tfs, 1),
                           "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)})
    del x, q, k, v, o, y, bws, sws
    return out


def copy_calibration(nbytes: int, steps: int):
    """A plain device copy of known size, for scaling rocprofv3 byte counters."""
    import torch
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": steps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="full_minute")
    ap.add_argument("--settle-ms", type=float, default=40.0,
                    help="after the W warm-up steps, keep stepping (untimed) until this many "
                         "milliseconds have passed since the first warm-up step ended (0: off)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0: skip)")
    ap.add_argument("--stream-frames", type=int, default=16,
                    help="frames of the streaming-step measurement (0: skip)")
    ap.add_argument("--bwd-steps", type=int, default=20,
                    help="timed calls of the backward pass (0: skip)")
    ap.add_argument("--fp8-steps", type=int, default=20,
                    help="timed calls of each block-scaled input mode, MXFP8 and MXFP4 (0: skip)")
    ap.add_argument("--block-steps", type=int, default=10,
                    help="timed calls of the block around the scan: projections at model width "
                         "--block-width, the scan, the output projection (0: skip)")
    ap.add_argument("--block-width", type=int, default=2048)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES bytes --steps times")
    ap.add_argument("--flush", choices=["auto", "on", "off"], default="auto",
                    help="write a 1 GiB buffer before every timed step, so no input is left "
                         "in the 256 MB last-level cache (auto: when the workload moves less "
                         "than 1 GiB); each step is then timed by its own HIP events")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: the library runs on one GPU per process; --gpus %d is not supported "
              "(a scan would shard by (batch, head), with no communication between GPUs)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return

    import torch
    from gated_deltanet_scan_amd import api, inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    w = inputs.make_config(args.workload, seed=args.seed)
    q, k, v, beta, alpha, S0 = inputs.to_torch(w, "cuda")
    o = torch.empty_like(q)
    S_final = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device="cuda")
    desc = api.make_desc(w.B, w.H, w.F, w.N, w.Dk, q.dtype)
    ws = api.alloc_workspace(desc, q.device)
    stream = torch.cuda.current_stream()

    def step():
        api.frame_scan_fwd(q, k, v, beta, alpha, S0, o=o, S_final=S_final, workspace=ws,
                           stream=stream)

    total_bytes, per_kernel_bytes, flops, flops_kernel = algorithmic(w)
    flush = args.flush == "on" or (args.flush == "auto" and total_bytes < (1 << 30))
    junk = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if flush else None

    # (the first call loads the kernels' code; the settle clock starts after it)
    for i in range(args.warmup):
        step()
        if i == 0:
            torch.cuda.synchronize()
            t_settle = time.perf_counter()
    if args.warmup == 0:
        t_settle = time.perf_counter()
    torch.cuda.synchronize()
    # Clock settle.  A GPU that was idle runs the first milliseconds of this
    # load through a clock transient (every kernel slows alike, by up to a
    # quarter, from about 2 ms to about 15 ms into the load, then steadies);
    # a few warm-up steps end inside it.  So warm-up continues, whole steps,
    # until --settle-ms of wall time have passed since its first step ended;
    # the timed steps then see the steady clock.  Reported as "settle".
    settle_steps = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(4):
            step()
        settle_steps += 4
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3

    def timed(profiled: bool):
        # K steps bracketed by synchronisation; with `profiled` the library
        # also records a HIP event pair around every kernel launch (on the
        # launch stream), which adds a few microseconds between kernels.
        # With the flush, each step is timed by its own events and the 1 GiB
        # write before it is outside them.
        if profiled:
            api.profile_begin()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps if flush else 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if flush:
            for e0, e1 in ev:
                junk.fill_(1.0)
                e0.record(stream)
                step()
                e1.record(stream)
        else:
            ev[0][0].record(stream)
            for _ in range(args.steps):
                step()
            ev[0][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern = api.profile_end() if profiled else None
        return sum(e0.elapsed_time(e1) for e0, e1 in ev), wall, kern

    # throughput from a clean timed region; per-kernel durations from a second
    # timed region of the same K steps with per-launch events
    gpu_ms, wall, _ = timed(False)
    prof_ms, _, kern = timed(True)
    ms_per_step = gpu_ms / args.steps

    tokens = w.B * w.F * w.N
    value = tokens / (ms_per_step * 1e-3)

    kernels = {}
    for name, (ms, n) in kern.items():
        if n == 0:
            continue
        launches_per_step = n / args.steps
        avg_ms = ms / n
        b = per_kernel_bytes.get(name, 0) / launches_per_step
        kernels[name] = {"avg_ms": round(avg_ms, 5), "launches": n,
                         "share": round(ms / max(prof_ms, 1e-9), 4),
                         "alg_gbs": round(b / (avg_ms * 1e-3) / 1e9, 1)}
    dom = max(kernels, key=lambda n: kernels[n]["avg_ms"] * kernels[n]["launches"])
    dom_launches_per_step = kern[dom][1] / args.steps
    dom_bytes = per_kernel_bytes[dom] / dom_launches_per_step
    dom_avg_s = kernels[dom]["avg_ms"] * 1e-3
    achieved = dom_bytes / dom_avg_s / 1e9
    src_hash = kernel_source_hash()
    traffic = load_traffic(dom, args.workload, src_hash, dom_launches_per_step)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom, "alg_bytes_per_launch": int(dom_bytes),
                "scope": "the dominant kernel alone, on the bytes it must move; the whole "
                         "scan against the same peak is path_roofline"}
    path_gbs = total_bytes / (ms_per_step * 1e-3) / 1e9
    # measured after the timed regions: the 8192^3 products draw enough power
    # to slow the scan timed right after them
    peaks = measured_peaks()
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "settle": {"steps": settle_steps, "ms": round(settle_ms, 2),
                   "why": "untimed whole steps after the warm-up until --settle-ms have passed, so "
                          "that the timed steps run at the steady clock, not in the transient that "
                          "follows an idle GPU"},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded Gaussians in the workload's shapes; no trained weights)",
        "config": {"workload": args.workload, "B": w.B, "H": w.H, "F": w.F, "N": w.N, "Dk": w.Dk,
                   "Dv": w.Dv, "seed": args.seed, "state": "fp32"},
        "roofline": roofline,
        "path_roofline": {"bound": "hbm", "alg_bytes_per_step": total_bytes,
                          "achieved": round(path_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(path_gbs / HBM_PEAK_GBS, 4),
                          "mfma_frac": round(flops / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
                          "alg_flops_per_step": flops,
                          "frac_of_measured_copy": round(path_gbs / peaks["copy_gbs"], 4),
                          "mfma_frac_of_measured_gemm": round(
                              flops / (ms_per_step * 1e-3) / 1e12 / peaks["gemm_bf16_tfs"], 4),
                          "target": "frac >= 0.5 (ms_per_step <= %.4f)"
                                    % (total_bytes / (0.5 * HBM_PEAK_GBS * 1e9) * 1e3)},
        "measured_peaks": peaks,
        "llc_flush": flush,
        "frame_steps_per_s": round(w.B * w.F / (ms_per_step * 1e-3), 1),
        "head_frame_steps_per_s": round(w.B * w.H * w.F / (ms_per_step * 1e-3), 1),
        "kernels": kernels,
        "wall_s_timed": round(wall, 4),
        "kernel_timing": "HIP events around each launch, separate timed region of the same %d steps "
                         "(%.5f ms per step with the events)" % (args.steps, prof_ms / args.steps),
        "kernel_src": src_hash,
    }
    line["backward"] = (backward(w, q, k, v, beta, alpha, S0, args.bwd_steps, min(args.warmup, 5), junk)
                        if args.bwd_steps > 0 else None)
    for fmt in ("fp8", "fp4"):
        line[fmt + "_inputs"] = (mx_inputs(fmt, w, q, k, v, beta, alpha, S0, args.fp8_steps, min(args.warmup, 5),
                                           junk, ms_per_step)
                                 if args.fp8_steps > 0 and w.Dk % 32 == 0 and w.dtype == "bf16" else None)
    line["block"] = (block_projections(w, args.block_steps, min(args.warmup, 3), args.block_width, args.seed)
                     if args.block_steps > 0 and w.dtype == "bf16" else None)
    line["streaming_step"] = streaming_step(args.stream_frames) if args.stream_frames > 0 else None
    if args.cpu_budget > 0:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line))


if __name__ == "__main__":
    main()
