#!/usr/bin/env python3
"""Benchmark of the frame-wise GDN forward scan on one MI355X.

One step is one gdn_frame_scan_fwd call over the whole workload (every frame,
head and batch item), with inputs already resident in HBM.  Prints one JSON
line: throughput in tokens/s from a clean timed region of K steps, the
roofline of the dominant kernel (HIP events recorded by the library around
every launch in a second timed region of K steps), and the fp64 CPU oracle
timed on a bounded sample of the same workload; also the per-step GPU time of
gdn_frame_step at the streaming workload's shape.

    python bench.py [--steps K] [--warmup W] [--workload full_minute]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN scan tokens/s (121 frames×880 tok, 16h×d128, bf16) + % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, published
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


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle on the first F_s frames of every (b, h) of the workload."""
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
    return {"value": w.B * fs * w.N / dt, "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": "first %d of %d frames, all %d (b,h) units, %d tokens/frame: %.2f s"
                      % (fs, w.F, w.B * w.H, w.N, dt)}


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
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0: skip)")
    ap.add_argument("--stream-frames", type=int, default=16,
                    help="frames of the streaming-step measurement (0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES bytes --steps times")
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed(profiled: bool):
        # K steps bracketed by synchronisation; with `profiled` the library
        # also records a HIP event pair around every kernel launch (on the
        # launch stream), which adds a few microseconds between kernels
        if profiled:
            api.profile_begin()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern = api.profile_end() if profiled else None
        return ev0.elapsed_time(ev1), wall, kern

    # throughput from a clean timed region; per-kernel durations from a second
    # timed region of the same K steps with per-launch events
    gpu_ms, wall, _ = timed(False)
    prof_ms, _, kern = timed(True)
    ms_per_step = gpu_ms / args.steps

    total_bytes, per_kernel_bytes, flops, flops_kernel = algorithmic(w)
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
                "kernel": dom, "alg_bytes_per_launch": int(dom_bytes)}
    path_gbs = total_bytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded Gaussians in the workload's shapes; no trained weights)",
        "config": {"workload": args.workload, "B": w.B, "H": w.H, "F": w.F, "N": w.N, "Dk": w.Dk,
                   "Dv": w.Dv, "seed": args.seed, "state": "fp32"},
        "roofline": roofline,
        "path_roofline": {"bound": "hbm", "alg_bytes_per_step": total_bytes,
                          "achieved": round(path_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(path_gbs / HBM_PEAK_GBS, 4),
                          "mfma_frac": round(flops / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
                          "alg_flops_per_step": flops},
        "frame_steps_per_s": round(w.B * w.F / (ms_per_step * 1e-3), 1),
        "head_frame_steps_per_s": round(w.B * w.H * w.F / (ms_per_step * 1e-3), 1),
        "kernels": kernels,
        "wall_s_timed": round(wall, 4),
        "kernel_timing": "HIP events around each launch, separate timed region of the same %d steps "
                         "(%.5f ms per step with the events)" % (args.steps, prof_ms / args.steps),
        "kernel_src": src_hash,
    }
    line["streaming_step"] = streaming_step(args.stream_frames) if args.stream_frames > 0 else None
    if args.cpu_budget > 0:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line))


if __name__ == "__main__":
    main()
