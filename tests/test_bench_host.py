"""bench.py's host-side contract, without a GPU: more than one GPU is refused
with a message, and the algorithmic byte and flop counts of the full-minute
workload are the ones its roofline figures divide by."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU per process" in r.stderr and "--gpus 2" in r.stderr


def test_algorithmic_counts():
    # full-minute workload (B1 H16 F121 N880 d128, bf16): q, k, v, o at
    # 1*121*880*16 tokens x 128 values x 2 bytes = 436,142,080 bytes each;
    # beta 4 bytes per token and head, alpha 4 per frame and head; S0 and
    # S_F 16 x 128 x 128 x 4 bytes each
    import types
    import bench
    w = types.SimpleNamespace(B=1, H=16, F=121, N=880, Dk=128, Dv=128, dtype="bf16")
    total, per, flops, per_flops = bench.algorithmic(w)
    qkvo = 436_142_080
    assert per["frame_gram"] == 2 * qkvo + 1 * 121 * 880 * 16 * 4 + 121 * 16 * 4 == 879_106_624
    assert per["frame_output"] == 2 * qkvo
    assert per["state_scan"] == 2 * 16 * 128 * 128 * 4
    assert total == 1_753_487_936
    units = 121 * 16
    assert per_flops["frame_gram"] == units * 4 * 880 * 128 * 128      # G and U: 2 N D^2 each
    assert per_flops["frame_output"] == units * 2 * 880 * 128 * 128    # O = Q S^T
    assert per_flops["state_scan"] == units * 2 * 128 * 128 * 128      # S G
    assert flops == sum(per_flops.values())
