"""bench.py on the CPU: it refuses more than one GPU before touching any
device, and its algorithmic work counts follow their definitions (KV-read
bytes 4·H·D·L per request-layer-step with L = P + min(t + 1, W), prefill
flops 4·H·D·P(P+1)/2 per request-layer)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_work_counts():
    import bench
    from kv_cache_management_amd import workloads as W

    w = W.Workload(9, "t", layers=2, heads=3, head_dim=64, dtype="bf16", prefill_lens=(5, 0, 130),
                   window=4, decode_steps=3, input_std=1.0)
    # visible keys before the step's write: P + min(t + 1, W)
    assert bench.visible_keys(5, 0, 4) == 6 and bench.visible_keys(5, 3, 4) == 9
    assert bench.visible_keys(5, 10, 4) == 9 and bench.visible_keys(0, 0, 4) == 1
    # standard window: the newest min(W, P + t + 1) positions only
    assert bench.visible_keys(130, 0, 4, "swa") == 4 and bench.visible_keys(0, 1, 4, "swa") == 2
    t = [0, 2, 7]
    want = sum(4 * 3 * 64 * (p + min(ti + 1, 4)) for p, ti in zip((5, 0, 130), t))
    assert bench.kv_bytes_per_layer_step(w, t) == want
    assert bench.prefill_flops(w) == 2 * sum(4 * 3 * 64 * p * (p + 1) // 2 for p in (5, 0, 130))
