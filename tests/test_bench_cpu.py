"""Host logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte count of the
roofline, and the rule that counter-measured traffic is reported only for the kernel
sources it was measured on."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from moe_layer_persistent_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_algorithmic_bytes_of_the_sliding_window_layer():
    """The step's bytes written out from the layer's shapes: bf16 dense weights (2 B per
    element), NVFP4 experts (0.5 B per code + 1 B per 16-element scale) per distinct expert,
    the keys and values of the window (2,048 + 15 positions) and x, y and the KV writes."""
    w = synth.WORKLOADS["swa_fp4"]
    H, P, I = 8192, 4096, 4096
    dense = 2 * ((64 + 16) * 128 * H + H * 64 * 128 + 256 * H + P * H + H * P + 2 * H)
    per_expert = (2 * I * P + P * I) // 2 + (2 * I * P + P * I) // 16
    kv = (2048 + 15) * 8 * 128 * 2 * 2
    io = 16 * H * 4 * 2 + 16 * 8 * 128 * 2 * 2
    idx = np.arange(16 * 8).reshape(16, 8) % 104           # 104 distinct experts
    got, U = bench.algorithmic_bytes(w, idx, w.pos, 2048, 16)
    assert U == 104
    assert got == dense + 104 * per_expert + kv + io
    # global attention reads every cached key and the step's own
    g = synth.WORKLOADS["global_fp4"]
    got_g, _ = bench.algorithmic_bytes(g, idx, g.pos, 0, 16)
    assert got_g - got == (g.pos + 16 - (2048 + 15)) * 8 * 128 * 2 * 2


def test_counter_traffic_only_for_the_sources_it_was_measured_on(monkeypatch):
    path = os.path.join(ROOT, "profiles", "k_layer_fused_swa_fp4_traffic.txt")
    kv = dict(line.split(":", 1) for line in open(path) if ":" in line and not line.startswith((" ", "#")))
    digest = kv["source_sha256"].strip()
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: digest)
    t = bench.measured_traffic("swa_fp4")
    assert t is not None and t["bytes_per_launch"] == float(kv["traffic_bytes_per_launch"])
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 64)
    assert bench.measured_traffic("swa_fp4") is None


def test_batched_algorithmic_bytes_add_each_requests_window():
    import numpy as np
    w = synth.WORKLOADS["swa_fp4"]
    idx = np.arange(16 * w.top_k).reshape(16, w.top_k) % w.n_experts
    one, U = bench.algorithmic_bytes(w, idx, 2048, w.window, 16)
    reqs = [(4, 2048, r * 2052, 2052) for r in range(4)]
    four, U4 = bench.algorithmic_bytes(w, idx, 0, w.window, 0, requests=reqs)
    kv_row = w.n_kv_heads * w.head_dim * 2 * 2          # one key and one value of every kv head
    # one request at history 2048 reads 2048 - 1 + 16 rows, each of four reads 2048 - 1 + 4
    assert U == U4
    assert four - one == kv_row * (4 * (2047 + 4) - (2047 + 16))
