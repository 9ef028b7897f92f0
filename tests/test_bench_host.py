"""Host-side checks of bench.py: its algorithmic byte and flop counts against
the figures worked out from the method's own steps, and its refusal of more
than one GPU.  No GPU needed."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bytes_per_query_head():
    # Q, K, V read once (bf16: 2 B x 64 each), out written once (fp32: 4 B x 64)
    for name in ("deit-t", "deit-s", "hires-3136", "long-16k"):
        assert bench.algorithmic(synth.workload(name))["bytes_per_qh"] == 3 * 64 * 2 + 64 * 4
    assert bench.algorithmic(synth.workload("tiny-fp32"))["bytes_per_qh"] == 4 * 64 * 4


def test_flops_per_query_head():
    # 2d each for S, V_L, q.Q_L and P.V_L per landmark, 2d each for q.K and P.V per routed key
    assert bench.algorithmic(synth.workload("deit-s"))["flops_per_qh"] == 4 * 64 * (2 * 25 + 25) == 19200
    assert bench.algorithmic(synth.workload("hires-3136"))["flops_per_qh"] == 4 * 64 * (2 * 49 + 64) == 41472


def test_kernel_counts_add_up():
    w = synth.workload("hires-3136")
    a = bench.algorithmic(w)
    BH, N, d, m, k = w["B"] * w["H"], 3136, 64, 49, 64
    f = a["kernel_flops"]
    # the staged kernels' matrix work: S + V_L, routing, expert attention
    assert f["landmark"] == BH * 4 * m * N * d
    assert f["route"] == BH * 2 * N * m * d
    assert f["attend"] == BH * 4 * N * d * (m + k)
    # the per-query-head count covers the same contractions (routing's logits
    # are the shared logits reused)
    assert f["landmark"] + f["attend"] == a["qh"] * a["flops_per_qh"]
    ws = synth.workload("deit-s")
    assert bench.algorithmic(ws)["kernel_bytes"]["fused"] == ws["B"] * ws["H"] * 196 * 640


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
