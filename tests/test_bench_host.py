"""Host logic of bench.py (no GPU): the one-GPU contract, the algorithmic byte
and flop counts the roofline divides by, the kernel names that tie the bench
line to the committed rocprofv3 summaries, and the source-hash gate on the
committed HBM traffic figures."""

import json
import os
import subprocess
import sys

import numpy as np

import bench
import bit_weight_quantized_qgemm_amd as qg
from synth import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_alg_bytes_and_flops_from_the_arrays():
    # the arrays the method reads and writes: packed 4-bit codes, one fp16 scale
    # per 128 k and column, fp16 A, fp16 C
    for (M, K, N) in [(1, 256, 64), (16, 1024, 192), (128, 2048, 256)]:
        p = gen.w4a16_problem(M, K, N, seed=1)
        moved = p["codes"].nbytes + p["scales"].nbytes + p["A"].nbytes + M * N * np.dtype(np.float16).itemsize
        assert bench.alg_bytes(M, K, N) == moved
        assert bench.alg_flops(M, K, N) == 2 * M * K * N
    # the metric's layer at M = 1: 117.4 MB of codes, 3.7 MB of scales
    assert bench.alg_bytes(1, 8192, 28672) == 8192 * 28672 // 2 + 64 * 28672 * 2 + 8192 * 2 + 28672 * 2


def test_every_sweep_kernel_is_named_in_the_committed_profiles():
    with open(os.path.join(ROOT, "profiles", "w4a16_sweep_70b_layer_kernel_stats.txt")) as f:
        stats = f.read()
    with open(os.path.join(ROOT, "profiles", "w4a16_sweep_70b_layer_hbm_traffic.txt")) as f:
        traffic = f.read()
    labels = {bench.kernel_label(qg.plan(qg.FMT_W4A16, M, K, N)) for (K, N) in bench.SHAPES for M in bench.MS}
    assert len(labels) >= 2
    for label in labels:
        assert label in stats, label
        assert "kernel=" + label + " " in traffic, label


def test_traffic_figures_are_gated_by_the_source_hash(monkeypatch):
    label = bench.kernel_label(qg.plan(qg.FMT_W4A16, 16, 8192, 28672))
    with open(bench.TRAFFIC_FILE) as f:
        recorded = next(l.split("=", 1)[1].strip() for l in f if l.startswith("source_sha="))
    if recorded == bench.source_sha():
        v = bench.measured_traffic(label)
        assert v is not None and v >= bench.alg_bytes(16, 8192, 28672)
    assert bench.measured_traffic("no_such_kernel") is None
    monkeypatch.setattr(bench, "source_sha", lambda: "0" * 16)
    assert bench.measured_traffic(label) is None
