#!/usr/bin/env python3
"""Benchmark of the W4A16 quantized-weight GEMM on one MI355X.

Metric: W4A16 GEMM TFLOP/s and fraction of the HBM roofline versus batch size
M = 1..128 on the K x N = 8192 x 28672 layer (70B-class MLP up-projection) and
its transpose 28672 x 8192 (down-projection).

One step = one pass of the hot path over the whole sweep: for both shapes and
every M in {1, 2, 4, 8, 16, 32, 64, 128}, one C = A * dequant(W) launch through
the C ABI (16 launches). Inputs are seeded synthetic tensors with the workload's
distributions (fp16 A ~ N(0,1); uint4 codes uniform with zero point 8; fp16
group scales uniform in [0.005, 0.02], g = 128), resident in HBM before timing.
The weight blob rotates over several copies (more bytes than the 256 MB
Infinity Cache), one copy further at every launch of its shape, so every launch
streams its weights from HBM.

The warm-up steps (default 80, about 40-50 ms) carry the GPU past the transient
that follows the start of sustained load: a kernel trace of this sweep shows
every launch slowing by up to 35 % from about 3 ms after the load starts and
recovering over the next 30 ms, after which the step time stays flat; the timed
steps measure that steady state.

Prints one JSON line. ``value`` is the aggregate TFLOP/s of the timed steps;
``per_m`` gives each launch's mean duration over a burst of back-to-back
launches (HIP events around the burst), its TFLOP/s and roofline fractions;
``roofline`` describes the kernel with the largest share of a step (found in
the warm-up steps; algorithmic work of its launches in the timed steps / their
time between the two events that bracket its group of launches in every timed
step), with
``traffic`` = HBM bytes per launch from the committed counter summary when it
was taken on the current kernel sources; ``cpu_baseline`` times the NumPy oracle
on a bounded sample of the same work.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 MFMA, published
SHAPES = [(8192, 28672), (28672, 8192)]
MS = [1, 2, 4, 8, 16, 32, 64, 128]
METRIC = "W4A16 GEMM TFLOP/s and % HBM roofline vs M=1–128, K×N=8192×28672"


def alg_bytes(M, K, N):
    """Bytes the method must move: 4-bit codes, fp16 group scales, A and C."""
    return K * N // 2 + (K // 128) * N * 2 + M * K * 2 + M * N * 2


def alg_flops(M, K, N):
    return 2 * M * K * N


def kernel_label(pl: dict) -> str:
    """Name of the HIP kernel a plan launches (as rocprofv3 lists it, shortened)."""
    if pl["kernel"] == 2:
        if pl["nb"] == 2:
            return f"w4a16_wide_m{16 * pl['mb']}_n128"
        return f"w4a16_wide_m{16 * pl['mb']}" + ("_kp2" if pl["wpt"] == 16 else "")
    policy = "PolicyW4A16M32" if (pl["mb"], pl["nb"]) == (2, 2) else "PolicyW4A16"
    return f"skinny_gemm_kp{pl['wpt'] // 4}<{policy},{pl['mb']},{pl['nb']}>"


# sources of the W4A16 kernels the sweep launches (and their planner)
W4A16_SOURCES = ("api.cpp", "qgemm_device.h", "qgemm_internal.h", "skinny.h", "w4a16.hip", "wide.hip")


def source_sha() -> str:
    """Hash of the W4A16 kernel and planner sources with comments and blank
    lines removed: HBM byte counters taken on other code are not reported."""
    import hashlib
    import re
    d = os.path.join(ROOT, "bit_weight_quantized_qgemm_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(W4A16_SOURCES):
        with open(os.path.join(d, f)) as fh:
            txt = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        txt = re.sub(r"//[^\n]*", "", txt)
        code = "\n".join(l.rstrip() for l in txt.splitlines() if l.strip())
        h.update(f.encode() + b"\0" + code.encode())
    return h.hexdigest()[:16]


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4a16_sweep_70b_layer_hbm_traffic.txt")


def measured_traffic(label: str):
    """HBM bytes per launch of `label` from the committed counter summary, or
    None when it is absent or was taken on other kernel sources."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    sha = next((l.split("=", 1)[1].strip() for l in lines if l.startswith("source_sha=")), None)
    if sha != source_sha():
        return None
    for l in lines:
        if l.startswith("kernel=") and l.split()[0] == "kernel=" + label:
            kv = dict(x.split("=", 1) for x in l.split() if "=" in x)
            return float(kv["traffic_bytes_per_launch"])
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=80,
                    help="untimed steps first (80: past the start-of-load transient, see the module notes)")
    ap.add_argument("--burst", type=int, default=40, help="launches per per-kernel timing burst")
    ap.add_argument("--rotate-mb", type=int, default=640, help="minimum bytes of distinct weight copies")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU oracle sample time")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--shapes", default="all", choices=["all", "up", "down"])
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other configured workloads (7B layers, W4A8, mixed 2/4-bit)")
    ap.add_argument("--only-secondary", action="store_true",
                    help="time only the other configured workloads (for kernel traces of them)")
    ap.add_argument("--secondary-filter", default="",
                    help="comma-separated substrings: keep only secondary workloads whose name contains one")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the dense fp16 torch.matmul context line and the achievable-peak probes")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (the known-size "
                         "reference for HBM byte counters)")
    return ap.parse_args()


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(target_s: float) -> dict:
    """The NumPy oracle as it stands, on a bounded sample of the step's work:
    the full M sweep on both shapes restricted to the first n_cols output
    columns of each shape (n_cols chosen from a short calibration pass so that
    one pass takes about target_s / 6 seconds). Inputs are generated before
    any timing. The oracle call is timed three times (median reported as
    ``value``); its two steps, the explicit dequantization and the fp64 matmul,
    are timed separately the same way."""
    from oracle import ref
    from synth import gen

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1

    def inputs(n_cols):
        out = []
        for (K, N) in SHAPES:
            n = min(n_cols, N)
            p = gen.w4a16_problem(128, K, n, seed=0)
            out.append((K, n, p["A"], p["codes"], p["scales"]))
        return out

    def flops_of(data):
        return sum(alg_flops(M, K, n) for (K, n, *_r) in data for M in MS)

    def oracle_pass(data):
        t0 = time.perf_counter()
        for (K, n, A, codes, scales) in data:
            for M in MS:
                ref.gemm_w4a16(A[:M], codes, scales)
        return time.perf_counter() - t0

    def dequant_pass(data):
        # the oracle's dequantization step alone, once per launch of the sweep
        t0 = time.perf_counter()
        for (K, n, A, codes, scales) in data:
            for M in MS:
                ref.dequant_w4a16(codes, scales)
        return time.perf_counter() - t0

    def matmul_pass(data, W):
        t0 = time.perf_counter()
        for (K, n, A, codes, scales), Wi in zip(data, W):
            for M in MS:
                A[:M].astype(np.float64) @ Wi
        return time.perf_counter() - t0

    cal = inputs(256)
    dt_cal = oracle_pass(cal)
    n_cols = int(256 * (target_s / 6.0) / max(dt_cal, 1e-3))
    n_cols = max(64, min(max(N for _, N in SHAPES), n_cols // 64 * 64))
    data = inputs(n_cols)
    flops = flops_of(data)
    t_total = sorted(oracle_pass(data) for _ in range(3))
    t_deq = sorted(dequant_pass(data) for _ in range(3))
    W = [ref.dequant_w4a16(codes, scales) for (_K, _n, _A, codes, scales) in data]
    t_mm = sorted(matmul_pass(data, W) for _ in range(3))
    del W
    med = t_total[1]
    return {
        "value": flops / med / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "host_cpus": len(os.sched_getaffinity(0)),
        "seconds_median_of_3": round(med, 3),
        "dequant_seconds_median_of_3": round(t_deq[1], 3),
        "matmul_seconds_median_of_3": round(t_mm[1], 3),
        "sample": f"fp64 dequantize+matmul (oracle.ref.gemm_w4a16) of the M sweep {MS} on both shapes, "
                  f"first {n_cols} output columns of each ({flops / 1e9:.2f} GFLOP per pass); median of 3 "
                  f"timed passes, inputs generated before timing; dequant and matmul steps timed apart "
                  f"(median of 3 each)",
    }


INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published

SECONDARY = (
    [("w4a16 config-0", 1, 1024, 1024, 16)]
    + [("w4a16 7B layer", 1, K, N, M) for (K, N) in [(4096, 4096), (4096, 11008), (11008, 4096)]
       for M in (1, 16, 32, 64, 128)]
    + [("w4a8", 2, 4096, 11008, M) for M in (16, 64, 128)]
    + [("mixed 2/4-bit", 3, 4096, 4096, M) for M in (1, 16, 64)]
    + [("per-token int8 quantization", 4, 4096, 0, M) for M in (16, 64, 128)]
    + [("w4a8 from fp16 (quantize + GEMM)", 5, 4096, 11008, M) for M in (16, 64, 128)]
    + [("w4a16 2:4 sparse", 7, K, N, M) for (K, N) in [(8192, 28672), (4096, 11008)] for M in (1, 16, 64)]
    + [(f"bit-plane w{b}a8", 8, 4096, 11008, M) for b in (1, 2, 3, 4, 8) for M in (1, 16)]
    + [(name, 6, 4096, 11008, M) for name in ("w4g g64 fp16", "w4g g128 zeros fp16", "w4g per-channel fp16",
                                              "w4g g128 bf16", "w4g g128 zeros bf16") for M in (1, 16)]
    + [("w4g g128 zeros fp16", 6, K, N, M) for (K, N) in [(8192, 28672), (28672, 8192)] for M in (16, 64, 128)]
)
# general-grid variants: name -> (group size (0 = K), stored zero points, activation type)
W4G_VARIANTS = {"w4g g64 fp16": (64, False, "fp16"), "w4g g128 zeros fp16": (128, True, "fp16"),
                "w4g per-channel fp16": (0, False, "fp16"), "w4g g128 bf16": (128, False, "bf16"),
                "w4g g128 zeros bf16": (128, True, "bf16")}


def secondary_bytes_ops(fmt, K, N, M, n4=0, gs=128, zeros=False, name_bits=4):
    """Algorithmic bytes and ops of one launch (codes, scales, A, C)."""
    G = K // 128
    if fmt == 8:   # b bit planes, channel scales, int8 A + row scales, fp16 C
        b = int(name_bits)
        return K * N * b // 8 + 2 * N + M * K + 2 * M + 2 * M * N, alg_flops(M, K, N)
    if fmt == 7:   # kept codes (half the weights x 4 bits) + 2-bit positions + scales, A, C
        return K * N // 4 + K * N // 8 + G * N * 2 + 2 * M * K + 2 * M * N, alg_flops(M, K, N)
    if fmt == 6:   # codes, one 2-byte scale (4 with a zero point) per group, A, C
        return K * N // 2 + (K // gs) * N * (4 if zeros else 2) + 2 * M * K + 2 * M * N, alg_flops(M, K, N)
    if fmt == 4:   # read fp16 A, write int8 codes and fp16 scales
        return 3 * M * K + 2 * M, M * K
    if fmt == 5:   # the quantization's bytes plus the W4A8 GEMM's
        b, o = secondary_bytes_ops(2, K, N, M)
        return b + 3 * M * K + 2 * M, o
    if fmt == 1:
        return alg_bytes(M, K, N), alg_flops(M, K, N)
    if fmt == 2:
        return K * N // 2 + G * N + 2 * N + M * K + 2 * M + 2 * M * N, alg_flops(M, K, N)
    groups = G * N
    return (32 * (groups - n4) + 64 * n4 + 2 * groups + groups // 8 + 2 * M * K + 2 * M * N,
            alg_flops(M, K, N))


def secondary(torch, qg, dev, rotate_mb, name_filter=""):
    """The other configured workloads, each timed as replays of a captured HIP
    graph of back-to-back launches over rotating weight copies (kernel time
    without host launch overhead; weights stream from HBM)."""
    from synth import gen
    stream = torch.cuda.current_stream()
    rows = []
    built = {}
    keep = [f for f in name_filter.split(",") if f]
    for (name, fmt, K, N, M) in SECONDARY:
        if keep and not any(f in name for f in keep):
            continue
        key = (fmt, K, N, name if fmt in (6, 8) else "")
        if key not in built:
            if fmt == 8:
                bits = int(name.split("w")[1].split("a")[0])
                p = gen.bitplane_problem(128, K, N, bits, seed=0)
                blob = qg.repack_bitplane(torch.from_numpy(p["codes"]).to(dev),
                                          torch.from_numpy(p["chan_scales"]).to(dev), bits)
                A = torch.from_numpy(p["A"]).to(dev)
                extra = {"a_scale": torch.from_numpy(p["a_scale"]).to(dev), "bits": bits}
            elif fmt == 7:
                p = gen.w4a16_sp24_problem(128, K, N, seed=0)
                blob = qg.repack_sp24(torch.from_numpy(p["codes"].view(np.int32)).to(dev),
                                      torch.from_numpy(p["scales"]).to(dev))
                A = torch.from_numpy(p["A"]).to(dev)
                extra = {}
            elif fmt == 6:
                gs0, zeros, act = W4G_VARIANTS[name]
                gs = gs0 or K
                p = gen.w4g_problem(128, K, N, gs, zeros, act, seed=0)
                sc = torch.from_numpy(p["scales"].view(np.int16)).to(dev)
                zt = None if p["zeros"] is None else torch.from_numpy(p["zeros"]).to(dev)
                blob = qg.repack_w4g(torch.from_numpy(p["codes"].view(np.int32)).to(dev), sc, zt, gs)
                A = torch.from_numpy(p["A"].view(np.int16)).to(dev)
                A = A.view(torch.float16) if act == "fp16" else A.view(torch.bfloat16)
                extra = {"gs": gs, "zeros": zeros}
            elif fmt == 4:
                A = torch.from_numpy(gen.w4a16_problem(128, K, 128, seed=0, weights=False)["A"]).to(dev)
                blob, extra = None, {}
            elif fmt == 1:
                p = gen.w4a16_problem(128, K, N, seed=0)
                blob = qg.repack_w4a16(torch.from_numpy(p["codes"].view(np.int32)).to(dev),
                                       torch.from_numpy(p["scales"]).to(dev))
                A = torch.from_numpy(p["A"]).to(dev)
                extra = {}
            elif fmt in (2, 5):
                p = gen.w4a8_problem(128, K, N, seed=0)
                blob = qg.repack_w4a8(torch.from_numpy(p["codes"].view(np.int32)).to(dev),
                                      torch.from_numpy(p["group_scales"]).to(dev),
                                      torch.from_numpy(p["chan_scales"]).to(dev))
                A = torch.from_numpy(p["A"]).to(dev)
                extra = {"a_scale": torch.from_numpy(p["a_scale"]).to(dev)}
                if fmt == 5:
                    A = torch.from_numpy(gen.w4a16_problem(128, K, 128, seed=0, weights=False)["A"]).to(dev)
            else:
                p = gen.w2w4_problem(128, K, N, seed=0)
                blob = qg.repack_w2w4(torch.from_numpy(p["codes"]).to(dev), torch.from_numpy(p["scales"]).to(dev),
                                      p["bitmap"])
                A = torch.from_numpy(p["A"]).to(dev)
                extra = {"n4": int(p["mask"].sum())}
            if blob is None:   # no weights: a graph of 64 launches
                built = {key: ([None] * 64, A, extra)}
            else:
                reps = max(2, math.ceil(rotate_mb * 2**20 / blob.numel()))
                built = {key: (([blob] + [blob.clone() for _ in range(reps - 1)]), A, extra)}
        blobs, A_all, extra = built[key]
        A = A_all[:M].contiguous()
        C = torch.empty((M, max(N, 1)), dtype=A.dtype if fmt == 6 else torch.float16, device=dev)
        ws = qg.Workspace()
        if fmt == 8:
            a_s = extra["a_scale"][:M].contiguous()
            run = lambda b: qg.bitplane_a8(A, a_s, b, K, N, extra["bits"], out=C, workspace=ws)
        elif fmt == 7:
            run = lambda b: qg.w4a16_sp24(A, b, K, N, out=C, workspace=ws)
        elif fmt == 6:
            run = lambda b: qg.w4g(A, b, K, N, extra["gs"], extra["zeros"], out=C, workspace=ws)
        elif fmt == 1:
            run = lambda b: qg.w4a16(A, b, K, N, out=C, workspace=ws)
        elif fmt == 2:
            a_s = extra["a_scale"][:M].contiguous()
            run = lambda b: qg.w4a8(A, a_s, b, K, N, out=C, workspace=ws)
        elif fmt == 4:
            Qb = torch.empty((M, K), dtype=torch.int8, device=dev)
            Sb = torch.empty((M,), dtype=torch.float16, device=dev)
            run = lambda b: qg.quantize_a8(A, out=Qb, scale_out=Sb)
        elif fmt == 5:
            Qb = torch.empty((M, K), dtype=torch.int8, device=dev)
            Sb = torch.empty((M,), dtype=torch.float16, device=dev)

            def run(b):
                qg.quantize_a8(A, out=Qb, scale_out=Sb)
                qg.w4a8(Qb, Sb, b, K, N, out=C, workspace=ws)
        else:
            run = lambda b: qg.w2w4_mixed(A, b, K, N, out=C, workspace=ws)
        for i in range(3):
            run(blobs[i % len(blobs)])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        n = len(blobs)
        with torch.cuda.graph(g):
            for i in range(n):
                run(blobs[i])
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(5):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (5 * n)
        byt, ops = secondary_bytes_ops(fmt, K, N, M, extra.get("n4", 0), extra.get("gs", 128),
                                       extra.get("zeros", False), extra.get("bits", 4))
        peak = INT8_PEAK_TOPS if fmt in (2, 5, 8) else FP16_PEAK_TFLOPS
        gbs = byt / (us * 1e-6) / 1e9
        tops = ops / (us * 1e-6) / 1e12
        roof_us = max(byt / (HBM_PEAK_GBS * 1e9), ops / (peak * 1e12)) * 1e6
        rows.append({"workload": name, "fmt": ["", "w4a16", "w4a8", "w2w4", "quant_a8", "w4a8_fp16", "w4g", "w4a16_sp24", "bitplane_a8"][fmt],
                     "K": K, "N": N, "M": M,
                     "us": round(us, 2), "tops": round(tops, 2), "gbs": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "roofline_frac": round(roof_us / us, 4),
                     "bound": "hbm" if byt / (HBM_PEAK_GBS * 1e9) >= ops / (peak * 1e12) else "mfma",
                     "launches_per_graph": n})
        print(f"[bench] secondary {name} K={K} N={N} M={M}: {us:.2f} us", file=sys.stderr, flush=True)
        del g
    return rows


def dense_fp16_context(torch, dev, per_m):
    """The same GEMMs with dense fp16 weights through torch.matmul (the vendor
    BLAS), for the MARLIN abstract's comparison of the 4-bit kernel with the
    uncompressed layer; weights rotate over two copies (more than the 256 MB
    Infinity Cache). Context only: it is run and timed, not inspected."""
    stream = torch.cuda.current_stream()
    rows = []
    for (K, N) in SHAPES:
        W = [torch.randn(K, N, device=dev, dtype=torch.float16) for _ in range(2)]
        A_all = torch.randn(128, K, device=dev, dtype=torch.float16)
        for M in MS:
            A = A_all[:M].contiguous()
            for i in range(4):
                torch.matmul(A, W[i % 2])
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            L = 20
            a.record(stream)
            for i in range(L):
                torch.matmul(A, W[i % 2])
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / L
            q = next((r["us"] for r in per_m if r["shape"] == f"{K}x{N}" and r["M"] == M), None)
            rows.append({"shape": f"{K}x{N}", "M": M, "fp16_dense_us": round(us, 2),
                         "w4a16_us": q, "w4a16_speedup": None if q is None else round(us / q, 2)})
        del W, A_all
        torch.cuda.empty_cache()
    return rows


def peak_probes(torch, dev):
    """Achievable peaks on this GPU: the hand-written probes of
    libqgemm_probes.so (a streaming read of 2 GiB, more than the Infinity
    Cache, with its checksum verified; back-to-back matrix-core instructions of
    each kind the kernels use) and a large dense fp16 GEMM through the vendor
    BLAS (torch.matmul, 8192^3)."""
    from bit_weight_quantized_qgemm_amd import probes

    out = probes.measure(torch, dev)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p = torch.randn(8192, 8192, device=dev, dtype=torch.float16)
    q = torch.randn(8192, 8192, device=dev, dtype=torch.float16)
    for _ in range(3):
        torch.matmul(p, q)
    a.record(stream)
    for _ in range(10):
        torch.matmul(p, q)
    b.record(stream)
    torch.cuda.synchronize()
    out["fp16_gemm_torch_matmul_tflops"] = round(2 * 8192**3 * 10 / (a.elapsed_time(b) * 1e-3) / 1e12, 1)
    del p, q
    torch.cuda.empty_cache()
    return out


def copy_probe(torch, dev, mib):
    """One plain device copy of `mib` MiB: the known-size reference for HBM
    byte counters (FETCH_SIZE, WRITE_SIZE) in profiled runs."""
    src = torch.ones(mib * 2**20 // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; multi-GPU runs are not "
                                   "supported (N-sharding would split the layer's columns across GPUs)"}))
        sys.exit(2)

    import torch

    import bit_weight_quantized_qgemm_amd as qg
    from synth import gen

    if args.only_secondary:
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        if args.copy_probe_mib:
            copy_probe(torch, dev, args.copy_probe_mib)
        print(json.dumps({"secondary": secondary(torch, qg, dev, 512, args.secondary_filter)}), flush=True)
        return

    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = qg.lib()
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    shapes = SHAPES if args.shapes == "all" else ([SHAPES[0]] if args.shapes == "up" else [SHAPES[1]])

    # ---- inputs resident in HBM
    cases = []   # (K, N, M, blobs, A, C, ws)
    for (K, N) in shapes:
        p = gen.w4a16_problem(128, K, N, seed=0)
        codes = torch.from_numpy(p["codes"].view(np.int32)).to(dev)
        scales = torch.from_numpy(p["scales"]).to(dev)
        blob = qg.repack_w4a16(codes, scales)
        del codes, scales
        reps = max(1, math.ceil(args.rotate_mb * 2**20 / blob.numel()))
        blobs = [blob] + [blob.clone() for _ in range(reps - 1)]
        A_all = torch.from_numpy(p["A"]).to(dev)
        for M in MS:
            A = A_all[:M].contiguous()
            C = torch.empty((M, N), dtype=torch.float16, device=dev)
            wsb = qg.workspace_bytes(qg.FMT_W4A16, M, K, N)
            ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device=dev)
            cases.append(dict(K=K, N=N, M=M, blobs=blobs, A=A, C=C, ws=ws, wsb=wsb,
                              plan=qg.plan(qg.FMT_W4A16, M, K, N)))
    torch.cuda.synchronize()

    # Every launch reads another copy of its layer's blob than the launch before
    # it: the k-th launch of a shape takes copy k mod copies, so a copy is read
    # again only after the other copies (more than the 256 MB Infinity Cache in
    # between) and the weights stream from HBM in the timed steps as in bursts.
    shape_launches = {}

    def launch(cs, i=None):
        key = (cs["K"], cs["N"])
        k = shape_launches.get(key, 0)
        shape_launches[key] = k + 1
        b = cs["blobs"][k % len(cs["blobs"])]
        st = L.qgemm_w4a16(ctypes.c_void_p(cs["A"].data_ptr()), cs["K"], ctypes.c_void_p(b.data_ptr()),
                           ctypes.c_void_p(cs["C"].data_ptr()), cs["N"], cs["M"], cs["K"], cs["N"],
                           ctypes.c_void_p(cs["ws"].data_ptr()), cs["ws"].numel(), sptr)
        if st != 0:
            raise RuntimeError(f"qgemm_w4a16 failed: {st} {L.qgemm_last_error().decode()}")

    def step(i):
        for cs in cases:
            launch(cs, i)

    if args.copy_probe_mib:
        copy_probe(torch, dev, args.copy_probe_mib)

    print(f"[bench] inputs resident: {len(cases)} launches per step", file=sys.stderr, flush=True)
    # Launches of one kernel run back to back (the step's order groups them).
    # The warm-up steps close every group with an event to find the kernel with
    # the largest share of a step (the last half of them, past most of the
    # start-of-load transient); the timed steps then record two events per step
    # only, after that kernel's group (first in the step) and at the end of the
    # step: each timestamped event holds the next launch back by about 6 us,
    # which one event per group would add to the step time four times over.
    groups = {}
    for j, cs in enumerate(cases):
        groups.setdefault(kernel_label(cs["plan"]), []).append(j)
    glist = list(groups.items())
    ev = lambda: torch.cuda.Event(enable_timing=True)
    wbounds = [[ev() for _ in glist] for _ in range(args.warmup)]
    w0 = ev()
    w0.record(stream)
    for i in range(args.warmup):
        for gi, (_, idx) in enumerate(glist):
            for j in idx:
                launch(cases[j], i)
            wbounds[i][gi].record(stream)
    torch.cuda.synchronize()
    warm_us = {}
    for i in range(args.warmup // 2, args.warmup):
        for gi, (label, _) in enumerate(glist):
            start = wbounds[i][gi - 1] if gi else (wbounds[i - 1][-1] if i else w0)
            warm_us[label] = warm_us.get(label, 0.0) + start.elapsed_time(wbounds[i][gi]) * 1e3
    dom_label = max(warm_us, key=warm_us.get) if warm_us else glist[0][0]
    order = [g for g in glist if g[0] == dom_label] + [g for g in glist if g[0] != dom_label]

    # ---- timed steps
    dom_end = [ev() for _ in range(args.steps)]
    step_end = [ev() for _ in range(args.steps)]
    e0 = ev()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        for gi, (_, idx) in enumerate(order):
            for j in idx:
                launch(cases[j], i)
            if gi == 0:
                dom_end[i].record(stream)
        step_end[i].record(stream)
    e1 = step_end[-1]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = e0.elapsed_time(e1) / args.steps
    step_flops = sum(alg_flops(c["M"], c["K"], c["N"]) for c in cases)
    value = step_flops / (step_ms * 1e-3) / 1e12
    dom_us = sum((step_end[i - 1] if i else e0).elapsed_time(dom_end[i]) * 1e3 for i in range(args.steps))

    # ---- per-launch table: bursts of back-to-back launches of each case
    per_m = []
    for cs in cases:
        for i in range(3):
            launch(cs, i)
        a, b = ev(), ev()
        a.record(stream)
        for i in range(args.burst):
            launch(cs, i)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / args.burst
        M, K, N = cs["M"], cs["K"], cs["N"]
        byt, fl = alg_bytes(M, K, N), alg_flops(M, K, N)
        gbs = byt / (us * 1e-6) / 1e9
        tf = fl / (us * 1e-6) / 1e12
        roof_us = max(byt / (HBM_PEAK_GBS * 1e9), fl / (FP16_PEAK_TFLOPS * 1e12)) * 1e6
        per_m.append({"shape": f"{K}x{N}", "M": M, "us": round(us, 2), "tflops": round(tf, 2),
                      "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                      "mfma_frac": round(tf / FP16_PEAK_TFLOPS, 4),
                      "roofline_frac": round(roof_us / us, 4), "kernel": kernel_label(cs["plan"]),
                      "plan": {k: cs["plan"][k] for k in ("mb", "nb", "wpt", "splits", "mt", "waves")}})

    # ---- roofline of the dominant kernel (the largest share of the warm-up
    # steps): algorithmic work of its launches in the timed steps / their
    # event time there
    dom = {"us": dom_us, "n": 0, "bytes": 0, "flops": 0}
    for cs in cases:
        if kernel_label(cs["plan"]) != dom_label:
            continue
        M, K, N = cs["M"], cs["K"], cs["N"]
        dom["n"] += args.steps
        dom["bytes"] += alg_bytes(M, K, N) * args.steps
        dom["flops"] += alg_flops(M, K, N) * args.steps
    mfma_bound = dom["flops"] / (FP16_PEAK_TFLOPS * 1e12) > dom["bytes"] / (HBM_PEAK_GBS * 1e9)
    traffic = measured_traffic(dom_label)
    if mfma_bound:
        ach = dom["flops"] / (dom["us"] * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / FP16_PEAK_TFLOPS, 4)}
    else:
        ach = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof["traffic"] = None if traffic is None else round(traffic)
    roof.update({"kernel": dom_label, "launches": dom["n"], "us_per_launch": round(dom["us"] / dom["n"], 2),
                 "alg_bytes_per_launch": round(dom["bytes"] / dom["n"]),
                 "alg_flops_per_launch": round(dom["flops"] / dom["n"]),
                 "share_of_step": round(dom["us"] / (step_ms * 1e3 * args.steps), 3),
                 "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                 "source_sha": source_sha()})

    sec = None if args.no_secondary else secondary(torch, qg, dev, 512, args.secondary_filter)
    context = None
    if not args.no_context:
        context = {"dense_fp16_torch_matmul": dense_fp16_context(torch, dev, per_m),
                   "achievable_peaks": peak_probes(torch, dev)}
        # the dominant kernel against what the probes sustain on this GPU (context;
        # `peak` above stays the published figure)
        pk = context["achievable_peaks"]
        # the matrix cores sustain less on random operands than on constants:
        # the random-operand rate is the one a GEMM on real data can reach
        mfma_ach = pk["mfma_v_mfma_f32_32x32x16_f16_random_operands_2_waves_per_simd_tops"]
        ach_peak = pk["stream_read_gbs"] if roof["bound"] == "hbm" else mfma_ach
        roof["achievable_peak"] = ach_peak
        roof["frac_of_achievable"] = round(roof["achieved"] / ach_peak, 4)
        for r in per_m:
            r["mfma_frac_of_achievable"] = round(r["tflops"] / mfma_ach, 4)
            r["hbm_frac_of_achievable"] = round(r["gbs"] / pk["stream_read_gbs"], 4)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "W4A16 GEMM, K x N = 8192 x 28672 and 28672 x 8192, "
                               "M in {1,2,4,8,16,32,64,128}, g=128 fp16 scales, zero point 8",
                   "launches_per_step": len(cases),
                   "weight_copies_rotated": len(cases[0]["blobs"]),
                   "wall_s_timed": round(wall, 3)},
        "roofline": roof,
        "per_m": per_m,
        "cpu_baseline": cpu,
        "secondary": sec,
        "context": context,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
