"""ctypes binding of the achievable-peak probes (``include/qgemm_probes.h``,
``libqgemm_probes.so``): argument marshalling and timing with HIP events on
the current stream. The probes compute no GEMM; they give the streaming-read
bandwidth and matrix-core rate that the GEMM kernels' roofline fractions can
be read against."""

from __future__ import annotations

import ctypes
import os

from bit_weight_quantized_qgemm_amd import build as _b

SYMBOLS = ("qgemm_probe_stream_read", "qgemm_probe_mfma", "qgemm_probe_mfma_ops")
KINDS = {0: "v_mfma_f32_32x32x16_f16", 1: "v_mfma_f32_16x16x32_f16", 2: "v_mfma_i32_16x16x64_i8",
         3: "v_mfma_f32_32x32x16_f16_a_from_lds_1kb_per_mfma",
         4: "v_mfma_f32_32x32x16_f16_a_from_lds_1kb_per_2_mfma",
         5: "v_mfma_f32_32x32x16_f16_random_operands", 6: "v_mfma_i32_16x16x64_i8_random_operands"}
_lib = None


def lib_path() -> str:
    return _b.PROBES_LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path()):
            raise RuntimeError(f"{lib_path()} is not built: run python -m bit_weight_quantized_qgemm_amd.build")
        L = ctypes.CDLL(lib_path())
        L.qgemm_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.qgemm_probe_stream_read.restype = ctypes.c_int
        L.qgemm_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
        L.qgemm_probe_mfma.restype = ctypes.c_int
        L.qgemm_probe_mfma_ops.argtypes = [ctypes.c_int]
        L.qgemm_probe_mfma_ops.restype = ctypes.c_int64
        _lib = L
    return _lib


def _check(st: int, what: str) -> None:
    if st != 0:
        raise RuntimeError(f"{what} failed with status {st}")


def stream_read(torch, src, workgroups: int, sink, chunked: bool = False) -> None:
    """Enqueue one read of all of ``src`` (a contiguous CUDA tensor) on the
    current stream; each wave writes the sum of its 32-bit words to its slot of
    ``sink`` (int32, at least 4 * workgroups elements)."""
    nbytes = src.numel() * src.element_size()
    s = torch.cuda.current_stream().cuda_stream
    _check(lib().qgemm_probe_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), sink.numel(), workgroups,
                                         int(chunked), s), "stream_read")


def read_checksum(sink, workgroups: int) -> int:
    """Sum of the wave slots of the last read, modulo 2^32."""
    import numpy as np
    return int(sink[: 4 * workgroups].cpu().numpy().astype(np.uint32).astype(np.uint64).sum()) % 2**32


def mfma(torch, sink, workgroups: int, iters: int, kind: int) -> None:
    s = torch.cuda.current_stream().cuda_stream
    _check(lib().qgemm_probe_mfma(sink.data_ptr(), sink.numel(), workgroups, iters, kind, s), "mfma")


def measure(torch, dev, read_gib: float = 2.0, reps: int = 10) -> dict:
    """Best streaming-read GB/s over a few grid sizes (a buffer larger than the
    256 MB Infinity Cache, read ``reps`` times back to back), and the
    matrix-core rate of each instruction kind on a full grid."""
    stream = torch.cuda.current_stream()
    out = {}
    n = int(read_gib * 2**30) // 4
    x = torch.ones(n, dtype=torch.int32, device=dev)
    sink = torch.zeros(8192 * 4, dtype=torch.int32, device=dev)
    reads = {}
    for chunked in (False, True):
        for wg in (1024, 2048, 4096, 8192):
            stream_read(torch, x, wg, sink, chunked)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                stream_read(torch, x, wg, sink, chunked)
            b.record(stream)
            torch.cuda.synchronize()
            reads[f"{'chunked' if chunked else 'strided'}_{wg}"] = round(n * 4 * reps / (a.elapsed_time(b) * 1e-3) / 1e9,
                                                                         1)
            # every word is 1: the slots of a read add up to n, modulo 2^32
            got = read_checksum(sink, wg)
            if got != n % 2**32:
                raise RuntimeError(f"stream-read probe checksum {got} != {n % 2**32}")
    out["stream_read_gbs_by_order_and_workgroups"] = reads
    out["stream_read_gbs"] = max(reads.values())
    # the floor of a short streaming launch: 1 MiB read by 256 workgroups, 50
    # launches captured in a HIP graph and replayed (time per launch on the
    # GPU, gaps between launches included, host launch cost excluded)
    small = x[: 2**18]
    for _ in range(3):
        stream_read(torch, small, 256, sink, True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(50):
            stream_read(torch, small, 256, sink, True)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    out["stream_read_1mib_us_per_launch"] = round(a.elapsed_time(b) * 1e3 / 50, 2)
    if read_checksum(sink, 256) != 2**18:
        raise RuntimeError("stream-read probe checksum of the short read")
    del g
    del x
    # 2048 workgroups of 4 waves: 8 waves per SIMD; 512: 2 waves per SIMD
    iters = 2048
    sinkm = torch.zeros(2048 * 4, dtype=torch.int32, device=dev)
    for wgs in (2048, 512):
        for kind, name in KINDS.items():
            mfma(torch, sinkm, wgs, 64, kind)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            mfma(torch, sinkm, wgs, iters, kind)
            b.record(stream)
            torch.cuda.synchronize()
            ops = wgs * 4 * iters * 8 * (2 if kind == 4 else 1) * lib().qgemm_probe_mfma_ops(kind)
            out[f"mfma_{name}_{wgs * 4 // 1024}_waves_per_simd_tops"] = round(ops / (a.elapsed_time(b) * 1e-3) / 1e12, 1)
    return out
