"""The achievable-peak probes (include/qgemm_probes.h): exported symbols and
host-side argument checks on the CPU; on the GPU, the streaming read's
checksum proves that every byte was read, and the matrix-core loop runs."""

import os
import re

import pytest

from bit_weight_quantized_qgemm_amd import probes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_probe():
    text = open(os.path.join(ROOT, "include", "qgemm_probes.h")).read()
    names = sorted(set(re.findall(r"^\s*(?:int|int64_t)\s+(qgemm_probe_\w+)\s*\(", text, re.M)))
    assert names == sorted(probes.SYMBOLS)
    L = probes.lib()
    for n in names:
        assert hasattr(L, n), n


def test_probe_argument_checks_need_no_gpu():
    L = probes.lib()
    assert L.qgemm_probe_mfma_ops(0) == 32768
    assert L.qgemm_probe_mfma_ops(1) == 16384
    assert L.qgemm_probe_mfma_ops(2) == 32768
    assert L.qgemm_probe_mfma_ops(3) == 32768
    assert L.qgemm_probe_mfma_ops(4) == 32768
    assert L.qgemm_probe_mfma_ops(5) == 32768
    assert L.qgemm_probe_mfma_ops(6) == 32768
    assert L.qgemm_probe_mfma_ops(7) == 0
    # rejected before any HIP call: null pointers, sizes, alignment, 32-bit offset range
    assert L.qgemm_probe_stream_read(None, 1024, 16, 32, 8, 0, None) == -1
    assert L.qgemm_probe_stream_read(16, 1000, 16, 32, 8, 0, None) == -1
    assert L.qgemm_probe_stream_read(24, 1024, 16, 32, 8, 0, None) == -1
    assert L.qgemm_probe_stream_read(16, 3 << 30, 16, 4 * 65536, 65536, 1, None) == -1
    assert L.qgemm_probe_stream_read(16, 4 << 30, 16, 32, 8, 0, None) == -1
    assert L.qgemm_probe_stream_read(16, 1024, 16, 32, 8, 2, None) == -1
    assert L.qgemm_probe_stream_read(16, 1024, 16, 31, 8, 0, None) == -1   # fewer slots than waves
    assert L.qgemm_probe_mfma(16, 31, 8, 1, 0, None) == -1   # sink smaller than 4 words per workgroup
    assert L.qgemm_probe_mfma(16, 32, 8, 1, 7, None) == -1   # unknown kind
    assert L.qgemm_probe_mfma(16, 32, 8, 0, 0, None) == -1


@pytest.mark.gpu
def test_stream_read_checksum_and_mfma_loop():
    import torch

    dev = torch.device("cuda:0")
    x = torch.randint(0, 2**31 - 1, (3 * 2**20 + 4 * 1000,), dtype=torch.int32, device=dev)   # ragged vs the grid
    sink = torch.zeros(4 * 1024, dtype=torch.int32, device=dev)
    want = int(x.cpu().numpy().astype("uint64").sum()) % 2**32
    for chunked in (False, True):
        for wg in (1, 7, 1024):
            sink.fill_(-1)
            probes.stream_read(torch, x, wg, sink, chunked)
            torch.cuda.synchronize()
            assert probes.read_checksum(sink, wg) == want, (chunked, wg)
    m = probes.measure(torch, dev, read_gib=0.5, reps=2)
    assert m["stream_read_gbs"] > 100
    for name in probes.KINDS.values():
        for w in (8, 2):
            assert m[f"mfma_{name}_{w}_waves_per_simd_tops"] > 10
