"""CPU tests of the C ABI: the library loads, exports every symbol declared in
include/qgemm.h, validates arguments before any HIP call, and plans work that
covers every (m-tile, n-tile, group) exactly once. No kernel is launched."""

import ctypes
import os
import re

import numpy as np
import pytest

import bit_weight_quantized_qgemm_amd as qg
from oracle import layout
from synth import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WS, ERR_FMT, ERR_RANGE, ERR_ALIAS, ERR_HIP, ERR_DEV, ERR_SIZE = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10)

CONFIG_SHAPES = [(1024, 1024), (4096, 4096), (4096, 11008), (11008, 4096), (8192, 28672),
                 (28672, 8192)]


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qg.lib_path()):
        pytest.fail("libqgemm.so is not built: run python -m bit_weight_quantized_qgemm_amd.build")
    return qg.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(qgemm_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 11
    assert sorted(qg.EXPORTED_SYMBOLS) == names
    for n in names:
        assert hasattr(L, n), n
    assert L.qgemm_version() >= 100
    assert L.qgemm_status_str(-4).decode() == "QGEMM_ERR_WORKSPACE"
    assert L.qgemm_status_str(12345).decode() == "QGEMM_ERR_UNKNOWN"


@pytest.mark.parametrize("K,N", CONFIG_SHAPES + [(128, 64), (1152, 320)])
def test_packed_bytes_match_independent_layout(K, N):
    assert qg.packed_bytes(qg.FMT_W4A16, K, N) == layout.packed_bytes(layout.FMT_W4A16, K, N)
    if K <= 16384:
        assert qg.packed_bytes(qg.FMT_W4A8, K, N) == layout.packed_bytes(layout.FMT_W4A8, K, N)
    mask = np.zeros((K // 128, N), dtype=bool)
    mask.ravel()[::7] = True
    bm = gen.bitmap_from_mask(mask)
    assert qg.packed_bytes(qg.FMT_W2W4, K, N, bm) == layout.packed_bytes(layout.FMT_W2W4, K, N,
                                                                         int(mask.sum()))


def _st(L, fn, *args):
    return getattr(L, fn)(*args)


def test_shape_and_format_validation(L):
    out = ctypes.c_size_t(0)
    assert L.qgemm_packed_bytes(7, 1024, 1024, None, ctypes.byref(out)) == ERR_FMT
    assert L.qgemm_packed_bytes(1, 1000, 1024, None, ctypes.byref(out)) == ERR_SHAPE
    assert L.qgemm_packed_bytes(1, 1024, 96, None, ctypes.byref(out)) == ERR_SHAPE
    assert L.qgemm_packed_bytes(1, 0, 64, None, ctypes.byref(out)) == ERR_SHAPE
    assert L.qgemm_packed_bytes(1, 1024, 64, None, None) == ERR_NULL
    assert L.qgemm_packed_bytes(2, 16384, 64, None, ctypes.byref(out)) == OK
    assert L.qgemm_packed_bytes(2, 16512, 64, None, ctypes.byref(out)) == ERR_SHAPE
    # K*N above 2^32 (blob offsets are 32-bit); exactly 2^32 is accepted
    assert L.qgemm_packed_bytes(1, 1 << 20, 1 << 13, None, ctypes.byref(out)) == ERR_SHAPE
    assert L.qgemm_packed_bytes(1, 1 << 19, 1 << 13, None, ctypes.byref(out)) == OK
    assert L.qgemm_packed_bytes(3, 1024, 64, None, ctypes.byref(out)) == ERR_NULL
    assert L.qgemm_workspace_bytes(1, -1, 1024, 64, ctypes.byref(out)) == ERR_SHAPE
    assert L.qgemm_workspace_bytes(1, 65536, 1024, 64, ctypes.byref(out)) == ERR_SHAPE
    assert L.qgemm_workspace_bytes(1, 0, 1024, 64, ctypes.byref(out)) == OK and out.value == 0


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_gemm_validation_order_without_gpu(L):
    A, P, C, W = _fake(0x10000000), _fake(0x20000000), _fake(0x30000000), _fake(0x40000000)
    M, K, N = 16, 4096, 4096
    ws = qg.workspace_bytes(qg.FMT_W4A16, M, K, N)
    # M == 0 is a no-op even with NULL pointers
    assert L.qgemm_w4a16(None, K, None, None, N, 0, K, N, None, 0, None) == OK
    assert L.qgemm_w4a16(None, K, P, C, N, M, K, N, W, ws, None) == ERR_NULL
    assert L.qgemm_w4a16(A, K, P, C, N, M, 1000, N, W, ws, None) == ERR_SHAPE
    assert L.qgemm_w4a16(_fake(0x10000008), K, P, C, N, M, K, N, W, ws, None) == ERR_ALIGN
    assert L.qgemm_w4a16(A, K - 8, P, C, N, M, K, N, W, ws, None) == ERR_ALIGN   # lda < K
    assert L.qgemm_w4a16(A, K + 4, P, C, N, M, K, N, W, ws, None) == ERR_ALIGN   # lda*2 % 16
    assert L.qgemm_w4a16(A, K, P, C, N - 8, M, K, N, W, ws, None) == ERR_ALIGN   # ldc < N
    if ws:
        assert L.qgemm_w4a16(A, K, P, C, N, M, K, N, W, ws - 1, None) == ERR_WS
        assert L.qgemm_w4a16(A, K, P, C, N, M, K, N, None, 0, None) == ERR_NULL
    # C overlapping A
    assert L.qgemm_w4a16(A, K, P, _fake(0x10000000 + 256), N, M, K, N, W, ws, None) == ERR_ALIAS
    # W4A8 needs a_scale and K <= 16384
    w8 = qg.workspace_bytes(qg.FMT_W4A8, M, K, N)
    assert L.qgemm_w4a8(A, K, None, P, C, N, None, M, K, N, W, w8, None) == ERR_NULL
    assert L.qgemm_w4a8(A, K, _fake(0x50000000), P, C, N, None, M, 16512, N, W, w8, None) == ERR_SHAPE
    assert L.qgemm_w4a8(A, K + 8, _fake(0x50000000), P, C, N, None, M, K, N, W, w8, None) == ERR_ALIGN
    assert L.qgemm_w4a8(A, K, _fake(0x50000000), P, C, N, _fake(0x30000000), M, K, N, W, w8,
                        None) == ERR_ALIAS   # acc_out overlaps C
    # valid arguments reach the device check: without a gfx950 GPU that is an error, not a crash
    st = L.qgemm_w4a16(A, K, P, C, N, M, K, N, W, ws, None)
    if st != OK:
        assert st in (ERR_HIP, ERR_DEV)
        assert len(L.qgemm_last_error()) > 0


def test_quantize_a8_validation_without_gpu(L):
    A, Q, S = _fake(0x10000000), _fake(0x20000000), _fake(0x30000000)
    M, K = 16, 4096
    assert L.qgemm_quantize_a8(None, K, 0, K, None, K, None, None) == OK       # M == 0: no launch
    assert L.qgemm_quantize_a8(A, K, M, 0, Q, K, S, None) == ERR_SHAPE
    assert L.qgemm_quantize_a8(A, K, M, 12, Q, K, S, None) == ERR_SHAPE       # K % 8
    assert L.qgemm_quantize_a8(A, K, -1, K, Q, K, S, None) == ERR_SHAPE
    assert L.qgemm_quantize_a8(A, K, 65536, K, Q, K, S, None) == ERR_SHAPE
    assert L.qgemm_quantize_a8(A, K, M, K, None, K, S, None) == ERR_NULL
    assert L.qgemm_quantize_a8(A, K, M, K, Q, K, None, None) == ERR_NULL
    assert L.qgemm_quantize_a8(_fake(0x10000008), K, M, K, Q, K, S, None) == ERR_ALIGN
    assert L.qgemm_quantize_a8(A, K, M, K, _fake(0x20000008), K, S, None) == ERR_ALIGN
    assert L.qgemm_quantize_a8(A, K, M, K, Q, K, _fake(0x30000001), None) == ERR_ALIGN
    assert L.qgemm_quantize_a8(A, K - 8, M, K, Q, K, S, None) == ERR_ALIGN     # lda < K
    assert L.qgemm_quantize_a8(A, K + 4, M, K, Q, K, S, None) == ERR_ALIGN     # lda % 8
    assert L.qgemm_quantize_a8(A, K, M, K, Q, K + 8, S, None) == ERR_ALIGN     # ldq % 16
    assert L.qgemm_quantize_a8(A, K, M, K, _fake(0x10000000 + 1024), K, S, None) == ERR_ALIAS
    assert L.qgemm_quantize_a8(A, K, M, K, Q, K, _fake(0x20000000 + 64), None) == ERR_ALIAS
    st = L.qgemm_quantize_a8(A, K, M, K, Q, K, S, None)
    if st != OK:
        assert st in (ERR_HIP, ERR_DEV)


def test_repack_validation_without_gpu(L):
    K, N = 1024, 1024
    nb = qg.packed_bytes(qg.FMT_W4A16, K, N)
    codes, sc, out = _fake(0x10000000), _fake(0x20000000), _fake(0x30000000)
    assert L.qgemm_repack(9, K, N, codes, sc, None, None, out, nb, None) == ERR_FMT
    assert L.qgemm_repack(1, K, N, None, sc, None, None, out, nb, None) == ERR_NULL
    assert L.qgemm_repack(2, K, N, codes, sc, None, None, out, nb, None) == ERR_NULL
    assert L.qgemm_repack(3, K, N, codes, sc, None, None, out, nb, None) == ERR_NULL
    assert L.qgemm_repack(1, K, N, codes, sc, None, None, out, nb - 256, None) == ERR_SIZE
    assert L.qgemm_repack(1, K, N, codes, sc, None, None, _fake(0x30000008), nb, None) == ERR_ALIGN
    assert L.qgemm_repack(1, K, N, codes, sc, None, None, _fake(0x10000000 + 4096), nb, None) == ERR_ALIAS


def _launch_workgroups(nt, mt, splits):
    return nt * mt * splits


def _blocks_cover_tiles_once(p):
    # the kernels' block -> (column tile, row tile, k-split) decoding, re-derived:
    # row tiles of one column tile and k-split sit 8 block indices apart, except
    # for the pairs past the last whole group of 8
    nt, mt, s = p["nt"], p["mt"], p["splits"]
    pairs = nt * s
    whole = pairs - pairs % 8
    seen = {}
    for b in range(p["workgroups"]):
        if b < whole * mt:
            q = b // 8
            g, r = (q // mt) * 8 + b % 8, q % mt
        else:
            j = b - whole * mt
            g, r = whole + j % (pairs - whole), j // (pairs - whole)
        t = (g % nt, r, g // nt)
        assert t not in seen
        seen[t] = b
    assert len(seen) == nt * mt * s
    for (n, r, sp), b in seen.items():
        if (sp * nt + n) < whole:
            assert all(seen[(n, r2, sp)] % 8 == b % 8 for r2 in range(mt))


def _check_plan(p, M, K, N, ws=None, exact_ws=True):
    G = K // 128
    if p["kernel"] == 2:
        # 256-column tiles of 8 or 16 waves, or 128-column tiles of 8 (two K-parts of 4)
        assert p["mb"] == 4 and (p["nb"], p["wpt"]) in ((4, 8), (4, 16), (2, 8))
        assert p["nt"] * 64 * p["nb"] == N and p["mt"] * p["mb"] * 16 >= M > (p["mt"] - 1) * p["mb"] * 16
        assert p["workgroups"] == _launch_workgroups(p["nt"], p["mt"], p["splits"])
        _blocks_cover_tiles_once(p)
        cover = np.zeros(G, dtype=int)
        for s in range(p["splits"]):
            G0, G1 = s * p["gps"], min(G, (s + 1) * p["gps"])
            assert G1 > G0
            cover[G0:G1] += 1
        assert np.all(cover == 1)
        return
    assert p["kernel"] in (1, 3) and p["nb"] in (1, 2) and p["mb"] in (1, 2)
    assert p["nt"] * p["nb"] * 64 == N
    assert p["mt"] * p["mb"] * 16 >= M > (p["mt"] - 1) * p["mb"] * 16
    assert p["wpt"] in (4, 8, 16) and p["wpt"] // 4 <= p["gps"]
    assert p["workgroups"] == _launch_workgroups(p["nt"], p["mt"], p["splits"])
    assert p["waves"] == p["workgroups"] * p["wpt"]
    _blocks_cover_tiles_once(p)
    # every group of K is streamed by exactly one K-part of each tile
    kp = p["wpt"] // 4
    cover = np.zeros(G, dtype=int)
    for s in range(p["splits"]):
        G0, G1 = s * p["gps"], min(G, (s + 1) * p["gps"])
        assert G1 > G0
        iters = -(-(G1 - G0) // kp)
        for k in range(kp):
            g0 = G0 + k * iters
            g1 = min(G1, g0 + iters)
            if g1 > g0:
                cover[g0:g1] += 1
    assert np.all(cover == 1)
    if ws is None:
        ws = qg.workspace_bytes(qg.FMT_W4A16, M, K, N)
    if p["splits"] == 1:
        assert ws == 0 or not exact_ws
    else:
        assert ws >= p["splits"] * p["mt"] * p["mb"] * 16 * N * 4 + 65536
        assert p["mt"] * p["nt"] <= 16384


@pytest.mark.parametrize("K,N", CONFIG_SHAPES)
@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 17, 32, 64, 100, 128])
def test_plan_covers_every_unit_once(K, N, M):
    _check_plan(qg.plan(qg.FMT_W4A16, M, K, N), M, K, N)


@pytest.mark.parametrize("force", [(1, 4, 1), (2, 8, 1), (2, 16, 1), (1, 16, 4), (1, 4, 3),
                                   (2, 8, 2), (2, 4, 7), (1, 8, 64)])
@pytest.mark.parametrize("M,K,N", [(16, 4096, 1024), (20, 1280, 192), (1, 28672, 8192)])
def test_forced_plans_cover_every_unit_once(force, M, K, N):
    try:
        qg.set_plan_override(*force)
        _check_plan(qg.plan(qg.FMT_W4A16, M, K, N), M, K, N)
    finally:
        qg.set_plan_override(0, 0, 0)


def test_plan_override(L):
    try:
        assert L.qgemm_set_plan_override(0, 3, 0, 0) == ERR_RANGE
        assert L.qgemm_set_plan_override(0, 1, 9, 0) == ERR_RANGE
        assert L.qgemm_set_plan_override(0, 1, 0, -1) == ERR_RANGE
        assert L.qgemm_set_plan_override(4, 0, 0, 0) == ERR_RANGE
        qg.set_plan_override(2, 8, 4)
        p = qg.plan(qg.FMT_W4A16, 16, 4096, 4096)
        assert (p["nb"], p["wpt"], p["splits"], p["gps"]) == (2, 8, 4, 8)
        qg.set_plan_override(1, 16, 64)   # more splits than groups: one group per split
        p = qg.plan(qg.FMT_W4A16, 16, 4096, 4096)
        assert p["splits"] == 32 and p["gps"] == 1 and p["wpt"] == 4
    finally:
        qg.set_plan_override()
    assert qg.plan(qg.FMT_W4A16, 16, 4096, 4096)["nb"] in (1, 2)
    # large batches use the wide kernel when N is a multiple of 256
    assert qg.plan(qg.FMT_W4A16, 128, 8192, 28672)["kernel"] == 2
    assert qg.plan(qg.FMT_W4A16, 128, 8192, 28736)["kernel"] == 1
    assert qg.plan(qg.FMT_W4A8, 128, 4096, 11008)["kernel"] == 1
    try:
        qg.set_plan_override(kernel=1)
        assert qg.plan(qg.FMT_W4A16, 128, 8192, 28672)["kernel"] == 1
        assert qg.plan(qg.FMT_W4G, 128, 8192, 28672)["kernel"] == 1
        qg.set_plan_override(kernel=3)   # the general-grid kernel with per-lane entries; 1 elsewhere
        assert qg.plan(qg.FMT_W4A16, 128, 8192, 28672)["kernel"] == 1
        assert qg.plan(qg.FMT_W4G, 1, 4096, 4096)["kernel"] == 3
        qg.set_plan_override(kernel=2, k_splits=3)
        p = qg.plan(qg.FMT_W4A16, 8, 8192, 28672)
        assert p["kernel"] == 2 and p["splits"] == 3
        # tile width of the wide kernel: nb 4 (256 columns) or 2 (128 columns)
        for nb, wpt in [(4, 16), (4, 8), (2, 8), (2, 16)]:
            qg.set_plan_override(nb, wpt, 0, kernel=2)
            p = qg.plan(qg.FMT_W4A16, 64, 8192, 28672)
            assert (p["kernel"], p["nb"], p["nt"]) == (2, nb, 28672 // (64 * nb))
            assert p["wpt"] == (wpt if nb == 4 else 8)
    finally:
        qg.set_plan_override()


def test_binding_needs_built_library_and_no_cpu_path():
    import inspect
    src = inspect.getsource(qg)
    assert "oracle" not in src and "numpy.matmul" not in src and "torch.matmul" not in src


# --------------------------------------------------------------------------- general grid
@pytest.mark.parametrize("K,N,gs", [(1024, 1024, 64), (1024, 1024, 128), (1024, 1024, 1024),
                                    (4096, 11008, 256), (11008, 4096, 11008), (384, 64, 384)])
@pytest.mark.parametrize("zeros", [False, True])
def test_w4g_packed_bytes_match_independent_layout(K, N, gs, zeros):
    assert qg.packed_bytes_w4g(K, N, gs, zeros) == layout.packed_bytes_w4g(K, N, gs, zeros)


def test_w4g_validation_without_gpu(L):
    out = ctypes.c_size_t(0)
    K, N = 1024, 1024
    for gs in (0, 32, 96, 192, 2048, -128):
        assert L.qgemm_w4g_packed_bytes(K, N, gs, 0, ctypes.byref(out)) == ERR_RANGE, gs
    assert L.qgemm_w4g_packed_bytes(K, N, 128, 2, ctypes.byref(out)) == ERR_RANGE
    assert L.qgemm_w4g_packed_bytes(K, 96, 128, 0, ctypes.byref(out)) == ERR_SHAPE
    assert L.qgemm_w4g_packed_bytes(K, N, 128, 0, None) == ERR_NULL
    nb = qg.packed_bytes_w4g(K, N, 64, True)
    codes, sc, z, blob = _fake(0x10000000), _fake(0x20000000), _fake(0x28000000), _fake(0x30000000)
    assert L.qgemm_w4g_repack(K, N, 64, None, sc, z, blob, nb, None) == ERR_NULL
    assert L.qgemm_w4g_repack(K, N, 96, codes, sc, z, blob, nb, None) == ERR_RANGE
    assert L.qgemm_w4g_repack(K, N, 64, codes, sc, None, blob, nb, None) == ERR_SIZE   # blob sized for zeros
    assert L.qgemm_w4g_repack(K, N, 64, codes, _fake(0x20000001), z, blob, nb, None) == ERR_ALIGN
    assert L.qgemm_w4g_repack(K, N, 64, codes, sc, _fake(0x30000000 + 512), blob, nb, None) == ERR_ALIAS
    A, P, C, W = _fake(0x10000000), _fake(0x20000000), _fake(0x30000000), _fake(0x40000000)
    M = 16
    ws = qg.workspace_bytes_w4g(M, K, N)
    assert L.qgemm_w4g(None, K, None, None, N, 0, K, N, 128, 0, 1, None, 0, None) == OK
    assert L.qgemm_w4g(A, K, P, C, N, M, K, N, 96, 0, 1, W, ws, None) == ERR_RANGE
    assert L.qgemm_w4g(A, K, P, C, N, M, K, N, 128, 3, 1, W, ws, None) == ERR_RANGE
    assert L.qgemm_w4g(A, K, P, C, N, M, K, N, 128, 0, 3, W, ws, None) == ERR_RANGE
    assert L.qgemm_w4g(A, K, P, C, N, M, 1000, N, 128, 0, 1, W, ws, None) == ERR_SHAPE
    assert L.qgemm_w4g(None, K, P, C, N, M, K, N, 128, 0, 2, W, ws, None) == ERR_NULL
    assert L.qgemm_w4g(A, K, P, _fake(0x10000000 + 256), N, M, K, N, 64, 1, 2, W, ws, None) == ERR_ALIAS
    st = L.qgemm_w4g(A, K, P, C, N, M, K, N, 64, 1, 2, W, ws, None)
    if st != OK:
        assert st in (ERR_HIP, ERR_DEV)


@pytest.mark.parametrize("K,N", [(4096, 11008), (11008, 4096), (1024, 1024), (8192, 28672), (28672, 8192)])
@pytest.mark.parametrize("M", [1, 16, 32, 64, 128])
@pytest.mark.parametrize("gs,zeros", [(128, True), (64, True), (64, False), (None, False)])
@pytest.mark.parametrize("act", [qg.DT_F16, qg.DT_BF16])
def test_w4g_plan_covers_every_unit_once(K, N, M, gs, zeros, act):
    gs = gs or K   # None: one group per column
    p = qg.plan(qg.FMT_W4G, M, K, N, group_size=gs, zeros=zeros, act_dtype=act)
    if act == qg.DT_BF16 or N % 256:
        assert p["kernel"] in (1, 3)   # grid entries staged in LDS / loaded per lane
    else:
        assert p["kernel"] in (1, 2, 3)   # fp16 may take the wide kernel
    if p["kernel"] == 2:
        assert M >= 33
        assert p == {k: v for k, v in qg.plan(qg.FMT_W4A16, M, K, N).items()}   # the W4A16 wide plan
    # the workspace query covers every grid and type, so it may exceed this plan's need
    info = qg.plan_info(qg.FMT_W4G, M, K, N, group_size=gs, zeros=zeros, act_dtype=act)
    assert info["ws_bytes"] <= qg.workspace_bytes_w4g(M, K, N)
    _check_plan(p, M, K, N, ws=qg.workspace_bytes_w4g(M, K, N), exact_ws=False)
    if (gs, zeros, act) == (128, True, qg.DT_F16):
        assert p == qg.plan(qg.FMT_W4G, M, K, N)   # the grid qgemm_plan reports


def test_w4g_plan_validation(L):
    out = (ctypes.c_int64 * 10)()
    assert L.qgemm_w4g_plan(16, 4096, 4096, 128, 1, 1, None) == ERR_NULL
    assert L.qgemm_w4g_plan(16, 4096, 4096, 96, 1, 1, out) == ERR_RANGE
    assert L.qgemm_w4g_plan(16, 4096, 4096, 128, 2, 1, out) == ERR_RANGE
    assert L.qgemm_w4g_plan(16, 4096, 4096, 128, 1, 3, out) == ERR_RANGE   # activation type
    assert L.qgemm_w4g_plan(16, 4096, 4096, 8192, 0, 1, out) == ERR_RANGE   # does not divide K
    assert L.qgemm_w4g_plan(0, 4096, 4096, 128, 1, 1, out) == ERR_SHAPE
    assert L.qgemm_w4g_plan(16, 4096, 4096, 4096, 0, 2, out) == OK
    out12 = (ctypes.c_int64 * 12)()
    assert L.qgemm_plan_info(qg.FMT_W4G, 16, 4096, 4096, 4, 128, 1, 0, out12) == ERR_RANGE
    assert L.qgemm_plan_info(qg.FMT_W4A16, 16, 4096, 4096, 4, 128, 1, 0, out12) == OK   # ignored there


def _w4g_lds_bytes(p, K, gs, zeros):
    """Dynamic LDS of a general-grid streaming launch, written from the kernel's
    layout: staged grid entries (kernel 1: per column and chunk of the split,
    two entries for group length 64, else one; 4 bytes with zero points, else
    2), then K-parts x 3 activation slots of 4 KB per 16 rows; the reduction
    buffer reuses the start. The wide kernel (kernel 2) holds only its
    activation ring: K-parts (of 8 waves for 256-column tiles, of 4 for
    128-column tiles) x 4 slots of 16 KB (64 rows x 128 k fp16)."""
    if p["kernel"] == 2:
        return (p["wpt"] // (2 * p["nb"])) * 4 * 16 * 1024
    ng = min(K // 128, p["gps"])
    nb_blocks, kp = 4 * p["nb"], p["wpt"] // 4
    extra = ng * nb_blocks * 16 * (2 if gs == 64 else 1) * (4 if zeros else 2) if p["kernel"] == 1 else 0
    rings = (extra + 255) // 256 * 256 + kp * 3 * p["mb"] * 4 * 1024
    return max(rings, kp * 4 * p["mb"] * p["nb"] * 1024)


@pytest.mark.parametrize("K,N", [(28672, 8192), (8192, 28672), (11008, 4096), (57344, 8192)])
def test_w4g_plans_leave_room_for_static_lds(K, N):
    # A launch's LDS is this dynamic part plus the kernel's 16-byte arrival flag;
    # a dynamic part of the full 160 KB made the queue abort (28672 x 8192, M = 64).
    for gs, zeros in [(64, True), (64, False), (128, True), (128, False)]:
        for act in (qg.DT_F16, qg.DT_BF16):
            for M in range(1, 129, 7):
                p = qg.plan(qg.FMT_W4G, M, K, N, group_size=gs, zeros=zeros, act_dtype=act)
                lds = _w4g_lds_bytes(p, K, gs, zeros)
                assert lds <= 160 * 1024 - 256, (M, gs, zeros, act, p)
                info = qg.plan_info(qg.FMT_W4G, M, K, N, group_size=gs, zeros=zeros, act_dtype=act)
                assert info["lds_bytes"] == lds, (M, gs, zeros, act, p, info)


# --------------------------------------------------------------------------- 2:4 sparse
@pytest.mark.parametrize("K,N", CONFIG_SHAPES + [(128, 64), (1152, 320)])
def test_sp24_packed_bytes_match_independent_layout(K, N):
    assert qg.packed_bytes(qg.FMT_W4A16_SP24, K, N) == layout.packed_bytes(layout.FMT_SP24, K, N)


def test_sp24_validation_without_gpu(L):
    A, P, C, W = _fake(0x10000000), _fake(0x20000000), _fake(0x30000000), _fake(0x40000000)
    M, K, N = 16, 4096, 4096
    ws = qg.workspace_bytes(qg.FMT_W4A16_SP24, M, K, N)
    assert L.qgemm_w4a16_sp24(None, K, None, None, N, 0, K, N, None, 0, None) == OK
    assert L.qgemm_w4a16_sp24(None, K, P, C, N, M, K, N, W, ws, None) == ERR_NULL
    assert L.qgemm_w4a16_sp24(A, K, P, C, N, M, 1000, N, W, ws, None) == ERR_SHAPE
    assert L.qgemm_w4a16_sp24(A, K + 4, P, C, N, M, K, N, W, ws, None) == ERR_ALIGN
    assert L.qgemm_w4a16_sp24(A, K, P, _fake(0x10000000 + 256), N, M, K, N, W, ws, None) == ERR_ALIAS
    nb = qg.packed_bytes(qg.FMT_W4A16_SP24, K, N)
    assert L.qgemm_repack(5, K, N, _fake(0x10000000), _fake(0x20000000), None, None, _fake(0x30000000),
                          nb - 256, None) == ERR_SIZE
    st = L.qgemm_w4a16_sp24(A, K, P, C, N, M, K, N, W, ws, None)
    if st != OK:
        assert st in (ERR_HIP, ERR_DEV)


@pytest.mark.parametrize("K,N", [(4096, 11008), (8192, 28672), (28672, 8192), (1024, 1024)])
@pytest.mark.parametrize("M", [1, 16, 33, 128])
def test_sp24_plan_covers_every_unit_once(K, N, M):
    p = qg.plan(qg.FMT_W4A16_SP24, M, K, N)
    assert p["kernel"] == 1
    _check_plan(p, M, K, N, ws=qg.workspace_bytes(qg.FMT_W4A16_SP24, M, K, N))


# --------------------------------------------------------------------------- bit planes
@pytest.mark.parametrize("K,N", [(1024, 1024), (4096, 11008), (11008, 4096), (128, 64)])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 8])
def test_bitplane_packed_bytes_match_independent_layout(K, N, bits):
    assert qg.packed_bytes_bitplane(K, N, bits) == layout.packed_bytes_bitplane(K, N, bits)


def test_bitplane_validation_without_gpu(L):
    out = ctypes.c_size_t(0)
    assert L.qgemm_bitplane_packed_bytes(1024, 1024, 0, ctypes.byref(out)) == ERR_RANGE
    assert L.qgemm_bitplane_packed_bytes(1024, 1024, 9, ctypes.byref(out)) == ERR_RANGE
    assert L.qgemm_bitplane_packed_bytes(65536, 64, 4, ctypes.byref(out)) == OK
    assert L.qgemm_bitplane_packed_bytes(65536 + 128, 64, 4, ctypes.byref(out)) == ERR_SHAPE
    A, S, P, C, W = (_fake(0x10000000), _fake(0x50000000), _fake(0x20000000), _fake(0x30000000),
                     _fake(0x40000000))
    M, K, N = 16, 4096, 4096
    ws = qg.workspace_bytes_bitplane(M, K, N, 3)
    assert L.qgemm_bitplane_a8(None, K, None, None, None, N, None, 0, K, N, 3, None, 0, None) == OK
    assert L.qgemm_bitplane_a8(A, K, None, P, C, N, None, M, K, N, 3, W, ws, None) == ERR_NULL   # a_scale
    assert L.qgemm_bitplane_a8(A, K, S, P, C, N, None, M, K, N, 0, W, ws, None) == ERR_RANGE
    assert L.qgemm_bitplane_a8(A, K + 8, S, P, C, N, None, M, K, N, 3, W, ws, None) == ERR_ALIGN
    assert L.qgemm_bitplane_a8(A, K, S, P, C, N, _fake(0x30000000), M, K, N, 3, W, ws, None) == ERR_ALIAS
    nb = qg.packed_bytes_bitplane(K, N, 3)
    assert L.qgemm_bitplane_repack(K, N, 3, None, S, P, nb, None) == ERR_NULL
    assert L.qgemm_bitplane_repack(K, N, 3, A, S, P, nb - 256, None) == ERR_SIZE
    assert L.qgemm_bitplane_repack(K, N, 9, A, S, P, nb, None) == ERR_RANGE
    st = L.qgemm_bitplane_a8(A, K, S, P, C, N, None, M, K, N, 3, W, ws, None)
    if st != OK:
        assert st in (ERR_HIP, ERR_DEV)


def test_bitplane_plan_validation(L):
    out = (ctypes.c_int64 * 10)()
    assert L.qgemm_bitplane_plan(16, 4096, 4096, 0, out) == ERR_RANGE
    assert L.qgemm_bitplane_plan(16, 4096, 4096, 9, out) == ERR_RANGE
    assert L.qgemm_bitplane_plan(16, 4096, 4096, 4, None) == ERR_NULL
    assert L.qgemm_bitplane_plan(0, 4096, 4096, 4, out) == ERR_SHAPE
    assert L.qgemm_bitplane_plan(16, 65536 + 128, 64, 4, out) == ERR_SHAPE
    assert L.qgemm_bitplane_plan(16, 4096, 4096 + 32, 4, out) == ERR_SHAPE


@pytest.mark.parametrize("bits", [1, 2, 4, 6, 8])
@pytest.mark.parametrize("K,N", [(1024, 1024), (4096, 11008), (11008, 4096), (8192, 28672), (28672, 8192)])
@pytest.mark.parametrize("M", [1, 16, 32, 64, 128])
def test_bitplane_plan_covers_every_unit_once(K, N, M, bits):
    p = qg.plan(qg.FMT_BITPLANE, M, K, N, bits=bits)
    assert p["kernel"] == 1
    _check_plan(p, M, K, N, ws=qg.workspace_bytes_bitplane(M, K, N, bits))



_LDS_BUDGET = 160 * 1024 - 256
_FORMATS = [(qg.FMT_W4A16, {}), (qg.FMT_W4A8, {}), (qg.FMT_W2W4, {}), (qg.FMT_W4A16_SP24, {}),
            (qg.FMT_W4G, {"group_size": 64, "zeros": True}), (qg.FMT_W4G, {"group_size": 128, "zeros": False}),
            (qg.FMT_BITPLANE, {"bits": 8}), (qg.FMT_BITPLANE, {"bits": 1})]


@pytest.mark.parametrize("fmt,kw", _FORMATS)
@pytest.mark.parametrize("K,N", [(262144, 4160), (57344, 8192), (1048576, 64), (128, 1048576), (1024, 1024),
                                 (28672, 8192)])
def test_every_automatic_plan_fits_lds_and_covers_the_layer(fmt, kw, K, N):
    # long K with many tiles (M up to 65535) once forced a single k-split whose
    # staged scales or grid entries outgrew the LDS; every automatic plan must
    # now fit, cover every unit once, and size its counters for its tiles
    if fmt == qg.FMT_W4A8 and K > 16384:
        pytest.skip("W4A8 accepts K <= 16384")
    if fmt == qg.FMT_BITPLANE and K > 65536:
        pytest.skip("bit-plane accepts K <= 65536")
    for M in (1, 16, 17, 64, 128, 1000, 16384, 65535):
        p = qg.plan_info(fmt, M, K, N, **kw)
        assert 0 < p["lds_bytes"] <= _LDS_BUDGET, (M, p)
        G = K // 128
        assert p["splits"] * p["gps"] >= G and (p["splits"] - 1) * p["gps"] < G, (M, p)
        tiles = p["mt"] * p["nt"]
        assert p["workgroups"] == _launch_workgroups(p["nt"], p["mt"], p["splits"])
        if p["splits"] > 1:
            assert p["ws_bytes"] >= max(65536, 4 * tiles), (M, p)


def test_counter_region_grows_past_the_fixed_region():
    # W4G 16384 x 57344 x 8192 with group 64 and zero points: the case that
    # once returned a plan needing 253,952 B of staged entries (bf16
    # activations: the streaming kernel, which fp16 calls of this width leave
    # for the wide kernel)
    p = qg.plan_info(qg.FMT_W4G, 16384, 57344, 8192, group_size=64, zeros=True, act_dtype=qg.DT_BF16)
    assert p["lds_bytes"] <= _LDS_BUDGET
    tiles = p["mt"] * p["nt"]
    assert tiles > 16384 and p["splits"] > 1
    assert p["ws_bytes"] >= (tiles * 4 + 255) // 256 * 256
    assert qg.workspace_bytes_w4g(16384, 57344, 8192) >= p["ws_bytes"]


def test_w4g_takes_the_wide_kernel_on_70b_layers_with_fp16_activations():
    # the wide kernel reads fp16 activations only: bf16 calls stay on the
    # streaming kernels
    for K, N in [(8192, 28672), (28672, 8192)]:
        for M in (48, 64, 128):
            for gs, zeros in [(64, True), (128, True), (128, False), (K, True)]:
                assert qg.plan(qg.FMT_W4G, M, K, N, group_size=gs, zeros=zeros)["kernel"] == 2
                assert qg.plan(qg.FMT_W4G, M, K, N, group_size=gs, zeros=zeros, act_dtype=qg.DT_BF16)["kernel"] != 2


def test_wide_plans_take_128_column_tiles_where_they_save_k_splits():
    # the 70B layers at M = 33-64 and 7B-class layers at M = 96-128 (8-wave
    # 256-column plans with k-splits); M > 64 on the 70B layers keeps the
    # 16-wave 256-column tiles
    for (K, N, M, nb, splits) in [(8192, 28672, 33, 2, 1), (8192, 28672, 64, 2, 1), (28672, 8192, 48, 2, 4),
                                  (28672, 8192, 64, 2, 4), (4096, 11008, 128, 2, 1), (8192, 28672, 128, 4, 1),
                                  (28672, 8192, 128, 4, 4), (8192, 28672, 96, 4, 1)]:
        p = qg.plan(qg.FMT_W4A16, M, K, N)
        assert (p["kernel"], p["nb"], p["splits"]) == (2, nb, splits), (K, N, M, p)
        assert qg.plan(qg.FMT_W4G, M, K, N) == p
        _check_plan(p, M, K, N)


def test_unsplit_plans_on_7b_class_layers():
    # layers whose tiles cover half to all of the CUs: one workgroup per tile and
    # no k-split at M = 17-32 (W4A16, one 32-row tile), M = 33-64 (two 32-row
    # tiles of W4A16, W4A8 and the 2:4 format) and M <= 16 (2:4)
    K, N = 4096, 11008
    for M in (17, 24, 32):
        p = qg.plan(qg.FMT_W4A16, M, K, N)
        assert (p["kernel"], p["mb"], p["nb"], p["wpt"], p["splits"]) == (1, 2, 1, 16, 1), (M, p)
    for fmt, wpt in [(qg.FMT_W4A16, 8), (qg.FMT_W4A8, 16), (qg.FMT_W4A16_SP24, 16)]:
        for M in (33, 48, 64):
            p = qg.plan(fmt, M, K, N)
            assert (p["kernel"], p["mb"], p["nb"], p["wpt"], p["splits"], p["mt"]) == (1, 2, 2, wpt, 1, 2), (fmt, M, p)
            _check_plan(p, M, K, N)
    p = qg.plan(qg.FMT_W4A16_SP24, 16, K, N)
    assert (p["nb"], p["wpt"], p["splits"]) == (1, 16, 1)
    # W4A16 layers below 2^27 weights leave the wide kernel for that plan
    assert qg.plan(qg.FMT_W4A16, 48, 4096, 14336)["kernel"] == 1
    # the 70B layers keep theirs: the wide kernel, and k-splits where each CU
    # would stream far more than its share
    assert qg.plan(qg.FMT_W4A16, 48, 28672, 8192)["kernel"] == 2
    assert qg.plan(qg.FMT_W4A16_SP24, 48, 28672, 8192)["splits"] > 1
    assert qg.plan(qg.FMT_W4A16, 16, 28672, 8192)["splits"] > 1
