"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: repacked blobs byte-identical to the independent layout oracle; W4A8 int32
accumulators bit-identical; one-hot activations reproduce fp16((q - z) * s)
bit-exactly; every fp16 GEMM output within
    max|e| <= 2e-3 * sqrt(K) * rms(C_ref)  and  ||e||_F / ||C_ref||_F <= 1e-3.
Full-size layers are checked on sampled columns the oracle computes one by one,
in the same launch configuration the benchmark times.
"""

import sys

import numpy as np
import pytest
import torch

import bit_weight_quantized_qgemm_amd as qg
from oracle import compare, layout, ref
from synth import gen

from sampling import block_cols

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _t(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def upload_w4a16(p):
    return qg.repack_w4a16(_t(p["codes"].view(np.int32)), _t(p["scales"]))


def upload_w4a8(p):
    return qg.repack_w4a8(_t(p["codes"].view(np.int32)), _t(p["group_scales"]), _t(p["chan_scales"]))


def upload_w2w4(p):
    return qg.repack_w2w4(_t(p["codes"]), _t(p["scales"]), p["bitmap"])


def _ok(C_gpu, C_ref, K, what):
    r = compare.check_fp16(C_gpu, C_ref, K)
    assert r["ok"], (what, r)
    return r


@pytest.fixture(autouse=True)
def _reset_plan():
    qg.set_plan_override()
    yield
    qg.set_plan_override()


# ----------------------------------------------------------------------------- repack bytes
@pytest.mark.parametrize("K,N", [(128, 64), (1152, 320), (1024, 1024), (4096, 11008)])
def test_repack_w4a16_bytes(K, N):
    _say("repack w4a16", K, N)
    p = gen.w4a16_problem(1, K, N, seed=K ^ N, activations=False)
    blob = upload_w4a16(p).cpu().numpy().tobytes()
    assert blob == layout.blob_w4a16(p["codes"], p["scales"])


@pytest.mark.parametrize("K,N", [(128, 64), (1152, 320), (4096, 11008)])
def test_repack_w4a8_bytes(K, N):
    _say("repack w4a8", K, N)
    p = gen.w4a8_problem(1, K, N, seed=3)
    blob = upload_w4a8(p).cpu().numpy().tobytes()
    assert blob == layout.blob_w4a8(p["codes"], p["group_scales"], p["chan_scales"])


@pytest.mark.parametrize("K,N,frac", [(128, 64, 0.1), (1152, 320, 0.3), (4096, 4096, 0.1),
                                      (1024, 256, 0.0), (1024, 256, 1.0)])
def test_repack_w2w4_bytes(K, N, frac):
    _say("repack w2w4", K, N, frac)
    p = gen.w2w4_problem(1, K, N, seed=5, frac4=frac)
    blob = upload_w2w4(p).cpu().numpy().tobytes()
    assert blob == layout.blob_w2w4(p["codes"], p["bitmap"], p["scales"])


# ----------------------------------------------------------------------------- W4A16
def _one_hot(M, K, rng):
    ks = rng.choice(K, size=M, replace=False)
    A = np.zeros((M, K), dtype=np.float16)
    A[np.arange(M), ks] = 1.0
    return A, ks


@pytest.mark.parametrize("M,K,N,force", [(16, 1024, 1024, None), (5, 4096, 256, (1, 8, 2)),
                                         (32, 1152, 384, (2, 16, 1)), (20, 8192, 128, (2, 4, 5))])
def test_w4a16_one_hot_bit_exact(M, K, N, force):
    _say("w4a16 one-hot", M, K, N, force)
    rng = np.random.default_rng(M * 7 + K)
    p = gen.w4a16_problem(1, K, N, seed=M + K, activations=False)
    A, ks = _one_hot(M, K, rng)
    if force:
        qg.set_plan_override(*force)
    blob = upload_w4a16(p)
    C = qg.w4a16(_t(A), blob, K, N).cpu().numpy()
    q = ref.unpack_u4(p["codes"])
    expect = ((q[ks] - 8).astype(np.float64) * p["scales"][ks // 128].astype(np.float64)).astype(np.float16)
    assert np.array_equal(C.view(np.uint16), expect.view(np.uint16))


def test_w4a16_identity_block_and_zero_point():
    _say("w4a16 identity / constant 8")
    K, N = 1024, 512
    p = gen.w4a16_problem(1, K, N, seed=2, activations=False)
    A = np.zeros((16, K), dtype=np.float16)
    A[:, 256:272] = np.eye(16, dtype=np.float16)
    C = qg.w4a16(_t(A), upload_w4a16(p), K, N).cpu().numpy()
    q = ref.unpack_u4(p["codes"])
    expect = ((q[256:272] - 8) * p["scales"][2].astype(np.float64)).astype(np.float16)
    assert np.array_equal(C.view(np.uint16), expect.view(np.uint16))
    # constant code 8 gives exactly zero for any activations
    codes8 = gen.pack_nibbles_u32(np.full((K, N), 8, dtype=np.uint8))
    blob8 = qg.repack_w4a16(_t(codes8.view(np.int32)), _t(p["scales"]))
    A2 = gen.w4a16_problem(16, K, N, seed=3, weights=False)["A"]
    C8 = qg.w4a16(_t(A2), blob8, K, N).cpu().numpy()
    assert np.all(C8 == 0)


def test_w4a16_config_small():
    _say("w4a16 M=16 K=1024 N=1024")
    p = gen.w4a16_problem(16, 1024, 1024, seed=0)
    blob = upload_w4a16(p)
    A = _t(p["A"])
    C1 = qg.w4a16(A, blob, 1024, 1024)
    C2 = qg.w4a16(A, blob, 1024, 1024)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    _ok(C1.cpu().numpy(), ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), 1024, "cfg0")


@pytest.mark.parametrize("K,N", [(4096, 4096), (4096, 11008), (11008, 4096)])
def test_w4a16_7b_layers(K, N):
    p = gen.w4a16_problem(128, K, N, seed=1)
    blob = upload_w4a16(p)
    Cref = ref.gemm_w4a16(p["A"], p["codes"], p["scales"])
    for M in (1, 16, 32, 64, 128):
        _say("w4a16 7B layer", M, K, N, qg.plan(qg.FMT_W4A16, M, K, N))
        A = _t(p["A"][:M])
        C = qg.w4a16(A, blob, K, N).cpu().numpy()
        _ok(C, Cref[:M], K, (M, K, N))


@pytest.mark.parametrize("K,N", [(8192, 28672), (28672, 8192)])
def test_w4a16_70b_layer_sampled(K, N):
    p = gen.w4a16_problem(128, K, N, seed=2)
    blob = upload_w4a16(p)
    # one column of every 16-column block (every tile and column wave of the
    # launches the benchmark times)
    cols = block_cols(N, seed=K)
    Cref = ref.gemm_w4a16(p["A"], p["codes"], p["scales"], cols=cols)
    for M in (1, 2, 4, 8, 16, 32, 64, 128):
        _say("w4a16 70B layer", M, K, N, qg.plan(qg.FMT_W4A16, M, K, N))
        C = qg.w4a16(_t(p["A"][:M]), blob, K, N).cpu().numpy()
        assert np.all(np.isfinite(C))
        _ok(C[:, cols], Cref[:M], K, (M, K, N))


@pytest.mark.parametrize("M", [1, 2, 3, 5, 7, 15, 17, 31, 33, 47, 100])
def test_w4a16_ragged_m(M):
    K, N = 1280, 192                     # G = 10: a partial 8-group scale block
    _say("w4a16 ragged", M, K, N)
    p = gen.w4a16_problem(M, K, N, seed=M)
    C = qg.w4a16(_t(p["A"]), upload_w4a16(p), K, N).cpu().numpy()
    _ok(C, ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), K, M)


@pytest.mark.parametrize("force", [(1, 4, 1), (2, 8, 1), (2, 16, 1), (1, 16, 4), (1, 4, 3),
                                   (2, 8, 2), (2, 4, 7), (1, 8, 32), (0, 0, 0)])
@pytest.mark.parametrize("M", [16, 20])
def test_w4a16_forced_splits(force, M):
    K, N = 4096, 1024
    _say("w4a16 forced", force, M, qg.plan(qg.FMT_W4A16, M, K, N))
    p = gen.w4a16_problem(M, K, N, seed=11)
    blob = upload_w4a16(p)
    qg.set_plan_override(*force)
    A = _t(p["A"])
    C1 = qg.w4a16(A, blob, K, N)
    C2 = qg.w4a16(A, blob, K, N)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    _ok(C1.cpu().numpy(), ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), K, (force, M))


@pytest.mark.parametrize("M,N,force", [(100, 704, (1, 8, 3)), (100, 1408, (2, 8, 3)), (64, 704, (1, 4, 5)),
                                     (129, 1408, (2, 16, 1)), (50, 704, (1, 8, 0))])
def test_row_tiles_block_order(M, N, force):
    """Several row tiles: their block indices follow the XCD-grouped order, with
    (column tile, split) pairs in whole groups of 8 and a ragged rest."""
    K = 2048
    qg.set_plan_override(*force)
    pl = qg.plan(qg.FMT_W4A16, M, K, N)
    pairs = pl["nt"] * pl["splits"]
    _say("row-tile order", M, N, force, pl)
    assert pl["mt"] > 1 and pairs >= 8
    p = gen.w4a16_problem(M, K, N, seed=M + N)
    A = _t(p["A"])
    blob = upload_w4a16(p)
    C1 = qg.w4a16(A, blob, K, N)
    C2 = qg.w4a16(A, blob, K, N)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    _ok(C1.cpu().numpy(), ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), K, ("row tiles", M, N, force))
    # W4A8 under the same forced decomposition: exact accumulators
    q = gen.w4a8_problem(M, K, N, seed=M + N + 1)
    C, acc = _w4a8_run(q)
    acc_ref, C_ref = ref.gemm_w4a8(q["A"], q["codes"], q["group_scales"], q["a_scale"], q["chan_scales"])
    assert np.array_equal(acc.astype(np.int64), acc_ref)
    _ok(C, C_ref, K, ("row tiles w4a8", M, N, force))


def test_w4a16_strided_and_guard_bands():
    _say("w4a16 strides + guards")
    M, K, N = 9, 1024, 256
    p = gen.w4a16_problem(M, K, N, seed=4)
    blob = upload_w4a16(p)
    Abig = torch.zeros((M, K + 64), dtype=torch.float16, device=DEV)
    Abig[:, :K] = _t(p["A"])
    sentinel = -12345.0
    Cbig = torch.full((M + 2, N + 64), sentinel, dtype=torch.float16, device=DEV)
    out = Cbig[1:M + 1, :N]
    L = qg.lib()
    import ctypes
    ws = torch.zeros(max(1, qg.workspace_bytes(qg.FMT_W4A16, M, K, N)), dtype=torch.uint8, device=DEV)
    st = L.qgemm_w4a16(ctypes.c_void_p(Abig.data_ptr()), K + 64, ctypes.c_void_p(blob.data_ptr()),
                       ctypes.c_void_p(out.data_ptr()), N + 64, M, K, N,
                       ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    Cb = Cbig.cpu().numpy()
    _ok(Cb[1:M + 1, :N], ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), K, "strided")
    assert np.all(Cb[0] == sentinel) and np.all(Cb[M + 1] == sentinel)
    assert np.all(Cb[:, N:] == sentinel)


def test_w4a16_minimal_and_empty():
    _say("w4a16 minimal")
    p = gen.w4a16_problem(1, 128, 64, seed=9)
    blob = upload_w4a16(p)
    C = qg.w4a16(_t(p["A"]), blob, 128, 64).cpu().numpy()
    _ok(C, ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), 128, "K=128,N=64")
    empty = qg.w4a16(torch.zeros((0, 128), dtype=torch.float16, device=DEV), blob, 128, 64)
    assert empty.shape == (0, 64)


# ----------------------------------------------------------------------------- W4A8
def _w4a8_run(p, M=None, acc=True):
    K, N = p["K"], p["N"]
    A = p["A"] if M is None else p["A"][:M]
    a_s = p["a_scale"] if M is None else p["a_scale"][:M]
    blob = upload_w4a8(p)
    acc_out = torch.empty((A.shape[0], N), dtype=torch.int32, device=DEV) if acc else None
    C = qg.w4a8(_t(A), _t(a_s), blob, K, N, acc_out=acc_out)
    return C.cpu().numpy(), (acc_out.cpu().numpy() if acc else None)


def test_w4a8_70b_up_projection_sampled():
    """W4A8 on the 70B-class up projection (K = 8192, the largest K of the
    format's exact-accumulator range that the 70B layers use) in its automatic
    plans: exact int32 accumulators on one column per 16-column block."""
    K, N = 8192, 28672
    p = gen.w4a8_problem(64, K, N, seed=4)
    blob = upload_w4a8(p)
    cols = block_cols(N, seed=K + 2)
    acc_ref, C_ref = ref.gemm_w4a8(p["A"], p["codes"], p["group_scales"], p["a_scale"], p["chan_scales"],
                                   cols=cols)
    for M in (1, 16, 32, 64):
        _say("w4a8 70B up", M, qg.plan(qg.FMT_W4A8, M, K, N))
        acc_out = torch.empty((M, N), dtype=torch.int32, device=DEV)
        C = qg.w4a8(_t(p["A"][:M]), _t(p["a_scale"][:M]), blob, K, N, acc_out=acc_out).cpu().numpy()
        acc = acc_out.cpu().numpy()
        assert np.array_equal(acc[:, cols].astype(np.int64), acc_ref[:M])
        _ok(C[:, cols], C_ref[:M], K, ("w4a8 70B", M))


@pytest.mark.parametrize("M", [16, 64, 128])
def test_w4a8_config_layer(M):
    K, N = 4096, 11008
    _say("w4a8", M, K, N, qg.plan(qg.FMT_W4A8, M, K, N))
    p = gen.w4a8_problem(M, K, N, seed=0)
    C, acc = _w4a8_run(p)
    acc_ref, C_ref = ref.gemm_w4a8(p["A"], p["codes"], p["group_scales"], p["a_scale"], p["chan_scales"])
    assert np.array_equal(acc.astype(np.int64), acc_ref)
    _ok(C, C_ref, K, ("w4a8", M))


@pytest.mark.parametrize("M,force", [(1, None), (3, (1, 8, 2)), (17, (2, 16, 1)), (40, (2, 4, 4)),
                                     (33, None), (9, (1, 4, 16))])
def test_w4a8_ragged_and_splits(M, force):
    K, N = 2048, 320
    _say("w4a8 ragged", M, force)
    p = gen.w4a8_problem(M, K, N, seed=M)
    if force:
        qg.set_plan_override(*force)
    C, acc = _w4a8_run(p)
    acc_ref, C_ref = ref.gemm_w4a8(p["A"], p["codes"], p["group_scales"], p["a_scale"], p["chan_scales"])
    assert np.array_equal(acc.astype(np.int64), acc_ref)
    _ok(C, C_ref, K, ("w4a8 ragged", M))


def test_w4a8_one_hot_and_extremes():
    _say("w4a8 one-hot + extremes")
    K, N = 1024, 128
    p = gen.w4a8_problem(8, K, N, seed=6)
    rng = np.random.default_rng(1)
    ks = rng.choice(K, size=8, replace=False)
    A = np.zeros((8, K), dtype=np.int8)
    A[np.arange(8), ks] = 1
    p1 = dict(p, A=A)
    _, acc = _w4a8_run(p1)
    Wi = ref.w4a8_weights_int(p["codes"], p["group_scales"])
    assert np.array_equal(acc.astype(np.int64), Wi[ks])
    # extreme values: A = -128, q = -8, s_g = 127 or -128 everywhere
    K2 = 16384
    ext = {"K": K2, "N": 64, "A": np.full((2, K2), -128, dtype=np.int8),
           "a_scale": np.full(2, 1e-4, dtype=np.float16),
           "codes": gen.pack_nibbles_u32(np.full((K2, 64), 8, dtype=np.uint8)),
           "group_scales": np.full((K2 // 128, 64), 127, dtype=np.int8),
           "chan_scales": np.full(64, 1e-4, dtype=np.float16)}
    ext["group_scales"][:, 1::2] = -128
    _, acc2 = _w4a8_run(ext)
    acc_ref = ref.w4a8_acc(ext["A"], ext["codes"], ext["group_scales"])
    assert np.array_equal(acc2.astype(np.int64), acc_ref)


# ----------------------------------------------------------------------------- mixed 2/4
@pytest.mark.parametrize("M", [1, 16, 64])
def test_w2w4_config_layer(M):
    K, N = 4096, 4096
    _say("w2w4", M, K, N, qg.plan(qg.FMT_W2W4, M, K, N))
    p = gen.w2w4_problem(M, K, N, seed=0)
    C = qg.w2w4_mixed(_t(p["A"]), upload_w2w4(p), K, N).cpu().numpy()
    _ok(C, ref.gemm_w2w4(p["A"], p["codes"], p["bitmap"], p["scales"]), K, ("w2w4", M))


@pytest.mark.parametrize("K,N", [(8192, 28672), (28672, 8192)])
def test_w2w4_70b_layer_sampled(K, N):
    """The mixed format on the 70B-class layer in its automatic plans (16-wave
    two-block tiles on the up projection at M <= 32), one column per 16-column
    block."""
    p = gen.w2w4_problem(64, K, N, seed=3)
    blob = upload_w2w4(p)
    cols = block_cols(N, seed=K + 1)
    Cref = ref.gemm_w2w4(p["A"], p["codes"], p["bitmap"], p["scales"], cols=cols)
    for M in (1, 16, 32, 64):
        _say("w2w4 70B layer", M, K, N, qg.plan(qg.FMT_W2W4, M, K, N))
        C = qg.w2w4_mixed(_t(p["A"][:M]), blob, K, N).cpu().numpy()
        assert np.all(np.isfinite(C))
        _ok(C[:, cols], Cref[:M], K, ("w2w4 70B", M, K, N))


@pytest.mark.parametrize("M,frac,force", [(3, 0.0, None), (17, 1.0, None), (20, 0.3, (1, 8, 2)),
                                          (9, 0.5, (2, 4, 4)), (33, 0.1, (2, 16, 1)),
                                          (5, 0.2, (1, 4, 16))])
def test_w2w4_ragged_and_extremes(M, frac, force):
    K, N = 2048, 320
    _say("w2w4 ragged", M, frac, force)
    p = gen.w2w4_problem(M, K, N, seed=M, frac4=frac)
    if force:
        qg.set_plan_override(*force)
    C = qg.w2w4_mixed(_t(p["A"]), upload_w2w4(p), K, N).cpu().numpy()
    _ok(C, ref.gemm_w2w4(p["A"], p["codes"], p["bitmap"], p["scales"]), K, ("w2w4", M, frac))


def test_w2w4_one_hot_and_all_four_bit_equals_w4a16():
    _say("w2w4 one-hot / all-4-bit")
    K, N, M = 1024, 512, 16
    p = gen.w2w4_problem(M, K, N, seed=8, frac4=0.25)
    rng = np.random.default_rng(2)
    A, ks = _one_hot(M, K, rng)
    C = qg.w2w4_mixed(_t(A), upload_w2w4(p), K, N).cpu().numpy()
    W = ref.dequant_w2w4(p["codes"], p["bitmap"], p["scales"])
    assert np.array_equal(C.view(np.uint16), W[ks].astype(np.float16).view(np.uint16))
    # every group 4-bit: same words, same plan -> bit-identical to the W4A16 kernel
    full = gen.w2w4_problem(M, K, N, seed=8, mask=np.ones((K // 128, N), dtype=bool))
    codes32 = gen.pack_nibbles_u32(full["codes"])
    blob16 = qg.repack_w4a16(_t(codes32.view(np.int32)), _t(full["scales"]))
    Cm = qg.w2w4_mixed(_t(full["A"]), upload_w2w4(full), K, N)
    C16 = qg.w4a16(_t(full["A"]), blob16, K, N)
    torch.cuda.synchronize()
    assert torch.equal(Cm, C16)


def test_workspace_shared_across_plans():
    # one workspace serves a sequence of calls whose plans differ in tiles and
    # splits: each call must find the counter region zero again
    _say("workspace shared across plans")
    ws = qg.Workspace()
    seq = [(5, 4096, 256, (1, 8, 4)), (20, 8192, 128, (2, 4, 8)), (1, 4096, 4096, None),
           (16, 2048, 1024, (1, 4, 16)), (3, 4096, 4096, (2, 16, 2)), (7, 1024, 64, None),
           (40, 2048, 512, (0, 0, 3, 2)), (9, 1024, 256, (0, 0, 2, 1))]
    for M, K, N, force in seq:
        qg.set_plan_override(*(force or (0, 0, 0)))
        p = gen.w4a16_problem(M, K, N, seed=M + N)
        C = qg.w4a16(_t(p["A"]), upload_w4a16(p), K, N, workspace=ws).cpu().numpy()
        _ok(C, ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), K, ("shared ws", M, K, N, force))


# ----------------------------------------------------------------------------- wide W4A16 kernel
# tiles of the wide kernel as (64-column units, waves per workgroup): 256
# columns with 8 waves or 16 (two K-parts of 8), 128 columns with 8 (two K-parts of 4)
WIDE_TILES = [(4, 8), (4, 16), (2, 8)]


@pytest.mark.parametrize("nb,wpt", WIDE_TILES)
@pytest.mark.parametrize("M,K,N,splits", [(48, 1024, 512, 0), (128, 2048, 256, 3), (130, 1280, 512, 0),
                                          (64, 4096, 768, 5), (48, 128, 256, 0), (40, 384, 256, 0)])
def test_w4a16_wide_one_hot_bit_exact(M, K, N, splits, nb, wpt):
    _say("w4a16 wide one-hot", M, K, N, splits, nb, wpt)
    rng = np.random.default_rng(M + K + N)
    p = gen.w4a16_problem(1, K, N, seed=M * 3 + 1, activations=False)
    A, ks = _one_hot(M, K, rng)
    qg.set_plan_override(nb, wpt, splits, kernel=2)
    pl = qg.plan(qg.FMT_W4A16, M, K, N)
    assert pl["kernel"] == 2 and (pl["nb"], pl["wpt"]) == (nb, wpt)
    C = qg.w4a16(_t(A), upload_w4a16(p), K, N).cpu().numpy()
    q = ref.unpack_u4(p["codes"])
    expect = ((q[ks] - 8).astype(np.float64) * p["scales"][ks // 128].astype(np.float64)).astype(np.float16)
    assert np.array_equal(C.view(np.uint16), expect.view(np.uint16))


@pytest.mark.parametrize("nb,wpt", WIDE_TILES)
@pytest.mark.parametrize("M", [1, 17, 33, 47, 64, 65, 100, 127, 128, 129, 200])
def test_w4a16_wide_ragged(M, nb, wpt):
    K, N = 1280, 512                      # G = 10, two 256-column tiles or four of 128
    _say("w4a16 wide ragged", M, K, N, nb, wpt)
    p = gen.w4a16_problem(M, K, N, seed=M + 5)
    qg.set_plan_override(nb, wpt, 0, kernel=2)
    C1 = qg.w4a16(_t(p["A"]), upload_w4a16(p), K, N)
    C2 = qg.w4a16(_t(p["A"]), upload_w4a16(p), K, N)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    _ok(C1.cpu().numpy(), ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), K, ("wide", M))


@pytest.mark.parametrize("nb,wpt", WIDE_TILES)
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16])
@pytest.mark.parametrize("M", [40, 128])
def test_w4a16_wide_forced_splits(splits, M, nb, wpt):
    K, N = 4096, 512
    _say("w4a16 wide splits", splits, M, nb, wpt)
    p = gen.w4a16_problem(M, K, N, seed=splits)
    qg.set_plan_override(nb, wpt, splits, kernel=2)
    pl = qg.plan(qg.FMT_W4A16, M, K, N)
    assert pl["kernel"] == 2 and pl["splits"] == splits and (pl["nb"], pl["wpt"]) == (nb, wpt)
    C = qg.w4a16(_t(p["A"]), upload_w4a16(p), K, N).cpu().numpy()
    _ok(C, ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), K, ("wide splits", splits, M))
