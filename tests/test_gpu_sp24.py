"""GPU parity of the 2:4 structured-sparse W4A16 GEMM (gfx950 sparse matrix
instruction) against the CPU oracle, through the C ABI.

The oracle is the W4A16 definition on the dense codes (pruned weights hold the
zero point 8, so they are exactly 0). Bars: blobs byte-identical to the
independent layout oracle; a broken 2:4 structure rejected with
QGEMM_ERR_RANGE; one-hot activations reproduce fp16((q - 8) * s) bit-exactly
(kept and pruned positions alike); every output within the fp16 rule
(max|e| <= 2e-3 sqrt(K) rms(C_ref), rel. Frobenius <= 1e-3); the 70B layer on
sampled columns in the benchmark's launch configuration.
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


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _upload(p):
    return qg.repack_sp24(_t(p["codes"].view(np.int32)), _t(p["scales"]))


def _ok(C_gpu, C_ref, K, what):
    r = compare.check_fp16(C_gpu, C_ref, K)
    assert r["ok"], (what, r)
    return r


@pytest.fixture(autouse=True)
def _reset_plan():
    qg.set_plan_override()
    yield
    qg.set_plan_override()


@pytest.mark.parametrize("K,N", [(128, 64), (1152, 320), (4096, 11008)])
def test_repack_sp24_bytes(K, N):
    _say("repack sp24", K, N)
    p = gen.w4a16_sp24_problem(1, K, N, seed=K ^ N, activations=False)
    blob = _upload(p).cpu().numpy().tobytes()
    assert blob == layout.blob_sp24(p["codes"], p["scales"])


def test_repack_sp24_rejects_broken_structure():
    _say("repack sp24 broken")
    K, N = 256, 64
    p = gen.w4a16_sp24_problem(1, K, N, seed=1, activations=False)
    q = ref.unpack_u4(p["codes"]).astype(np.uint8)
    quad = q[8:12, 5]
    q[8:12, 5] = np.where(quad == 8, 3, quad)          # all four positions nonzero
    with pytest.raises(qg.QgemmError) as e:
        qg.repack_sp24(_t(gen.pack_nibbles_u32(q).view(np.int32)), _t(p["scales"]))
    assert e.value.status == -6


@pytest.mark.parametrize("M,K,N,force", [(16, 1024, 1024, None), (5, 4096, 256, (1, 8, 2)),
                                         (32, 1152, 384, (2, 16, 1)), (20, 8192, 128, (2, 4, 5)),
                                         (33, 512, 256, None)])
def test_sp24_one_hot_bit_exact(M, K, N, force):
    _say("sp24 one-hot", M, K, N, force)
    rng = np.random.default_rng(M * 5 + K)
    p = gen.w4a16_sp24_problem(1, K, N, seed=M + K, activations=False)
    ks = rng.choice(K, size=M, replace=False)
    A = np.zeros((M, K), dtype=np.float16)
    A[np.arange(M), ks] = 1.0
    if force:
        qg.set_plan_override(*force)
    C = qg.w4a16_sp24(_t(A), _upload(p), K, N).cpu().numpy()
    q = ref.unpack_u4(p["codes"])
    expect = ((q[ks] - 8).astype(np.float64) * p["scales"][ks // 128].astype(np.float64)).astype(np.float16)
    assert np.array_equal(C.view(np.uint16), expect.view(np.uint16))


@pytest.mark.parametrize("M", [1, 2, 7, 16, 17, 32, 33, 64, 100, 128])
def test_sp24_gemm_ragged(M):
    K, N = 2048, 512
    _say("sp24 gemm", M)
    p = gen.w4a16_sp24_problem(M, K, N, seed=M)
    C = qg.w4a16_sp24(_t(p["A"]), _upload(p), K, N).cpu().numpy()
    _ok(C, ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), K, M)


@pytest.mark.parametrize("force", [(1, 4, 1), (2, 8, 1), (2, 16, 1), (1, 16, 4), (2, 4, 7), (1, 8, 32)])
def test_sp24_forced_splits(force):
    K, N, M = 4096, 1024, 20
    _say("sp24 forced", force)
    p = gen.w4a16_sp24_problem(M, K, N, seed=7)
    blob = _upload(p)
    qg.set_plan_override(*force)
    A = _t(p["A"])
    C1 = qg.w4a16_sp24(A, blob, K, N)
    C2 = qg.w4a16_sp24(A, blob, K, N)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    _ok(C1.cpu().numpy(), ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), K, force)


@pytest.mark.parametrize("K,N", [(4096, 11008), (11008, 4096)])
def test_sp24_7b_layers(K, N):
    _say("sp24 7b", K, N)
    p = gen.w4a16_sp24_problem(128, K, N, seed=2)
    blob = _upload(p)
    for M in (1, 16, 128):
        A = p["A"][:M]
        C = qg.w4a16_sp24(_t(A), blob, K, N).cpu().numpy()
        _ok(C, ref.gemm_w4a16(A, p["codes"], p["scales"]), K, (K, N, M))


@pytest.mark.parametrize("K,N", [(8192, 28672), (28672, 8192)])
def test_sp24_70b_layer_sampled(K, N):
    _say("sp24 70b sampled", K, N)
    p = gen.w4a16_sp24_problem(128, K, N, seed=0)
    blob = _upload(p)
    cols = block_cols(N, seed=1)
    for M in (1, 16, 128):
        A = p["A"][:M]
        C = qg.w4a16_sp24(_t(A), blob, K, N).cpu().numpy()
        _ok(C[:, cols], ref.gemm_w4a16(A, p["codes"], p["scales"], cols=cols), K, (K, N, M))


def test_sp24_equals_dense_w4a16_within_tolerance():
    K, N, M = 4096, 1024, 16
    _say("sp24 vs dense")
    p = gen.w4a16_sp24_problem(M, K, N, seed=4)
    Cs = qg.w4a16_sp24(_t(p["A"]), _upload(p), K, N).cpu().numpy()
    Cd = qg.w4a16(_t(p["A"]), qg.repack_w4a16(_t(p["codes"].view(np.int32)), _t(p["scales"])), K, N).cpu().numpy()
    C_ref = ref.gemm_w4a16(p["A"], p["codes"], p["scales"])
    _ok(Cs, C_ref, K, "sparse")
    _ok(Cd, C_ref, K, "dense")
