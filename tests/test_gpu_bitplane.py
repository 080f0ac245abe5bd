"""GPU parity of the bit-plane W_b A8 GEMM (b = 1..8, bipolar-INT weights)
against the CPU oracle, through the C ABI.

Bars: blobs byte-identical to the independent layout oracle; int32
accumulators bit-identical to the oracle's exact integers for every b,
ragged M and every forced plan shape; fp16 outputs within the fp16 rule
(max|e| <= 2e-3 sqrt(K) rms(C_ref), rel. Frobenius <= 1e-3); one-hot
activations give acc = the bipolar weight row exactly; the K limit's extreme
inputs (all +127 activations against all-ones codes) stay exact.
"""

import sys

import numpy as np
import pytest
import torch

import bit_weight_quantized_qgemm_amd as qg
from oracle import compare, layout, ref
from synth import gen

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _upload(p, bits=None):
    return qg.repack_bitplane(_t(p["codes"]), _t(p["chan_scales"]), bits or p["bits"])


def _run(p, A=None, a_s=None, blob=None):
    A = p["A"] if A is None else A
    a_s = p["a_scale"] if a_s is None else a_s
    M, K, N = A.shape[0], p["K"], p["N"]
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    C = qg.bitplane_a8(_t(A), _t(a_s), blob if blob is not None else _upload(p), K, N, p["bits"], acc_out=acc)
    return acc.cpu().numpy(), C.cpu().numpy()


@pytest.fixture(autouse=True)
def _reset_plan():
    qg.set_plan_override()
    yield
    qg.set_plan_override()


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_repack_bitplane_bytes(bits):
    K, N = 1152, 320
    _say("repack bitplane", bits)
    p = gen.bitplane_problem(1, K, N, bits, seed=bits)
    blob = _upload(p).cpu().numpy().tobytes()
    assert blob == layout.blob_bitplane(p["codes"], bits, p["chan_scales"])


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("M", [1, 7, 16, 33])
def test_bitplane_exact_accumulators(bits, M):
    K, N = 2048, 512
    _say("bitplane exact", bits, M)
    p = gen.bitplane_problem(M, K, N, bits, seed=M * 10 + bits)
    acc, C = _run(p)
    acc_ref, C_ref = ref.gemm_bitplane_a8(p["A"], p["codes"], bits, p["a_scale"], p["chan_scales"])
    assert np.array_equal(acc.astype(np.int64), acc_ref)
    r = compare.check_fp16(C, C_ref, K)
    assert r["ok"], r


@pytest.mark.parametrize("bits", [2, 5, 8])
@pytest.mark.parametrize("force", [(1, 4, 1), (2, 8, 1), (2, 16, 1), (1, 16, 4), (2, 4, 7), (1, 8, 32)])
def test_bitplane_forced_plans(bits, force):
    K, N, M = 4096, 1024, 20
    _say("bitplane forced", bits, force)
    p = gen.bitplane_problem(M, K, N, bits, seed=3)
    qg.set_plan_override(*force)
    acc, _ = _run(p)
    acc2, _ = _run(p)
    acc_ref, _ = ref.gemm_bitplane_a8(p["A"], p["codes"], bits, p["a_scale"], p["chan_scales"])
    assert np.array_equal(acc.astype(np.int64), acc_ref)
    assert np.array_equal(acc, acc2)


@pytest.mark.parametrize("bits", [1, 3, 8])
def test_bitplane_one_hot(bits):
    K, N, M = 1024, 256, 16
    _say("bitplane one-hot", bits)
    p = gen.bitplane_problem(M, K, N, bits, seed=5)
    ks = np.random.default_rng(bits).choice(K, size=M, replace=False)
    A = np.zeros((M, K), np.int8)
    A[np.arange(M), ks] = 1
    acc, _ = _run(p, A=A)
    assert np.array_equal(acc.astype(np.int64), ref.bipolar_value(p["codes"][ks], bits))


def test_bitplane_extremes_at_k_limit():
    # K = 16384: all activations +127 against all-ones codes (w = 2^b - 1) and
    # -127 against all-zero codes: |acc| = K * 127 * 255 at b = 8
    K, N, M, bits = 16384, 64, 2, 8
    _say("bitplane extremes")
    p = gen.bitplane_problem(M, K, N, bits, seed=1)
    codes = np.zeros((K, N), np.uint8)
    codes[:, : N // 2] = 255
    p = dict(p, codes=codes)
    A = np.full((M, K), 127, np.int8)
    A[1] = -127
    acc, _ = _run(p, A=A)
    acc_ref, _ = ref.gemm_bitplane_a8(A, codes, bits, p["a_scale"], p["chan_scales"])
    assert np.array_equal(acc.astype(np.int64), acc_ref)
    assert acc_ref.max() == K * 127 * 255


def test_bitplane_7b_layer_via_quantized_activations():
    # fp16 activations -> per-token int8 (qgemm_quantize_a8) -> 3-bit GEMM
    K, N, M, bits = 4096, 11008, 16, 3
    _say("bitplane 7b")
    p = gen.bitplane_problem(M, K, N, bits, seed=2)
    A16 = gen.w4a16_problem(M, K, 64, seed=2, weights=False)["A"]
    A_q, a_s = qg.quantize_a8(_t(A16))
    A_q = A_q.contiguous()
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    C = qg.bitplane_a8(A_q, a_s, _upload(p), K, N, bits, acc_out=acc).cpu().numpy()
    A_ref, s_ref = ref.quantize_a8(A16)
    acc_ref, C_ref = ref.gemm_bitplane_a8(A_ref, p["codes"], bits, s_ref, p["chan_scales"])
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    r = compare.check_fp16(C, C_ref, K)
    assert r["ok"], r
