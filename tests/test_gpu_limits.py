"""GPU parity at the largest shapes the C ABI accepts, through the C ABI.

The header admits 0 <= M <= 65535 and K up to 2^20 (K * N <= 2^32); these cases
run the automatic plans at those limits on layers small enough for the fp64
oracle to check every output:
  * M = 65535 on the wide kernel (N a multiple of 256) and on the streaming
    kernel (N = 64), W4A16; W4A8 with exact int32 accumulators; mixed 2/4-bit;
  * K = 2^20 (8192 groups per column, the longest k-range and the largest
    k-split count the planner makes), W4A16 and mixed 2/4-bit.
Bars as everywhere: fp16 outputs within max|e| <= 2e-3 sqrt(K) rms(C_ref) and
relative Frobenius error <= 1e-3; W4A8 accumulators bit-exact.
"""

import sys

import numpy as np
import pytest
import torch

import bit_weight_quantized_qgemm_amd as qg
from oracle import compare, ref
from synth import gen

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
M_MAX = 65535
K_MAX = 1 << 20


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _ok(C_gpu, C_ref, K, what):
    r = compare.check_fp16(C_gpu, C_ref, K)
    assert r["ok"], (what, r)


@pytest.fixture(autouse=True)
def _reset_plan():
    qg.set_plan_override()
    yield
    qg.set_plan_override()


@pytest.mark.parametrize("N", [256, 64])
def test_w4a16_max_m(N):
    K = 256
    pl = qg.plan(qg.FMT_W4A16, M_MAX, K, N)
    _say("w4a16 max M", M_MAX, K, N, pl)
    assert pl["mt"] * pl["mb"] * 16 >= M_MAX
    p = gen.w4a16_problem(M_MAX, K, N, seed=31)
    blob = qg.repack_w4a16(_t(p["codes"].view(np.int32)), _t(p["scales"]))
    C = qg.w4a16(_t(p["A"]), blob, K, N)
    torch.cuda.synchronize()
    _ok(C.cpu().numpy(), ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), K, ("max M", N))


def test_w4a8_max_m():
    K, N = 256, 64
    p = gen.w4a8_problem(M_MAX, K, N, seed=32)
    _say("w4a8 max M", M_MAX, K, N, qg.plan(qg.FMT_W4A8, M_MAX, K, N))
    blob = qg.repack_w4a8(_t(p["codes"].view(np.int32)), _t(p["group_scales"]), _t(p["chan_scales"]))
    acc = torch.empty((M_MAX, N), dtype=torch.int32, device=DEV)
    C = qg.w4a8(_t(p["A"]), _t(p["a_scale"]), blob, K, N, acc_out=acc)
    torch.cuda.synchronize()
    acc_ref, C_ref = ref.gemm_w4a8(p["A"], p["codes"], p["group_scales"], p["a_scale"], p["chan_scales"])
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    _ok(C.cpu().numpy(), C_ref, K, "w4a8 max M")


def test_w2w4_max_m():
    K, N = 256, 64
    p = gen.w2w4_problem(M_MAX, K, N, seed=33, frac4=0.3)
    _say("w2w4 max M", M_MAX, K, N, qg.plan(qg.FMT_W2W4, M_MAX, K, N))
    blob = qg.repack_w2w4(_t(p["codes"]), _t(p["scales"]), p["bitmap"])
    C = qg.w2w4_mixed(_t(p["A"]), blob, K, N)
    torch.cuda.synchronize()
    _ok(C.cpu().numpy(), ref.gemm_w2w4(p["A"], p["codes"], p["bitmap"], p["scales"]), K, "w2w4 max M")


@pytest.mark.parametrize("M", [1, 5])
def test_w4a16_max_k(M):
    N = 64
    pl = qg.plan(qg.FMT_W4A16, M, K_MAX, N)
    _say("w4a16 max K", M, K_MAX, N, pl)
    p = gen.w4a16_problem(M, K_MAX, N, seed=34 + M)
    blob = qg.repack_w4a16(_t(p["codes"].view(np.int32)), _t(p["scales"]))
    C = qg.w4a16(_t(p["A"]), blob, K_MAX, N)
    torch.cuda.synchronize()
    _ok(C.cpu().numpy(), ref.gemm_w4a16(p["A"], p["codes"], p["scales"]), K_MAX, ("max K", M))


def test_w2w4_max_k():
    M, N = 3, 64
    p = gen.w2w4_problem(M, K_MAX, N, seed=36)
    _say("w2w4 max K", M, K_MAX, N, qg.plan(qg.FMT_W2W4, M, K_MAX, N))
    blob = qg.repack_w2w4(_t(p["codes"]), _t(p["scales"]), p["bitmap"])
    C = qg.w2w4_mixed(_t(p["A"]), blob, K_MAX, N)
    torch.cuda.synchronize()
    _ok(C.cpu().numpy(), ref.gemm_w2w4(p["A"], p["codes"], p["bitmap"], p["scales"]), K_MAX, "w2w4 max K")
