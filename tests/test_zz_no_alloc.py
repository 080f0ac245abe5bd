"""The W4A16 entry point that allocates nothing (qgemm_w4a16_noalloc), through
the C ABI, against qgemm_w4a16 on the same inputs: two calls in a row, the
second on a smaller problem, each bit-identical to the workspace entry point
(same kernels and plan) and within the fp16 rule of the oracle on sampled
columns; a plan whose split-K scratch exceeds the built-in array is refused
before any launch.
"""

import ctypes
import sys

import numpy as np
import pytest
import torch

import bit_weight_quantized_qgemm_amd as qg
from oracle import compare, ref
from synth import gen

from sampling import block_cols

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _noalloc(A, blob, C, M, K, N):
    L = qg.lib()
    return L.qgemm_w4a16_noalloc(ctypes.c_void_p(A.data_ptr()), K, ctypes.c_void_p(blob.data_ptr()),
                                 ctypes.c_void_p(C.data_ptr()), N, M, K, N,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.fixture(autouse=True)
def _reset_plan():
    qg.set_plan_override()
    yield
    qg.set_plan_override()


def test_noalloc_matches_workspace_entry_point_twice_second_smaller():
    # first: the down projection at M = 128, whose wide plan needs the largest
    # split-K scratch of the automatic W4A16 plans (4 k-splits of 128 x 8192
    # fp32 partials, 16 MiB); second: a 7B-class layer at M = 16 (4 k-splits)
    for (K, N, M, seed) in [(28672, 8192, 128, 5), (4096, 4096, 16, 6)]:
        pl = qg.plan_info(qg.FMT_W4A16, M, K, N)
        _say("noalloc", M, K, N, pl)
        assert pl["splits"] > 1
        p = gen.w4a16_problem(M, K, N, seed=seed)
        blob = qg.repack_w4a16(torch.from_numpy(p["codes"].view(np.int32)).to(DEV),
                               torch.from_numpy(p["scales"]).to(DEV))
        A = torch.from_numpy(p["A"]).to(DEV)
        C_ws = qg.w4a16(A, blob, K, N)
        C_na = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        st = _noalloc(A, blob, C_na, M, K, N)
        assert st == 0, (st, qg.lib().qgemm_last_error())
        torch.cuda.synchronize()
        assert torch.equal(C_na, C_ws)
        cols = block_cols(N, seed=seed)
        r = compare.check_fp16(C_na.cpu().numpy()[:, cols],
                               ref.gemm_w4a16(p["A"], p["codes"], p["scales"], cols=cols), K)
        assert r["ok"], r


def test_noalloc_refuses_a_plan_beyond_its_scratch():
    # 64 forced k-splits of a 28672 x 8192 tile grid at M = 128 need more than
    # the 32 MiB array: refused with QGEMM_ERR_WORKSPACE, nothing written
    K, N, M = 28672, 8192, 128
    qg.set_plan_override(kernel=1, k_splits=64)
    need = qg.workspace_bytes(qg.FMT_W4A16, M, K, N)
    assert need > 32 << 20
    A = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    blob = torch.zeros(qg.packed_bytes(qg.FMT_W4A16, K, N), dtype=torch.uint8, device=DEV)
    C = torch.full((M, N), 3.0, dtype=torch.float16, device=DEV)
    st = _noalloc(A, blob, C, M, K, N)
    assert st == -4, st
    assert b"scratch" in qg.lib().qgemm_last_error()
    torch.cuda.synchronize()
    assert bool((C == 3.0).all())
