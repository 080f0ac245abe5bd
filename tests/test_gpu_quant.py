"""GPU parity of the per-token int8 activation quantization (qgemm_quantize_a8)
against ``oracle.ref.quantize_a8``: codes and scales bit-identical (both sides
decide each code in fp32 with round-half-to-even), and the quantize -> W4A8 GEMM
composition exact in its int32 accumulators."""

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


def _special_rows(K):
    rows = np.zeros((7, K), dtype=np.float16)
    rows[0, :3] = [1.0, -0.5, 0.25]                                  # hand case A
    rows[1, :6] = [127 / 128, 2.5 / 128, 3.5 / 128, -2.5 / 128, 0.5 / 128, -1.5 / 128]   # ties
    rows[2, :2] = [65504.0, -1000.0]                                 # largest fp16
    rows[3, :2] = [1.0, 1153 / 2048]                                 # stored-scale division
    rows[4, K // 2] = np.float16(2.0 ** -24)                         # scale underflows to 0
    rows[5, -1] = -3.0                                               # amax in the last element
    return rows                                                      # row 6 all zeros


def _check(A, what):
    M, K = A.shape
    Q, S = qg.quantize_a8(torch.from_numpy(A).to(DEV))
    q_ref, s_ref = ref.quantize_a8(A)
    assert np.array_equal(S.cpu().numpy().view(np.uint16), s_ref.view(np.uint16)), what
    assert np.array_equal(Q.cpu().numpy(), q_ref), what


@pytest.mark.parametrize("M,K", [(7, 128), (37, 4096), (128, 16384), (5, 1032), (1, 8)])
def test_quantize_matches_oracle(M, K):
    _say("quantize_a8", M, K)
    rng = np.random.default_rng(M * 31 + K)
    A = (rng.standard_normal((M, K)) * rng.uniform(1e-3, 50, size=(M, 1))).astype(np.float16)
    if K >= 8:
        sp = _special_rows(K)
        n = min(M, sp.shape[0])
        A[:n] = sp[:n]
    _check(A, (M, K))


def test_quantize_strided_with_guard_bands():
    _say("quantize_a8 strided")
    M, K, lda, ldq = 19, 2048, 2048 + 64, 2048 + 32
    rng = np.random.default_rng(4)
    Abig = (rng.standard_normal((M, lda)) * 3).astype(np.float16)
    A = torch.from_numpy(Abig).to(DEV)
    Q = torch.full((M, ldq), 0x5A, dtype=torch.int8, device=DEV)
    S = torch.full((M + 8,), 7.0, dtype=torch.float16, device=DEV)
    L = qg.lib()
    st = L.qgemm_quantize_a8(A.data_ptr(), lda, M, K, Q.data_ptr(), ldq, S.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    q_ref, s_ref = ref.quantize_a8(Abig[:, :K])
    Qh = Q.cpu().numpy()
    assert np.array_equal(Qh[:, :K], q_ref)
    assert np.all(Qh[:, K:] == 0x5A)
    Sh = S.cpu().numpy()
    assert np.array_equal(Sh[:M].view(np.uint16), s_ref.view(np.uint16))
    assert np.all(Sh[M:] == 7.0)


def test_quantize_then_w4a8_exact_accumulators():
    K, N, M = 4096, 11008, 64
    _say("quantize_a8 -> w4a8", M, K, N)
    p = gen.w4a8_problem(M, K, N, seed=11)
    A16 = gen.w4a16_problem(M, K, 64, seed=12, weights=False)["A"]
    blob = qg.repack_w4a8(torch.from_numpy(p["codes"].view(np.int32)).to(DEV),
                          torch.from_numpy(p["group_scales"]).to(DEV), torch.from_numpy(p["chan_scales"]).to(DEV))
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    C = qg.w4a8_fp16(torch.from_numpy(A16).to(DEV), blob, K, N, acc_out=acc)
    torch.cuda.synchronize()
    q_ref, s_ref = ref.quantize_a8(A16)
    cols = block_cols(N, seed=3)
    acc_ref, c_ref = ref.gemm_w4a8(q_ref, p["codes"], p["group_scales"], s_ref, p["chan_scales"], cols=cols)
    assert np.array_equal(acc.cpu().numpy()[:, cols].astype(np.int64), acc_ref)
    r = compare.check_fp16(C.cpu().numpy()[:, cols], c_ref, K)
    assert r["ok"], r
