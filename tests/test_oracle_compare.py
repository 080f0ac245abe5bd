"""Pins for the fp16 tolerance rule (oracle/compare.py).

The rule must accept the rounding a correct GPU kernel makes (fp16 output
rounding, fp16 rounding of each dequantized weight, fp32 accumulation in any
order) and reject each plausible kernel mistake. Mistakes are planted in a copy
of the oracle computation on the CPU.
"""

import numpy as np
import pytest

from oracle import compare, ref
from synth import gen


@pytest.fixture(scope="module")
def prob():
    p = gen.w4a16_problem(16, 1024, 1024, seed=0)
    p["C"] = ref.gemm_w4a16(p["A"], p["codes"], p["scales"])
    p["q"] = ref.unpack_u4(p["codes"])
    return p


def _gemm(A, q, s, zero=8, sidx=None):
    K = q.shape[0]
    g = np.arange(K) // 128 if sidx is None else sidx
    W = (q - zero).astype(np.float64) * s.astype(np.float64)[g, :]
    return A.astype(np.float64) @ W


def test_accepts_correct_roundings(prob):
    A, q, s, C = prob["A"], prob["q"], prob["scales"], prob["C"]
    assert compare.check_fp16(C.astype(np.float16), C, 1024)["ok"]
    # fp16-rounded dequantized weights, fp32 accumulation, fp16 output
    W16 = ((q - 8).astype(np.float32) * s.astype(np.float32)[np.arange(1024) // 128, :]).astype(np.float16)
    C32 = A.astype(np.float32) @ W16.astype(np.float32)
    r = compare.check_fp16(C32.astype(np.float16), C, 1024)
    assert r["ok"], r
    assert r["rel_fro"] < 5e-4


@pytest.mark.parametrize("mistake", [
    "zero7", "drop_last_group", "shift_group_scale", "reverse_nibbles",
    "swap_columns", "drop_one_k", "transpose_blocks", "nan",
])
def test_rejects_planted_mistakes(prob, mistake):
    A, q, s, C = prob["A"], prob["q"], prob["scales"], prob["C"]
    K = 1024
    if mistake == "zero7":
        bad = _gemm(A, q, s, zero=7)
    elif mistake == "drop_last_group":
        bad = _gemm(A[:, :K - 128], q[:K - 128], s)
    elif mistake == "shift_group_scale":
        bad = _gemm(A, q, s, sidx=np.minimum(np.arange(K) // 128 + 1, K // 128 - 1))
    elif mistake == "reverse_nibbles":
        perm = (np.arange(K) // 8) * 8 + (7 - np.arange(K) % 8)
        bad = _gemm(A, q[perm], s)
    elif mistake == "swap_columns":
        bad = C[:, np.arange(1024) ^ 1]
    elif mistake == "drop_one_k":
        q2 = q.copy()
        q2[517] = 8
        bad = _gemm(A, q2, s)
    elif mistake == "transpose_blocks":
        # the 16x16 output blocks transposed (row/column swap inside each tile)
        bad = C.copy()
        bad[:, :16] = C[:, :16].T
    elif mistake == "nan":
        bad = C.copy()
        bad[3, 3] = np.nan
    r = compare.check_fp16(bad.astype(np.float16), C, K)
    assert not r["ok"], (mistake, r)


def test_ulp_distance():
    a = np.array([1.0, -1.0, 0.0, 1000.0], dtype=np.float16)
    b = np.nextafter(a, np.float16(np.inf))
    assert compare.fp16_ulp_distance(a, b).tolist() == [1, 1, 1, 1]
    assert compare.fp16_ulp_distance(np.float16(-0.0), np.float16(0.0)) == 0
