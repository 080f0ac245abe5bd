"""Pins of the per-token int8 activation quantization oracle (``oracle.ref.quantize_a8``).

Hand-derived cases (``tests/golden/quant_a8.txt``), the round-half-to-even rule on
exact ties, exact rational rounding on random rows (outside the narrow window where
fp32 division may round a quotient onto a tie), and invariants of the rule.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import ref

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    out = {}
    for line in open(os.path.join(HERE, "golden", "quant_a8.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = (x.strip() for x in line.split("=", 1))
        out[k] = [int(t, 0) for t in v.split()]
    return out


def _row(vals, K=8):
    r = np.zeros((1, K), dtype=np.float16)
    r[0, :len(vals)] = np.asarray(vals, dtype=np.float16)
    return r


@pytest.mark.parametrize("case,vals", [
    ("A", [1.0, -0.5, 0.25]),
    ("B", [127 / 128, 2.5 / 128, 3.5 / 128, -2.5 / 128, 0.5 / 128, -1.5 / 128]),
    ("C", [65504.0, -1000.0]),
    ("F", [1.0, 1153 / 2048]),
])
def test_hand_derived_cases(case, vals):
    g = _golden()
    q, s = ref.quantize_a8(_row(vals))
    assert int(s.view(np.uint16)[0]) == g[f"case{case}_scale_bits"][0]
    assert q[0].tolist() == g[f"case{case}_q"]


def test_zero_and_underflowing_rows():
    g = _golden()
    A = np.zeros((2, 16), dtype=np.float16)
    A[1, 3] = np.float16(2.0 ** -24)
    A[1, 7] = -np.float16(2.0 ** -24)
    q, s = ref.quantize_a8(A)
    assert int(s.view(np.uint16)[0]) == g["caseD_scale_bits"][0]
    assert int(s.view(np.uint16)[1]) == g["caseE_scale_bits"][0]
    assert not q.any()


def _exact_q(x, s):
    """round-half-even of the exact rational x / s, clamped."""
    r = Fraction(float(x)) / Fraction(float(s))
    n = int(r // 1)
    frac = r - n
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return max(-127, min(127, n)), r


def test_matches_exact_rational_rounding_off_ties():
    rng = np.random.default_rng(5)
    A = (rng.standard_normal((6, 256)) * rng.uniform(0.01, 30, size=(6, 1))).astype(np.float16)
    q, s = ref.quantize_a8(A)
    checked = 0
    for m in range(A.shape[0]):
        for k in range(A.shape[1]):
            e, r = _exact_q(A[m, k], s[m])
            # fp32 division can land exactly on a half only within ~2^-17 of one
            if abs(r - (r // 1) - Fraction(1, 2)) < Fraction(1, 1 << 16):
                continue
            assert q[m, k] == e, (m, k, float(A[m, k]), float(s[m]))
            checked += 1
    assert checked > 1500


def test_invariants():
    rng = np.random.default_rng(9)
    A = (rng.standard_normal((32, 512)) * rng.uniform(1e-3, 100, size=(32, 1))).astype(np.float16)
    q, s = ref.quantize_a8(A)
    s32 = s.astype(np.float64)
    A64 = A.astype(np.float64)
    assert q.dtype == np.int8 and s.dtype == np.float16
    assert np.all(np.abs(q.astype(np.int64)) <= 127)
    # the absmax element of each row maps to +-127
    idx = np.abs(A64).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(32), idx].astype(np.int64)) == 127)
    # signs agree where the code is nonzero; reconstruction error at most half a step
    assert np.all(np.sign(q) * np.sign(A64) >= 0)
    err = np.abs(A64 - q.astype(np.float64) * s32[:, None])
    assert np.all(err <= 0.5 * s32[:, None] * (1 + 2.0 ** -10))
    # the scale is the fp16 rounding of amax/127 (within half an fp16 ulp)
    amax = np.abs(A64).max(axis=1)
    assert np.all(np.abs(s32 - amax / 127) <= np.abs(amax / 127) * 2.0 ** -11 + 1e-12)


def test_scaling_by_power_of_two_commutes():
    rng = np.random.default_rng(3)
    A = rng.standard_normal((4, 128)).astype(np.float16)
    q1, s1 = ref.quantize_a8(A)
    q2, s2 = ref.quantize_a8((A.astype(np.float32) * 4).astype(np.float16))
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2.astype(np.float32), s1.astype(np.float32) * 4)
