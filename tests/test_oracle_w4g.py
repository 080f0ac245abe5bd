"""Pins for the oracle of the 4-bit GEMM on a general quantization grid
(``oracle.ref.gemm_w4g``: group length 64 / 128 / ... / K, stored zero points,
fp16 or bf16 activations).

None of these compares the oracle with itself: each checks it against exact
rational brute force (Python ``Fraction``; codes read bit by bit; bf16 patterns
decoded through ``struct`` rather than NumPy views), closed forms, special cases
that reduce to the already pinned W4A16 oracle, or algebraic identities. A
wrong group index (k // g), a zero point applied to the wrong (g, n), a zero
point added instead of subtracted, a bf16 decode of the wrong half or a
transposed operand each fails at least one of them.
"""

import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import compare, ref
from synth import gen


def _bf16_exact(bits: int) -> Fraction:
    (v,) = struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))
    return Fraction(v)


def _val(x, act) -> Fraction:
    return Fraction(float(x)) if act == "fp16" else _bf16_exact(x)


def _bruteforce(A, qw, s, z, gs, act):
    M, K = A.shape
    N = qw.shape[1]
    out = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                q = (int(qw[k // 8, n]) >> (4 * (k % 8))) & 0xF
                zz = 8 if z is None else int(z[k // gs, n])
                acc += _val(A[m, k], act) * (q - zz) * _val(s[k // gs, n], act)
            out[m, n] = acc
    return out


@pytest.mark.parametrize("act", ["fp16", "bf16"])
@pytest.mark.parametrize("gs,zeros", [(64, False), (64, True), (128, True), (256, False), (256, True)])
def test_bruteforce_exact(act, gs, zeros):
    M, K, N = 2, 256, 5
    p = gen.w4g_problem(M, K, N, gs, zeros, act, seed=11)
    C = ref.gemm_w4g(p["A"], p["codes"], p["scales"], p["zeros"], gs, act)
    exact = _bruteforce(p["A"], p["codes"], p["scales"], p["zeros"], gs, act)
    for m in range(M):
        for n in range(N):
            # fp64 matmul rounding bound: K * 2**-52 * sum of |terms|
            terms = sum(abs(_val(p["A"][m, k], act)) * 15 * abs(_val(p["scales"][k // gs, n], act))
                        for k in range(K))
            assert abs(Fraction(C[m, n]) - exact[m, n]) <= Fraction(K) * Fraction(2) ** -52 * terms


def test_bf16_decode_known_patterns():
    # values fixed by the bfloat16 definition (binary32 with 16 low bits dropped)
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0080, 0x7F7F, 0x0001, 0x8000, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 0.5, 2.0 ** -126, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133, -0.0, 3.140625]
    got = ref.bf16_to_f64(bits)
    assert got.tolist() == want
    assert np.signbit(got[6])


def test_generator_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5, 3.14159265], np.float32)
    assert gen.to_bf16_bits(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x4049]


def test_reduces_to_w4a16_oracle():
    # group 128, zero point 8 (implicit or stored), fp16: the W4A16 oracle
    M, K, N = 3, 512, 32
    p = gen.w4a16_problem(M, K, N, seed=5)
    want = ref.gemm_w4a16(p["A"], p["codes"], p["scales"])
    got = ref.gemm_w4g(p["A"], p["codes"], p["scales"], None, 128, "fp16")
    got_z = ref.gemm_w4g(p["A"], p["codes"], p["scales"], np.full((K // 128, N), 8, np.uint8), 128, "fp16")
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(got_z, want, rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("act", ["fp16", "bf16"])
def test_group64_with_pairwise_equal_params_is_group128(act):
    M, K, N = 2, 384, 16
    p = gen.w4g_problem(M, K, N, 128, True, act, seed=3)
    s64 = np.repeat(p["scales"], 2, axis=0)
    z64 = np.repeat(p["zeros"], 2, axis=0)
    a = ref.gemm_w4g(p["A"], p["codes"], s64, z64, 64, act)
    b = ref.gemm_w4g(p["A"], p["codes"], p["scales"], p["zeros"], 128, act)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-12)
    # and a difference in the second half of a 128-group shows up only in gs=64
    s64b = s64.copy()
    s64b[1] = s64b[1] * 2 if act == "fp16" else s64b[1] + 0x80   # bf16: exponent + 1
    c = ref.gemm_w4g(p["A"], p["codes"], s64b, z64, 64, act)
    assert np.abs(c - a).max() > 1e-3


@pytest.mark.parametrize("act", ["fp16", "bf16"])
def test_per_channel_identity(act):
    # g = K: W = (q - z[n]) * s[n], so C = (A @ q - rowsum(A) z) * s, with A @ q
    # an exact integer-weighted sum computed here by torch-free float64 matmul
    M, K, N = 4, 512, 24
    p = gen.w4g_problem(M, K, N, K, True, act, seed=8)
    A = ref.act_to_f64(p["A"], act)
    q = np.stack([(p["codes"][k // 8] >> np.uint32(4 * (k % 8))) & np.uint32(0xF) for k in range(K)]).astype(np.float64)
    z = p["zeros"][0].astype(np.float64)
    s = ref.act_to_f64(p["scales"], act)[0]
    want = (A @ q - A.sum(axis=1, keepdims=True) * z[None, :]) * s[None, :]
    got = ref.gemm_w4g(p["A"], p["codes"], p["scales"], p["zeros"], K, act)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-10)


@pytest.mark.parametrize("gs", [64, 128, 512])
def test_codes_equal_to_zero_points_give_zero(gs):
    K, N = 512, 16
    rng = np.random.default_rng(4)
    z = rng.integers(0, 16, size=(K // gs, N), dtype=np.uint8)
    q = np.repeat(z, gs, axis=0)          # q[k, n] = z[k // gs, n]
    qw = gen.pack_nibbles_u32(q)
    A = rng.standard_normal((3, K)).astype(np.float16)
    s = rng.uniform(0.005, 0.02, size=(K // gs, N)).astype(np.float16)
    C = ref.gemm_w4g(A, qw, s, z, gs, "fp16")
    assert np.all(C == 0.0)


@pytest.mark.parametrize("act", ["fp16", "bf16"])
def test_constant_code_closed_form(act):
    # A = 1, q = c: C[m, n] = sum_g (c - z[g, n]) * s[g, n] * gs
    K, N, gs, c = 512, 8, 64, 13
    p = gen.w4g_problem(1, K, N, gs, True, act, seed=6, activations=False)
    qw = gen.pack_nibbles_u32(np.full((K, N), c, np.uint8))
    A = np.ones((2, K), np.float16) if act == "fp16" else np.full((2, K), 0x3F80, np.uint16)
    C = ref.gemm_w4g(A, qw, p["scales"], p["zeros"], gs, act)
    s = ref.act_to_f64(p["scales"], act)
    want = ((c - p["zeros"].astype(np.float64)) * s * gs).sum(axis=0)
    np.testing.assert_allclose(C, np.broadcast_to(want, C.shape), rtol=1e-14, atol=1e-12)


def test_check_bf16_rule():
    rng = np.random.default_rng(0)
    ref_c = rng.standard_normal((8, 64)) * 3
    bits = gen.to_bf16_bits(ref_c.astype(np.float32))
    r = compare.check_bf16(bits, ref_c, K=1024)
    assert r["ok"] and r["rel_fro"] < 2.5e-3
    bad2 = gen.to_bf16_bits((ref_c * 1.01).astype(np.float32))
    assert not compare.check_bf16(bad2, ref_c, K=1024)["ok"]
    big = bits.copy()
    big[3, 5] ^= 0x4000          # an exponent bit: a gross error in one output
    assert not compare.check_bf16(big, ref_c, K=1024)["ok"]
