"""Pins for the CPU oracle's GEMMs (oracle/ref.py).

None of these compares the oracle with itself: each checks it against exact
rational brute force (Python ``Fraction`` over the exact fp16 values, with the
codes read bit by bit from the canonical words), closed forms, special cases that
reduce to a library matmul, or invariants. Each was chosen so that a plausible
mistake in the oracle -- a wrong nibble order, zero point, group index, scale
orientation, sign convention or a transposed operand -- fails at least one.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import ref
from synth import gen


def _frac(x) -> Fraction:
    return Fraction(float(x))  # fp16 -> float is exact; Fraction(float) is exact


def _code_bruteforce(qw, k, n):
    return (int(qw[k // 8, n]) >> (4 * (k % 8))) & 0xF


def _bruteforce_w4a16(A, qw, s, zero=8):
    M, K = A.shape
    N = qw.shape[1]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                q = _code_bruteforce(qw, k, n)
                acc += _frac(A[m, k]) * (q - zero) * _frac(s[k // 128, n])
            out[m][n] = acc
    return out


def test_unpack_u4_hand_words():
    qw = np.array([[0x76543210, 0xFEDCBA98]], dtype=np.uint32)
    u = ref.unpack_u4(qw)
    assert u[:, 0].tolist() == list(range(8))
    assert u[:, 1].tolist() == list(range(8, 16))
    s = ref.unpack_s4(qw)
    assert s[:, 0].tolist() == list(range(8))
    assert s[:, 1].tolist() == [-8, -7, -6, -5, -4, -3, -2, -1]


@pytest.mark.parametrize("M,K,N,seed", [(1, 128, 3, 1), (3, 256, 5, 2), (2, 256, 8, 3)])
def test_w4a16_bruteforce_exact(M, K, N, seed):
    p = gen.w4a16_problem(M, K, N, seed=seed)
    C = ref.gemm_w4a16(p["A"], p["codes"], p["scales"])
    exact = _bruteforce_w4a16(p["A"], p["codes"], p["scales"])
    for m in range(M):
        for n in range(N):
            terms = sum(abs(_frac(p["A"][m, k])) * 8 * _frac(p["scales"][k // 128, n]) for k in range(K))
            bound = float(terms) * K * 2.0 ** -52
            assert abs(C[m, n] - float(exact[m][n])) <= bound + 1e-300


def test_w4a16_matches_library_matmul_on_integer_weights():
    # scales all 1: W = q - 8 is an integer matrix; compare with torch's fp64 matmul
    rng = np.random.default_rng(7)
    M, K, N = 4, 384, 64
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    A = rng.standard_normal((M, K)).astype(np.float16)
    s = np.ones((K // 128, N), dtype=np.float16)
    C = ref.gemm_w4a16(A, gen.pack_nibbles_u32(q), s)
    expect = torch.from_numpy(A.astype(np.float64)) @ torch.from_numpy(q.astype(np.float64) - 8.0)
    np.testing.assert_allclose(C, expect.numpy(), rtol=0, atol=1e-9)


def test_w4a16_one_hot_rows_are_dequantized_weights():
    rng = np.random.default_rng(11)
    K, N = 512, 64
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    s = rng.uniform(0.005, 0.02, size=(K // 128, N)).astype(np.float16)
    ks = np.array([0, 1, 7, 127, 128, 300, 511])
    A = np.zeros((len(ks), K), dtype=np.float16)
    A[np.arange(len(ks)), ks] = 1
    C = ref.gemm_w4a16(A, gen.pack_nibbles_u32(q), s)
    for i, k in enumerate(ks):
        row = (q[k].astype(np.float64) - 8) * s[k // 128].astype(np.float64)
        assert np.array_equal(C[i], row)


def test_w4a16_constant_code_closed_form():
    rng = np.random.default_rng(5)
    M, K, N = 3, 512, 64
    A = rng.standard_normal((M, K)).astype(np.float16)
    s = rng.uniform(0.005, 0.02, size=(K // 128, N)).astype(np.float16)
    for c in (0, 3, 8, 15):
        qw = gen.pack_nibbles_u32(np.full((K, N), c, dtype=np.uint8))
        C = ref.gemm_w4a16(A, qw, s)
        gsum = A.astype(np.float64).reshape(M, K // 128, 128).sum(axis=2)      # [M][G]
        expect = (c - 8) * gsum @ s.astype(np.float64)
        np.testing.assert_allclose(C, expect, rtol=1e-13, atol=1e-12)
        if c == 8:
            assert np.all(C == 0.0)


def test_w4a16_ones_times_constant_is_exact():
    K, N = 1024, 64
    A = np.ones((2, K), dtype=np.float16)
    s = np.full((K // 128, N), 2.0 ** -6, dtype=np.float16)
    qw = gen.pack_nibbles_u32(np.full((K, N), 11, dtype=np.uint8))
    C = ref.gemm_w4a16(A, qw, s)
    assert np.all(C == 3 * 2.0 ** -6 * K)


def test_w4a16_scale_doubling_and_linearity():
    p = gen.w4a16_problem(4, 512, 64, seed=9)
    C = ref.gemm_w4a16(p["A"], p["codes"], p["scales"])
    C2 = ref.gemm_w4a16(p["A"], p["codes"], (p["scales"].astype(np.float32) * 2).astype(np.float16))
    assert np.array_equal(C2, 2 * C)
    A2 = gen.w4a16_problem(4, 512, 64, seed=10)["A"]
    Csum = ref.gemm_w4a16(p["A"].astype(np.float64) + A2.astype(np.float64), p["codes"], p["scales"])
    np.testing.assert_allclose(Csum, C + ref.gemm_w4a16(A2, p["codes"], p["scales"]), atol=1e-12)
    assert np.all(ref.gemm_w4a16(np.zeros((2, 512), np.float16), p["codes"], p["scales"]) == 0)


def test_w4a16_group_orientation():
    # a scale that is nonzero in exactly one (group, column) only affects that column
    # and only through the 128 k of that group
    K, N = 512, 64
    q = np.full((K, N), 9, dtype=np.uint8)            # q - 8 = 1
    s = np.zeros((K // 128, N), dtype=np.float16)
    s[2, 5] = 1.0
    A = np.zeros((1, K), dtype=np.float16)
    A[0, 256:384] = 1.0                                # exactly group 2
    A[0, 0] = 100.0                                    # group 0: scale 0 -> no effect
    C = ref.gemm_w4a16(A, gen.pack_nibbles_u32(q), s)
    expect = np.zeros((1, N))
    expect[0, 5] = 128.0
    assert np.array_equal(C, expect)


def test_w4a16_column_subset_equals_full():
    p = gen.w4a16_problem(2, 1024, 128, seed=4)
    full = ref.gemm_w4a16(p["A"], p["codes"], p["scales"])
    cols = np.array([0, 17, 64, 127])
    sub = ref.gemm_w4a16(p["A"], p["codes"], p["scales"], cols=cols)
    np.testing.assert_allclose(sub, full[:, cols], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- W4A8
def _bruteforce_w4a8(A, qw, sg):
    M, K = A.shape
    N = qw.shape[1]
    out = np.zeros((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            acc = 0
            for k in range(K):
                nib = _code_bruteforce(qw, k, n)
                q = nib - 16 if nib & 8 else nib
                acc += int(A[m, k]) * q * int(sg[k // 128, n])
            out[m, n] = acc
    return out


@pytest.mark.parametrize("M,K,N,seed", [(1, 128, 4, 1), (3, 256, 6, 2)])
def test_w4a8_bruteforce_equal(M, K, N, seed):
    p = gen.w4a8_problem(M, K, N, seed=seed)
    acc = ref.w4a8_acc(p["A"], p["codes"], p["group_scales"])
    exact = _bruteforce_w4a8(p["A"], p["codes"], p["group_scales"])
    assert acc.tolist() == exact.tolist()
    C = ref.w4a8_out(acc, p["a_scale"], p["chan_scales"])
    for m in range(M):
        for n in range(N):
            e = Fraction(int(exact[m, n])) * _frac(p["a_scale"][m]) * _frac(p["chan_scales"][n])
            assert abs(C[m, n] - float(e)) <= abs(float(e)) * 2.0 ** -50


def test_w4a8_unit_scales_is_plain_integer_gemm():
    rng = np.random.default_rng(3)
    M, K, N = 5, 256, 64
    A = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    q = rng.integers(-8, 8, size=(K, N))
    qw = gen.pack_nibbles_u32((q & 0xF).astype(np.uint8))
    acc = ref.w4a8_acc(A, qw, np.ones((K // 128, N), dtype=np.int8))
    assert np.array_equal(acc, A.astype(np.int64) @ q.astype(np.int64))


def test_w4a8_extremes_exact():
    # |acc| reaches 16384 * 128 * 8 * 127 ~ 2.1e9: still exact (fp64 < 2**53)
    K, N = 16384, 64
    A = np.full((1, K), -128, dtype=np.int8)
    qw = gen.pack_nibbles_u32(np.full((K, N), 8, dtype=np.uint8))   # q = -8
    sg = np.full((K // 128, N), 127, dtype=np.int8)
    acc = ref.w4a8_acc(A, qw, sg)
    assert np.all(acc == K * 128 * 8 * 127)


def test_w4a8_one_hot_rows():
    p = gen.w4a8_problem(1, 512, 64, seed=5)
    q = ref.unpack_s4(p["codes"])
    for k in (0, 5, 129, 511):
        A = np.zeros((1, 512), dtype=np.int8)
        A[0, k] = 1
        acc = ref.w4a8_acc(A, p["codes"], p["group_scales"])
        nib = np.array([_code_bruteforce(p["codes"], k, n) for n in range(64)])
        expect = np.where(nib >= 8, nib - 16, nib) * p["group_scales"][k // 128].astype(np.int64)
        assert np.array_equal(acc[0], expect)
        assert np.array_equal(q[k], np.where(nib >= 8, nib - 16, nib))


# --------------------------------------------------------------------------- mixed 2/4
def test_w2w4_all_four_bit_equals_w4a16():
    rng = np.random.default_rng(21)
    M, K, N = 3, 512, 64
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    s = rng.uniform(0.005, 0.02, size=(K // 128, N)).astype(np.float16)
    A = rng.standard_normal((M, K)).astype(np.float16)
    bm = gen.bitmap_from_mask(np.ones((K // 128, N), dtype=bool))
    a = ref.gemm_w2w4(A, q, bm, s)
    b = ref.gemm_w4a16(A, gen.pack_nibbles_u32(q), s)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_w2w4_all_two_bit_bruteforce():
    rng = np.random.default_rng(22)
    M, K, N = 2, 256, 6
    q = rng.integers(0, 4, size=(K, 64), dtype=np.uint8)
    s = rng.uniform(0.005, 0.02, size=(K // 128, 64)).astype(np.float16)
    A = rng.standard_normal((M, K)).astype(np.float16)
    bm = gen.bitmap_from_mask(np.zeros((K // 128, 64), dtype=bool))
    C = ref.gemm_w2w4(A, q, bm, s)
    for m in range(M):
        for n in range(N):
            e = sum(_frac(A[m, k]) * (int(q[k, n]) - 2) * _frac(s[k // 128, n]) for k in range(K))
            assert abs(C[m, n] - float(e)) <= 1e-12


def test_w2w4_mixed_bruteforce_and_bitmap_orientation():
    rng = np.random.default_rng(23)
    K, N = 256, 64
    mask = np.zeros((2, N), dtype=bool)
    mask[0, 33] = True          # word 1, bit 1
    mask[1, 0] = True           # word 0, bit 0
    mask[1, 63] = True          # word 1, bit 31
    p = gen.w2w4_problem(2, K, N, seed=3, mask=mask)
    bm = p["bitmap"]
    assert bm[0, 1] == 1 << 1 and bm[1, 0] == 1 and bm[1, 1] == 1 << 31
    C = ref.gemm_w2w4(p["A"], p["codes"], bm, p["scales"])
    for m in range(2):
        for n in (0, 1, 33, 63):
            e = Fraction(0)
            for k in range(K):
                g = k // 128
                z = 8 if mask[g, n] else 2
                e += _frac(p["A"][m, k]) * (int(p["codes"][k, n]) - z) * _frac(p["scales"][g, n])
            assert abs(C[m, n] - float(e)) <= 1e-12
    cols = np.array([0, 33, 63])
    np.testing.assert_allclose(ref.gemm_w2w4(p["A"], p["codes"], bm, p["scales"], cols=cols),
                               C[:, cols], atol=1e-12, rtol=0)


def test_bits_per_weight_mixed():
    K, N = 4096, 4096
    G = (K // 128) * N
    n4 = round(0.1 * G)
    mask = np.zeros(G, dtype=bool)
    mask[:n4] = True
    bm = gen.bitmap_from_mask(mask.reshape(K // 128, N))
    bpw = ref.bits_per_weight_w2w4(bm, K, N)
    assert abs(bpw - (2 + 2 * n4 * 128 / (K * N) + 17 / 128)) < 1e-12


# --------------------------------------------------------------------------- K-slab accumulation
# The oracle adds the product slab by slab (2048 k per slab by default) once K
# exceeds one slab, as every 7B- and 70B-class comparison does. These pins run
# that branch with scales that differ in every (group, column), so a slab whose
# scale slice started at the wrong group, a dropped or repeated slab, or a
# ragged last slab handled wrongly changes at least one exact value.
_SLAB_KS = (0, 127, 128, 2047, 2048, 2049, 4095, 4096, 6143, 6144, 8191)


def _distinct_scales(G, N):
    # 1 + j/1024 for j = g*N + n: exactly representable fp16 values, all distinct
    j = np.arange(G * N).reshape(G, N)
    assert G * N <= 1024
    return (1.0 + j / 1024.0).astype(np.float16)


def _slab_one_hot_case():
    K, N = 8192, 16
    q = np.random.default_rng(31).integers(0, 16, size=(K, N), dtype=np.uint8)
    s = _distinct_scales(K // 128, N)
    A = np.zeros((len(_SLAB_KS), K), dtype=np.float16)
    A[np.arange(len(_SLAB_KS)), list(_SLAB_KS)] = 1
    expect = np.array([[(int(q[k, n]) - 8) * float(s[k // 128, n]) for n in range(N)] for k in _SLAB_KS])
    return A, gen.pack_nibbles_u32(q), s, expect


def _slab_closed_form_case():
    # constant code c and integer activations: C[m,n] = (c-8) * sum_g s[g,n] * sum_{k in g} A[m,k],
    # evaluated with exact rationals
    K, N, c = 8192, 8, 13
    A = np.random.default_rng(32).integers(-4, 5, size=(2, K)).astype(np.float16)
    s = _distinct_scales(K // 128, N)
    qw = gen.pack_nibbles_u32(np.full((K, N), c, dtype=np.uint8))
    expect = np.zeros((2, N))
    for m in range(2):
        gsum = [sum(int(A[m, k]) for k in range(128 * g, 128 * g + 128)) for g in range(K // 128)]
        for n in range(N):
            e = sum(Fraction(gsum[g]) * _frac(s[g, n]) for g in range(K // 128)) * (c - 8)
            expect[m, n] = float(e)
    return A, qw, s, expect


def _pins_hold(gemm):
    for case in (_slab_one_hot_case(), _slab_closed_form_case()):
        A, qw, s, expect = case
        if not np.array_equal(gemm(A, qw, s), expect):
            return False
    return True


@pytest.mark.parametrize("slab", [2048, 640, 128, 8192])
def test_w4a16_k_slabs_one_hot_and_closed_form(slab):
    # the default slab (2048) and slabs that do not divide K (640) or hold one
    # group (128) or all of K: every value exact (each product and partial sum
    # fits in fp64's significand)
    assert _pins_hold(lambda A, qw, s: ref.gemm_w4a16(A, qw, s, slab=slab))


def test_w4a16_k_slab_pins_catch_a_misaligned_scale_slice():
    # a planted mistake in a copy of the oracle's slab loop: the scales of every
    # slab taken from group 0 instead of group k0 // 128; the pins above must fail
    def misaligned(A, qw, s, slab=2048):
        K = qw.shape[0] * 8
        C = np.zeros((A.shape[0], qw.shape[1]))
        for k0 in range(0, K, slab):
            k1 = min(K, k0 + slab)
            C += A[:, k0:k1].astype(np.float64) @ ref.dequant_w4a16(qw[k0 // 8:k1 // 8], s[:(k1 - k0) // 128])
        return C

    def off_by_one(A, qw, s, slab=2048):
        K = qw.shape[0] * 8
        C = np.zeros((A.shape[0], qw.shape[1]))
        for k0 in range(0, K, slab):
            k1 = min(K, k0 + slab)
            g0 = min(k0 // 128 + 1, K // 128 - (k1 - k0) // 128)
            C += A[:, k0:k1].astype(np.float64) @ ref.dequant_w4a16(qw[k0 // 8:k1 // 8],
                                                                   s[g0:g0 + (k1 - k0) // 128])
        return C

    assert _pins_hold(lambda A, qw, s: ref.gemm_w4a16(A, qw, s))
    assert not _pins_hold(misaligned)
    assert not _pins_hold(off_by_one)


def test_w4a8_k_slabs_one_hot_with_varying_group_scales():
    # one-hot int8 rows across slab boundaries with a different int8 group scale
    # in every (group, column): acc row = q[k, :] * s_g[k // 128, :] exactly
    K, N = 8192, 16
    rng = np.random.default_rng(33)
    q = rng.integers(-8, 8, size=(K, N))
    sg = ((np.arange((K // 128) * N).reshape(K // 128, N) * 37) % 255 - 127).astype(np.int8)
    assert len(np.unique(sg)) == 255          # no two adjacent groups of a column agree
    qw = gen.pack_nibbles_u32((q & 0xF).astype(np.uint8))
    A = np.zeros((len(_SLAB_KS), K), dtype=np.int8)
    A[np.arange(len(_SLAB_KS)), list(_SLAB_KS)] = 1
    acc = ref.w4a8_acc(A, qw, sg)
    for i, k in enumerate(_SLAB_KS):
        assert acc[i].tolist() == [int(q[k, n]) * int(sg[k // 128, n]) for n in range(N)], k


def test_w4a8_bruteforce_at_k4096_with_random_group_scales():
    # two slabs; random int8 group scales over the whole int8 range, compared
    # with Python-int brute force on a few columns (equality)
    K, N, M = 4096, 64, 2
    rng = np.random.default_rng(34)
    A = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    q = rng.integers(-8, 8, size=(K, N))
    sg = rng.integers(-128, 128, size=(K // 128, N)).astype(np.int8)
    qw = gen.pack_nibbles_u32((q & 0xF).astype(np.uint8))
    cols = np.array([0, 5, 31, 63])
    acc = ref.w4a8_acc(A, qw, sg, cols=cols)
    exact = _bruteforce_w4a8(A, qw[:, cols], sg[:, cols])
    assert acc.tolist() == exact.tolist()
