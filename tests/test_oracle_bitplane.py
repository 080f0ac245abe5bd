"""Pins for the bit-plane W_b A8 parts of the oracle: the bipolar-INT value
(``oracle.ref.bipolar_value``), the exact GEMM (``gemm_bitplane_a8``) and the
blob layout of format 6 (``oracle.layout.blob_bitplane``).

Each check comes from outside the oracle: the values fixed by the format's
definition (each bit plane contributes +-2^i), exact brute force with Python
ints that decomposes every weight into its bit planes, the relation to the
already pinned W4A8 oracle at b = 4, symmetry, and hand-derived blob words.
A wrong offset (2^b instead of 2^b - 1), a plane weight off by one, a
transposed operand or a wrong bit position in the blob fails one of them."""

import numpy as np
import pytest

from oracle import layout, ref
from synth import gen


def test_bipolar_values_by_definition():
    assert ref.bipolar_value(np.array([0, 1]), 1).tolist() == [-1, 1]
    assert ref.bipolar_value(np.arange(4), 2).tolist() == [-3, -1, 1, 3]
    assert ref.bipolar_value(np.arange(8), 3).tolist() == [-7, -5, -3, -1, 1, 3, 5, 7]
    assert ref.bipolar_value(np.array([0, 255, 128]), 8).tolist() == [-255, 255, 1]
    for b in range(1, 9):
        u = np.arange(2 ** b)
        v = ref.bipolar_value(u, b)
        # sum over planes of +-2^i, read bit by bit
        planes = sum((2 * ((u >> i) & 1) - 1) * 2 ** i for i in range(b))
        assert np.array_equal(v, planes)
        assert np.array_equal(v, -v[::-1])          # symmetric grid, no zero
        assert np.all(v % 2 != 0)


@pytest.mark.parametrize("bits", [1, 2, 3, 5, 8])
def test_gemm_bruteforce_exact(bits):
    M, K, N = 3, 256, 5
    p = gen.bitplane_problem(M, K, N, bits, seed=bits)
    acc, C = ref.gemm_bitplane_a8(p["A"], p["codes"], bits, p["a_scale"], p["chan_scales"])
    for m in range(M):
        for n in range(N):
            want = 0
            for k in range(K):
                u = int(p["codes"][k, n])
                w = sum((1 if (u >> i) & 1 else -1) << i for i in range(bits))
                want += int(p["A"][m, k]) * w
            assert int(acc[m, n]) == want
            assert C[m, n] == float(want) * float(p["a_scale"][m]) * float(p["chan_scales"][n])


def test_b4_relates_to_w4a8_oracle():
    # 4-bit bipolar w = 2U - 15 = 2 (U - 8) + 1: with q = U - 8 as a signed int4
    # code and unit group scales, acc_bp = 2 acc_w4a8 + rowsum(A)
    M, K, N = 4, 512, 16
    p = gen.bitplane_problem(M, K, N, 4, seed=2)
    q = p["codes"].astype(np.int64) - 8
    qw = gen.pack_nibbles_u32((q & 0xF).astype(np.uint8))
    acc8 = ref.w4a8_acc(p["A"], qw, np.ones((K // 128, N), np.int8))
    acc, _ = ref.gemm_bitplane_a8(p["A"], p["codes"], 4, p["a_scale"], p["chan_scales"])
    assert np.array_equal(acc, 2 * acc8 + p["A"].astype(np.int64).sum(axis=1, keepdims=True))


def test_high_code_bits_are_ignored():
    p = gen.bitplane_problem(2, 128, 64, 3, seed=1)
    acc, _ = ref.gemm_bitplane_a8(p["A"], p["codes"], 3, p["a_scale"], p["chan_scales"])
    acc2, _ = ref.gemm_bitplane_a8(p["A"], p["codes"] | 0xF8, 3, p["a_scale"], p["chan_scales"])
    assert np.array_equal(acc, acc2)


def test_blob_hand_words():
    K, N, bits = 128, 64, 3
    U = np.zeros((K, N), np.uint8)
    # k = 64*1 + 16*2 + 5 (u = 1, h = 2, j = 5), column 16*1 + 7: U = 0b101
    U[64 + 32 + 5, 23] = 5
    # k = 0 + 16*3 + 15 (u = 0, h = 3, j = 15), column 2: U = 0b010
    U[48 + 15, 2] = 2
    blob = layout.blob_bitplane(U, bits, np.ones(N, np.float16))
    words = np.frombuffer(blob[:N // 16 * 256 * bits], dtype="<u4").reshape(1, N // 16, 64, bits)
    w = words[0, 1, 2 * 16 + 7]
    assert w.tolist() == [1 << 21, 0, 1 << 21]            # planes 0 and 2, bit 16 + 5
    w2 = words[0, 0, 3 * 16 + 2]
    assert w2.tolist() == [0, 1 << 15, 0]                 # plane 1, bit 15
    assert int(np.count_nonzero(words)) == 3
    assert blob[N // 16 * 256 * bits:][:2 * N] == np.ones(N, np.float16).tobytes()


def test_blob_round_trip():
    K, N, bits = 256, 64, 6
    p = gen.bitplane_problem(1, K, N, bits, seed=4)
    blob = layout.blob_bitplane(p["codes"], bits, p["chan_scales"])
    G, NB = K // 128, N // 16
    words = np.frombuffer(blob[:NB * G * 256 * bits], dtype="<u4").reshape(G, NB, 64, bits)
    U = np.zeros((K, N), np.int64)
    for g in range(G):
        for b in range(NB):
            for l in range(64):
                h, c = divmod(l, 16)
                for t in range(32):
                    u, j = divmod(t, 16)
                    k = 128 * g + 64 * u + 16 * h + j
                    U[k, 16 * b + c] = sum(((int(words[g, b, l, i]) >> t) & 1) << i for i in range(bits))
    assert np.array_equal(U, p["codes"])
