"""Pins for the 2:4 structured-sparse W4A16 parts of the oracle: the structure
check (``oracle.ref.sparse24_violations``), the seeded generator and the blob
layout of format 5 (``oracle.layout.blob_sp24``). The GEMM itself is the
W4A16 oracle on the dense codes (pruned weights hold the zero point, so they
are exactly 0), pinned in test_oracle_ref.py; here a planted extra nonzero, a
position index off by one, a swapped pair or a word of the wrong 64-k step
each fails a test."""

import numpy as np
import pytest

from oracle import layout, ref
from synth import gen


def _codes(q):
    return gen.pack_nibbles_u32(np.asarray(q, dtype=np.uint8))


def test_violations_hand_cases():
    # one column, K = 8: quads (k 0..3) and (k 4..7)
    assert ref.sparse24_violations(_codes([[8], [8], [8], [8], [1], [8], [8], [2]])) == 0
    assert ref.sparse24_violations(_codes([[0], [8], [0], [8], [15], [8], [8], [8]])) == 0
    assert ref.sparse24_violations(_codes([[1], [2], [3], [8], [8], [8], [8], [8]])) == 1
    assert ref.sparse24_violations(_codes([[1], [2], [3], [4], [5], [6], [8], [7]])) == 2
    # the quads are aligned to multiples of 4: k 2..5 holding 3 nonzeros is fine
    assert ref.sparse24_violations(_codes([[8], [8], [1], [2], [3], [8], [8], [8]])) == 0


def test_generator_structure_and_spread():
    p = gen.w4a16_sp24_problem(1, 512, 64, seed=3, activations=False)
    assert ref.sparse24_violations(p["codes"]) == 0
    q = ref.unpack_u4(p["codes"]).reshape(128, 4, 64)
    nz = q != 8
    assert nz.sum(axis=1).max() <= 2
    # pairs: all 6 position pairs occur; kept codes cover 0..15
    kept_pos = [tuple(np.flatnonzero(nz[j, :, n])) for j in range(128) for n in range(64)]
    assert {kp for kp in kept_pos if len(kp) == 2} == {(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)}
    assert 0.4 < nz.mean() < 0.5   # 2 of 4 kept, minus kept codes that happen to be 8
    assert set(np.unique(q[nz]).tolist()) == set(range(16)) - {8}


def _blob_words(blob, K, N):
    G, NB = K // 128, N // 16
    raw = np.frombuffer(blob, dtype=np.uint8)
    rec = raw[:NB * G * 768].view("<u4").reshape(G, NB, 64, 3)   # 12 bytes per lane
    return rec[..., :2], rec[..., 2]


def test_blob_hand_positions():
    K, N = 128, 64
    q = np.full((K, N), 8, dtype=np.uint8)
    # column 3, k = 64*1 + 16*2 + 4*1 + {1, 3}: step 1, lane 16*2 + 3, quad 1
    q[64 + 32 + 4 + 1, 3] = 5
    q[64 + 32 + 4 + 3, 3] = 11
    # column 7, k = 0 + 16*1 + 4*2 + 2 (single nonzero at position 2): step 0, lane 23, quad 2
    q[16 + 8 + 2, 7] = 13
    blob = layout.blob_sp24(_codes(q), np.ones((1, N), np.float16))
    words, meta = _blob_words(blob, K, N)
    w = int(words[0, 0, 35, 1])
    # v = 2 (nibble sigma(2) = 1) holds 5, v = 3 (nibble sigma(3) = 5) holds 11
    assert (w >> 4) & 0xF == 5 and (w >> 20) & 0xF == 11
    m = int(meta[0, 0, 35])
    assert (m >> (16 + 4)) & 3 == 1 and (m >> (16 + 6)) & 3 == 3
    # every other quad of that word: positions (0, 1) holding code 8
    for v in (0, 1, 4, 5, 6, 7):
        sig = v // 2 if v % 2 == 0 else 4 + (v - 1) // 2
        assert (w >> (4 * sig)) & 0xF == 8
    assert [(m >> (16 + 2 * v)) & 3 for v in (0, 1, 4, 5, 6, 7)] == [0, 1, 0, 1, 0, 1]
    # column 7: quad 2 keeps (0, 2) with the code at the second slot (v = 5, nibble 6)
    w7 = int(words[0, 0, 23, 0])
    m7 = int(meta[0, 0, 23])
    assert (w7 >> 24) & 0xF == 13 and (w7 >> 8) & 0xF == 8
    assert (m7 >> 8) & 3 == 0 and (m7 >> 10) & 3 == 2
    # status word is zero for a valid blob
    assert blob[-256:] == bytes(256)


def _decode(blob, K, N):
    """Dense codes from a format-5 blob, written from the layout text."""
    G, NB = K // 128, N // 16
    words, meta = _blob_words(blob, K, N)
    q = np.full((K, N), 8, dtype=np.int64)
    for g in range(G):
        for b in range(NB):
            for l in range(64):
                h, c = divmod(l, 16)
                for s in range(2):
                    w, m = int(words[g, b, l, s]), int(meta[g, b, l])
                    for v in range(8):
                        sig = v // 2 if v % 2 == 0 else 4 + (v - 1) // 2
                        code = (w >> (4 * sig)) & 0xF
                        p = (m >> (16 * s + 2 * v)) & 3
                        k = 128 * g + 64 * s + 16 * h + 4 * (v // 2) + p
                        if code != 8:
                            q[k, 16 * b + c] = code
    return q


def test_blob_round_trip():
    K, N = 256, 64
    p = gen.w4a16_sp24_problem(1, K, N, seed=9, activations=False)
    blob = layout.blob_sp24(p["codes"], p["scales"])
    assert np.array_equal(_decode(blob, K, N), ref.unpack_u4(p["codes"]))
    # scales region equals the W4A16 one
    d = layout.blob_w4a16(p["codes"], p["scales"])
    s_sp = blob[3 * K * N // 8:][:(N // 16) * 256]
    s_w4 = d[K * N // 2:][:(N // 16) * 256]
    assert s_sp == s_w4


def test_blob_rejects_broken_structure():
    q = np.full((128, 64), 8, dtype=np.uint8)
    q[0:3, 5] = [1, 2, 3]
    with pytest.raises(ValueError):
        layout.blob_sp24(_codes(q), np.ones((1, 64), np.float16))
