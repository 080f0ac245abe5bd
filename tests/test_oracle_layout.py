"""Pins for the independent blob-layout oracle (oracle/layout.py).

The hand-derived words in tests/golden/layout_words.txt come from applying the
layout specification by hand to simple code patterns; the round trip and the
region sizes pin the rest.
"""

import os

import numpy as np
import pytest

from oracle import layout
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layout_words.txt")


def _golden():
    out = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split("=")
            out[key.strip()] = int(val.strip(), 16)
    return out


def _pattern(K, N, fn):
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    return np.broadcast_to(fn(k, n), (K, N)).astype(np.uint8)


def test_w4a16_hand_derived_words():
    K, N = 256, 64
    q = _pattern(K, N, lambda k, n: k % 16)
    blob = np.frombuffer(layout.blob_w4a16(gen.pack_nibbles_u32(q),
                                           np.ones((2, N), np.float16)), dtype="<u4")
    g = _golden()
    # chunk (b=0, g=0): lane 0 word 0 is k = 0..7, word 1 is k = 32..39
    assert blob[0] == g["w4a16_codes0to7"]
    assert blob[1] == g["w4a16_codes0to7"]
    # lane 16 (h=1) word 0 is k = 8..15, word 1 is k = 40..47
    assert blob[16 * 4] == g["w4a16_codes8to15"]
    assert blob[16 * 4 + 1] == g["w4a16_codes8to15"]
    q2 = _pattern(K, N, lambda k, n: n % 16)
    blob2 = np.frombuffer(layout.blob_w4a16(gen.pack_nibbles_u32(q2),
                                            np.ones((2, N), np.float16)), dtype="<u4")
    # lane 5 (c=5) holds column 5 everywhere: all nibbles 5
    assert blob2[5 * 4] == g["w4a16_n_mod16_lane5"]
    # chunk (b=1, g=0) starts at word (0*NB + 1)*256 (group-major); lane 0 is column 16
    assert blob2[1 * 256] == 0


def test_w4a16_chunks_are_group_major():
    # codes constant per (group, column block): v = (5*g + b) % 16; every word of chunk
    # (b, g) is then v repeated in all 8 nibbles, and the chunk sits at (g*NB + b)*1 KB
    K, N = 384, 128
    G, NB = K // 128, N // 16
    q = _pattern(K, N, lambda k, n: (5 * (k // 128) + n // 16) % 16)
    words = np.frombuffer(layout.blob_w4a16(gen.pack_nibbles_u32(q), np.ones((G, N), np.float16)),
                          dtype="<u4")
    for g in range(G):
        for b in range(NB):
            chunk = words[(g * NB + b) * 256:(g * NB + b + 1) * 256]
            assert np.all(chunk == 0x11111111 * ((5 * g + b) % 16)), (g, b)


def test_w4a16_scale_region_hand():
    K, N = 1280, 64                     # G = 10 -> G8 = 2, padded with zeros
    G = K // 128
    s = (np.arange(G)[:, None] * 64 + np.arange(N)[None, :]).astype(np.float16)
    blob = layout.blob_w4a16(gen.pack_nibbles_u32(np.zeros((K, N), np.uint8)), s)
    NB, G8 = N // 16, 2
    base = NB * G * 1024
    sc = np.frombuffer(blob[base:base + NB * G8 * 256], dtype=np.float16)
    # index ((b*G8 + g8)*16 + c)*8 + j = s[8*g8 + j][16*b + c]
    assert sc[((1 * G8 + 0) * 16 + 3) * 8 + 2] == s[2, 19]
    assert sc[((3 * G8 + 1) * 16 + 15) * 8 + 1] == s[9, 63]
    assert sc[((0 * G8 + 1) * 16 + 0) * 8 + 2] == 0        # g = 10 is padding


def test_w4a8_hand_derived_words():
    K, N = 128, 64
    q = _pattern(K, N, lambda k, n: k % 16)                 # two's complement nibbles
    blob = np.frombuffer(layout.blob_w4a8(gen.pack_nibbles_u32(q),
                                          np.ones((1, N), np.int8),
                                          np.ones(N, np.float16)), dtype="<u4")
    assert blob[0] == _golden()["w4a8_lane0_word0"]
    assert blob[1] == _golden()["w4a8_lane0_word1"]


def test_w2w4_hand_derived_words_and_desc():
    K, N = 128, 64
    q = _pattern(K, N, lambda k, n: (k % 4) + 4 * ((k // 32) % 4))
    mask = np.zeros((1, N), dtype=bool)
    mask[0, [0, 2, 17]] = True
    bm = gen.bitmap_from_mask(mask)
    q = np.where(np.repeat(mask, 128, axis=0), q, q & 3).astype(np.uint8)
    blob = layout.blob_w2w4(q, bm, np.ones((1, N), np.float16))
    g = _golden()
    words = np.frombuffer(blob, dtype="<u4")
    assert words[0] == g["w2w4_base_l0_s0"]
    G, NB = 1, 4
    d0 = NB * G * 512
    desc = np.frombuffer(blob[d0:d0 + NB * G * 8], dtype="<u4").reshape(NB, 2)
    assert desc.tolist() == [[0, 0b101], [2, 0b10], [3, 0], [3, 0]]
    h0 = d0 + 256 + 1024                # desc region: 32 B -> 256; scales: NB*G8*256 = 1024
    hi = np.frombuffer(blob[h0:h0 + 96], dtype="<u4")
    assert hi[0] == g["w2w4_high_col0_h0_s0"]
    assert hi[1] == g["w2w4_high_col0_h0_s1"]
    assert len(blob) == layout.packed_bytes(layout.FMT_W2W4, K, N, n4=3)


@pytest.mark.parametrize("K,N", [(128, 64), (1280, 192), (1024, 1024)])
def test_w4a16_round_trip_and_size(K, N):
    p = gen.w4a16_problem(1, K, N, seed=K + N, activations=False)
    blob = layout.blob_w4a16(p["codes"], p["scales"])
    assert len(blob) == layout.packed_bytes(layout.FMT_W4A16, K, N)
    codes, scales = layout.decode_w4a16(blob, K, N)
    assert np.array_equal(gen.pack_nibbles_u32(codes), p["codes"])
    assert np.array_equal(scales.view(np.uint16), p["scales"].view(np.uint16))


def test_w4a16_blob_is_a_permutation_of_nibbles():
    p = gen.w4a16_problem(1, 512, 128, seed=3, activations=False)
    blob = np.frombuffer(layout.blob_w4a16(p["codes"], p["scales"]), dtype=np.uint8)
    code_bytes = blob[:4 * 8 * 1024]
    hist_blob = np.bincount(np.concatenate([code_bytes & 15, code_bytes >> 4]), minlength=16)
    src = p["codes"].view(np.uint8).ravel()
    hist_src = np.bincount(np.concatenate([src & 15, src >> 4]), minlength=16)
    assert np.array_equal(hist_blob, hist_src)


def test_sizes_and_padding_zero():
    K, N = 1152, 320             # G = 9 (odd), NB = 20
    p = gen.w4a16_problem(1, K, N, seed=1, activations=False)
    blob = layout.blob_w4a16(p["codes"], p["scales"])
    G, NB, G8 = 9, 20, 2
    codes_end = NB * G * 1024
    sc_end = codes_end + NB * G8 * 256
    assert len(blob) == sc_end        # both already multiples of 256
    sc = np.frombuffer(blob[codes_end:sc_end], dtype=np.uint16).reshape(NB, G8, 16, 8)
    assert np.all(sc[:, 1, :, 1:] == 0)   # groups 9..15 of block g8 = 1 are padding


def test_w2w4_all_four_bit_base_plus_high_reconstruct_w4a16_words():
    # with every group 4-bit, (base | high << 2) per slot must rebuild the W4A16 words
    K, N = 256, 64
    p = gen.w4a16_problem(1, K, N, seed=8, activations=False)
    from oracle.ref import unpack_u4
    q = unpack_u4(p["codes"]).astype(np.uint8)
    mask = np.ones((K // 128, N), dtype=bool)
    blob = layout.blob_w2w4(q, gen.bitmap_from_mask(mask), p["scales"])
    w16 = np.frombuffer(layout.blob_w4a16(p["codes"], p["scales"]), dtype="<u4")
    NB, G = N // 16, K // 128
    base = np.frombuffer(blob[:NB * G * 512], dtype="<u4").reshape(G, NB, 64, 2)
    d0 = NB * G * 512
    h0 = d0 + 256 + 1024                # desc: 64 B -> 256; scales: NB*G8*256 = 1024
    high_w = np.frombuffer(blob[h0:h0 + 32 * NB * G * 16], dtype="<u4").reshape(G, NB, 16, 4, 2)
    high = high_w.transpose(0, 1, 3, 2, 4).reshape(G, NB, 64, 2)   # (g, b, h, c, s) -> lane
    w16 = w16[:NB * G * 256].reshape(G, NB, 64, 4)
    for s in range(2):
        lo0 = base[..., s] & 0x33333333
        lo1 = (base[..., s] >> 2) & 0x33333333
        hi0 = (high[..., s] << 2) & 0xCCCCCCCC
        hi1 = high[..., s] & 0xCCCCCCCC
        assert np.array_equal(lo0 | hi0, w16[..., 2 * s])
        assert np.array_equal(lo1 | hi1, w16[..., 2 * s + 1])


# --------------------------------------------------------------------------- W4G
def test_w4g_codes_region_is_w4a16():
    p = gen.w4a16_problem(1, 512, 128, seed=2)
    a = layout.blob_w4a16(p["codes"], p["scales"])
    b = layout.blob_w4g(p["codes"], p["scales"][::2], None, 256, "fp16")
    n = 512 * 128 // 2
    assert a[:n] == b[:n]


def test_w4g_param_entries_hand_positions():
    K, N = 256, 64
    qw = np.zeros((K // 8, N), np.uint32)
    # gs = 64, stored zeros: 4 groups; scales as bf16 patterns 0x1000 + 16 g + n % 16
    s = np.array([[0x1000 + 16 * g + (n % 16) for n in range(N)] for g in range(4)], np.uint16)
    z = np.array([[(g * 5 + n) % 16 for n in range(N)] for g in range(4)], np.uint8)
    blob = layout.blob_w4g(qw, s, z, 64, "bf16")
    base = K * N // 2
    ent = np.frombuffer(blob[base:base + 4 * N * 4], dtype="<u4")
    # group 3, column 5: chunk row 1, second of its pair -> index (1*64 + 5)*2 + 1 = 139
    assert ent[139] == (0x1000 + 48 + 5) | (((15 + 5) % 16) << 16)
    # group 0, column 63 -> index 63*2 = 126; group 1, column 0 -> index 1
    assert ent[126] == (0x1000 + 15) | ((63 % 16) << 16)
    assert ent[1] == (0x1000 + 16) | (5 << 16)
    # gs = 128 without zeros: fp16 scale bits, entry (g, n) at g*N + n
    s16 = np.arange(2 * N, dtype=np.float16).reshape(2, N) / 64
    blob = layout.blob_w4g(qw, s16, None, 128, "fp16")
    ent = np.frombuffer(blob[base:base + 2 * N * 2], dtype="<u2")
    assert ent[N + 7] == s16[1, 7].view(np.uint16)
    assert len(blob) == base + 256 + 0  # 2*64*2 = 256 bytes of entries


def test_w4g_group_size_validation():
    with pytest.raises(ValueError):
        layout.packed_bytes_w4g(256, 64, 96, False)
    with pytest.raises(ValueError):
        layout.packed_bytes_w4g(384, 64, 256, False)
    assert layout.packed_bytes_w4g(384, 64, 384, True) == 384 * 64 // 2 + 256
