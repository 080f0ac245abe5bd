"""Independent implementation of the repacked weight blob layout (CPU, NumPy).

The GPU repack reorders codes and scales into the order in which the GEMM
kernels consume them (the arbitrary-precision Tensor Core page's abstract
preprocesses matrices into a layout suited to the later computation; the 2-bit
page's abstract stores mixed groups with aligned memory access in mind). This module builds the same
bytes from the canonical arrays with NumPy index arithmetic, written from the
layout specification alone, so the GPU blob can be compared byte for byte.

Layout specification (all integers little-endian; G = K/128 groups,
NB = N/16 column blocks, G8 = ceil(G/8); lane l in 0..63 has column
c = l % 16 and quarter h = l // 16; every region starts at a multiple of 256
bytes and its size is rounded up to 256):

W4A16 (format 1)
  codes   G*NB chunks of 1024 B, chunk (b, g) at (g*NB + b)*1024 (group-major:
          the chunks of one group of 128 k are adjacent for all column blocks,
          so the waves of a launch, which advance through K together, read
          neighbouring kilobytes at the same time). Lane l owns
          16 B at +16*l: words t = 0..3. Word t holds the codes of
          k = 128*g + 32*t + 8*h + e (e = 0..7), column n = 16*b + c, with
          element e in nibble sigma(e): sigma(e) = e/2 for even e and
          4 + (e-1)/2 for odd e.
  scales  fp16 at index ((b*G8 + g8)*16 + c)*8 + j  = s[8*g8 + j][16*b + c]
          (0 where 8*g8 + j >= G).

W4A8 (format 2)
  codes   same chunk geometry, but word t = 2*u + s (u, s in 0..1) holds
          k = 128*g + 64*u + 16*h + 8*s + e; element e in nibble tau(e):
          tau(e) = 2*e for e < 4 and 2*(e-4) + 1 for e >= 4; the nibble holds
          the biased code (q mod 16) XOR 8 = q + 8 in 0..15.
  gscales int8 at index ((b*G8 + g8)*16 + c)*8 + j = s_g[8*g8 + j][16*b + c].
  cscales fp16[N] = s_c[n].

W2W4 mixed (format 3)
  base    G*NB chunks of 512 B, chunk (b, g) at (g*NB + b)*512. Lane l owns 8 B
          at +8*l: words s = 0, 1. For slot p = 0..7 let e = sigma^-1(p); bits
          [4p, 4p+1] hold lo2 of the W4A16 word-2s code at slot p
          (k = 128*g + 32*(2s) + 8*h + e) and bits [4p+2, 4p+3] hold lo2 of the
          W4A16 word-(2s+1) code at slot p (k + 32).
          lo2 = code & 3.
  desc    8 B per chunk (b, g) at (g*NB + b)*8: u32 off, u32 mask. mask bit c is
          set when group (g, 16*b + c) is 4-bit; off is the count of 4-bit
          groups in all chunks before (b, g) in (g*NB + b) order.
  scales  as W4A16.
  high    for every 4-bit group (g, n = 16*b + c): 32 B at
          32*(off(b, g) + rank(c)), rank(c) = set mask bits below c; quarter h
          at +8*h holds 2 words in the base-plane arrangement but with
          hi2 = (code >> 2) & 3.

W4G (format 4: 4-bit codes on a general grid -- group length gs = 64 or a
multiple of 128 dividing K, optional stored zero points, fp16 or bf16
activations and scales)
  codes   as W4A16 (chunks of 128 k, whatever gs is).
  params  one entry per (group g = k // gs, column n): the scale's 16-bit
          pattern (fp16 or bf16) when there are no stored zero points, else a
          u32 = scale bits | zero point << 16. With P = 2 for gs = 64 and
          P = 1 otherwise, entry (g, n) sits at index ((g // P)*N + n)*P + g % P,
          so the entries of the two 64-k groups of one 128-k chunk of a column
          are adjacent.

W4A16 2:4 sparse (format 5: at most two nonzero weights, i.e. codes other
than 8, in every 4 consecutive k of a column)
  chunks  G*NB chunks of 768 B, chunk (b, g) at (g*NB + b)*768. Lane l owns
          12 B at +12*l: code words s = 0, 1 (64-k steps), then its position
          word. Code word s covers
          k = 128*g + 64*s + 16*h + 4*j + p (quads j = 0..3, positions p = 0..3)
          of column n = 16*b + c; each quad keeps two positions p0 < p1 (the
          positions of its codes other than 8, completed with the lowest other
          positions); kept value v = 2*j + i (i = 0 for p0, 1 for p1) sits in
          nibble sigma(v) (the W4A16 nibble order).
          The position word's bits 16*s + 2*v .. +1 hold the position p of
          kept value v of code word s.
  scales  as W4A16.
  status  256 B; u32 at +0 = number of quads that break the 2:4 structure
          (0 for a valid blob), the rest zero.

Bit-plane W_b A8 (format 6, b = 1..8 bits of a bipolar-INT code U)
  chunks  G*NB chunks of 256*b B, chunk (b_, g) at (g*NB + b_)*256*b. Lane l
          owns 4*b B at +4*b*l: plane words i = 0..b-1; bit 16*u + j of plane
          word i is bit i of U at k = 128*g + 64*u + 16*h + j (u = 0, 1;
          j = 0..15), column n = 16*b_ + c.
  cscales fp16[N] = s_c[n].
"""

from __future__ import annotations

import numpy as np

GROUP = 128

FMT_W4A16 = 1
FMT_W4A8 = 2
FMT_W2W4 = 3
FMT_W4G = 4
FMT_SP24 = 5
FMT_BP = 6


def _align256(x: int) -> int:
    return (x + 255) // 256 * 256


def _sigma(e: int) -> int:
    return e // 2 if e % 2 == 0 else 4 + (e - 1) // 2


def _sigma_inv(p: int) -> int:
    return 2 * p if p < 4 else 2 * (p - 4) + 1


def _tau(e: int) -> int:
    return 2 * e if e < 4 else 2 * (e - 4) + 1


def _codes_by_lane(q: np.ndarray, K: int, N: int) -> np.ndarray:
    """Rearrange codes ``[K][N]`` into ``[G][NB][lane=16h+c][t][e]``.

    k = 128*g + 32*t + 8*h + e, n = 16*b + c.
    """
    G, NB = K // GROUP, N // 16
    x = np.asarray(q).reshape(G, 4, 4, 8, NB, 16)      # g, t, h, e, b, c
    x = x.transpose(0, 4, 2, 5, 1, 3)                  # g, b, h, c, t, e
    return x.reshape(G, NB, 64, 4, 8)


def _codes_by_lane_w4a8(q: np.ndarray, K: int, N: int) -> np.ndarray:
    """``[K][N]`` -> ``[G][NB][lane][t = 2u + s][e]`` with
    k = 128*g + 64*u + 16*h + 8*s + e."""
    G, NB = K // GROUP, N // 16
    x = np.asarray(q).reshape(G, 2, 4, 2, 8, NB, 16)   # g, u, h, s, e, b, c
    x = x.transpose(0, 5, 2, 6, 1, 3, 4)               # g, b, h, c, u, s, e
    return x.reshape(G, NB, 64, 4, 8)


def _scale_region(values: np.ndarray, G: int, N: int, dtype) -> bytes:
    """``[G][N]`` -> ``[NB][G8][16][8]`` (zero padded in g)."""
    NB, G8 = N // 16, (G + 7) // 8
    pad = np.zeros((G8 * 8, N), dtype=dtype)
    pad[:G] = np.asarray(values).astype(dtype)
    x = pad.reshape(G8, 8, NB, 16).transpose(2, 0, 3, 1)  # b, g8, c, j
    return np.ascontiguousarray(x).tobytes()


def _pad_to(buf: bytes, size: int) -> bytes:
    assert len(buf) <= size
    return buf + bytes(size - len(buf))


def _unpack_nibbles(qw: np.ndarray) -> np.ndarray:
    qw = np.asarray(qw, dtype=np.uint32)
    Kq, N = qw.shape
    out = np.empty((Kq, 8, N), dtype=np.uint32)
    for j in range(8):
        out[:, j, :] = (qw >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(Kq * 8, N)


def _check_shape(K: int, N: int):
    if K % GROUP or N % 64 or K <= 0 or N <= 0:
        raise ValueError("K must be a positive multiple of 128 and N of 64")


# --------------------------------------------------------------------------- sizes
def packed_bytes(fmt: int, K: int, N: int, n4: int = 0) -> int:
    _check_shape(K, N)
    G, NB = K // GROUP, N // 16
    G8 = (G + 7) // 8
    if fmt == FMT_W4A16:
        return _align256(NB * G * 1024) + _align256(NB * G8 * 256)
    if fmt == FMT_W4A8:
        return _align256(NB * G * 1024) + _align256(NB * G8 * 128) + _align256(2 * N)
    if fmt == FMT_W2W4:
        return (_align256(NB * G * 512) + _align256(NB * G * 8) + _align256(NB * G8 * 256)
                + _align256(32 * n4))
    if fmt == FMT_SP24:
        return _align256(NB * G * 768) + _align256(NB * G8 * 256) + 256
    raise ValueError("unknown format")


# --------------------------------------------------------------------------- W4A16
def _w4a16_codes(qw: np.ndarray, K: int, N: int) -> bytes:
    G, NB = K // GROUP, N // 16
    q = _codes_by_lane(_unpack_nibbles(qw), K, N)         # [G][NB][64][4][8]
    words = np.zeros(q.shape[:4], dtype=np.uint32)
    for e in range(8):
        words |= q[..., e].astype(np.uint32) << np.uint32(4 * _sigma(e))
    return _pad_to(words.astype("<u4").tobytes(), _align256(NB * G * 1024))


def blob_w4a16(qw: np.ndarray, scales: np.ndarray) -> bytes:
    qw = np.asarray(qw, dtype=np.uint32)
    K, N = qw.shape[0] * 8, qw.shape[1]
    _check_shape(K, N)
    G, NB = K // GROUP, N // 16
    codes = _w4a16_codes(qw, K, N)
    sc = _pad_to(_scale_region(np.asarray(scales, dtype=np.float16), G, N, np.float16),
                 _align256(NB * ((G + 7) // 8) * 256))
    out = codes + sc
    assert len(out) == packed_bytes(FMT_W4A16, K, N)
    return out


# --------------------------------------------------------------------------- 2:4 sparse
def blob_sp24(qw: np.ndarray, scales: np.ndarray) -> bytes:
    """Blob of format 5 from dense canonical codes (pruned weights hold code 8)
    and fp16 scales [K/128][N]. Raises ValueError if a quad keeps more than two
    codes other than 8."""
    qw = np.asarray(qw, dtype=np.uint32)
    K, N = qw.shape[0] * 8, qw.shape[1]
    _check_shape(K, N)
    G, NB = K // GROUP, N // 16
    q = _unpack_nibbles(qw).astype(np.int64)                      # [K][N]
    # [g][s][h][j][p][b][c] with k = 128g + 64s + 16h + 4j + p, n = 16b + c
    x = q.reshape(G, 2, 4, 4, 4, NB, 16)
    nz = x != 8
    if (nz.sum(axis=4) > 2).any():
        raise ValueError("codes break the 2:4 structure")
    # kept positions per quad: nonzero positions first, then the lowest others,
    # sorted ascending (a stable sort of the key "zero?" then position)
    key = (~nz).astype(np.int64) * 4 + np.arange(4).reshape(1, 1, 1, 1, 4, 1, 1)
    order = np.argsort(key, axis=4, kind="stable")[:, :, :, :, :2]
    pos = np.sort(order, axis=4)                                   # [g][s][h][j][2][b][c]
    vals = np.take_along_axis(x, pos, axis=4)
    # to [g][b][h][c][s][v = 2j + i]
    vals = vals.transpose(0, 5, 2, 6, 1, 3, 4).reshape(G, NB, 4, 16, 2, 8)
    pos = pos.transpose(0, 5, 2, 6, 1, 3, 4).reshape(G, NB, 4, 16, 2, 8)
    words = np.zeros((G, NB, 4, 16, 2), dtype=np.uint32)
    meta = np.zeros((G, NB, 4, 16), dtype=np.uint32)
    for v in range(8):
        words |= vals[..., v].astype(np.uint32) << np.uint32(4 * _sigma(v))
        for st in range(2):
            meta |= pos[..., st, v].astype(np.uint32) << np.uint32(16 * st + 2 * v)
    rec = np.concatenate([words.reshape(G, NB, 64, 2), meta.reshape(G, NB, 64, 1)], axis=3)
    chunks = _pad_to(rec.astype("<u4").tobytes(), _align256(NB * G * 768))
    sc = _pad_to(_scale_region(np.asarray(scales, dtype=np.float16), G, N, np.float16),
                 _align256(NB * ((G + 7) // 8) * 256))
    out = chunks + sc + bytes(256)
    assert len(out) == packed_bytes(FMT_SP24, K, N)
    return out


# --------------------------------------------------------------------------- bit planes
def packed_bytes_bitplane(K: int, N: int, bits: int) -> int:
    _check_shape(K, N)
    if not 1 <= bits <= 8:
        raise ValueError("bits must be 1..8")
    G, NB = K // GROUP, N // 16
    return _align256(NB * G * 256 * bits) + _align256(2 * N)


def blob_bitplane(codes_u8: np.ndarray, bits: int, chan_scales: np.ndarray) -> bytes:
    U = np.asarray(codes_u8).astype(np.uint32) & np.uint32(2 ** bits - 1)
    K, N = U.shape
    _check_shape(K, N)
    G, NB = K // GROUP, N // 16
    x = U.reshape(G, 2, 4, 16, NB, 16)                   # g, u, h, j, b, c
    x = x.transpose(0, 4, 2, 5, 1, 3).reshape(G, NB, 64, 32)   # g, b, lane, 16u + j
    words = np.zeros((G, NB, 64, bits), dtype=np.uint32)
    for i in range(bits):
        for t in range(32):
            words[..., i] |= ((x[..., t] >> np.uint32(i)) & np.uint32(1)) << np.uint32(t)
    chunks = _pad_to(words.astype("<u4").tobytes(), _align256(NB * G * 256 * bits))
    cs = _pad_to(np.asarray(chan_scales, dtype=np.float16).tobytes(), _align256(2 * N))
    out = chunks + cs
    assert len(out) == packed_bytes_bitplane(K, N, bits)
    return out


# --------------------------------------------------------------------------- W4G
def check_group_size(K: int, gs: int):
    if not (gs == 64 or (gs > 0 and gs % GROUP == 0 and K % gs == 0)):
        raise ValueError("group size must be 64 or a multiple of 128 that divides K")


def packed_bytes_w4g(K: int, N: int, gs: int, has_zeros: bool) -> int:
    _check_shape(K, N)
    check_group_size(K, gs)
    G, NB = K // GROUP, N // 16
    return _align256(NB * G * 1024) + _align256((K // gs) * N * (4 if has_zeros else 2))


def blob_w4g(qw: np.ndarray, scales: np.ndarray, zeros, gs: int, act: str) -> bytes:
    """``scales``: fp16 array (act fp16) or bf16 bit patterns (act bf16), [K/gs][N];
    ``zeros``: uint8 [K/gs][N] or None."""
    qw = np.asarray(qw, dtype=np.uint32)
    K, N = qw.shape[0] * 8, qw.shape[1]
    _check_shape(K, N)
    check_group_size(K, gs)
    Gs, P = K // gs, (2 if gs == 64 else 1)
    if act == "fp16":
        s16 = np.asarray(scales, dtype=np.float16).view(np.uint16)
    elif act == "bf16":
        s16 = np.asarray(scales, dtype=np.uint16)
    else:
        raise ValueError("act must be fp16 or bf16")
    assert s16.shape == (Gs, N)
    if zeros is None:
        ent = s16.astype("<u2")
    else:
        z = np.asarray(zeros).astype(np.uint32)
        assert z.shape == (Gs, N) and z.max(initial=0) <= 15
        ent = (s16.astype(np.uint32) | (z << np.uint32(16))).astype("<u4")
    ent = np.ascontiguousarray(ent.reshape(Gs // P, P, N).transpose(0, 2, 1))
    params = _pad_to(ent.tobytes(), _align256(Gs * N * ent.itemsize))
    out = _w4a16_codes(qw, K, N) + params
    assert len(out) == packed_bytes_w4g(K, N, gs, zeros is not None)
    return out


# --------------------------------------------------------------------------- W4A8
def blob_w4a8(qw: np.ndarray, group_scales: np.ndarray, chan_scales: np.ndarray) -> bytes:
    qw = np.asarray(qw, dtype=np.uint32)
    K, N = qw.shape[0] * 8, qw.shape[1]
    _check_shape(K, N)
    G, NB = K // GROUP, N // 16
    biased = _unpack_nibbles(qw) ^ np.uint32(8)            # two's complement q -> q + 8
    q = _codes_by_lane_w4a8(biased, K, N)
    words = np.zeros(q.shape[:4], dtype=np.uint32)
    for e in range(8):
        words |= q[..., e].astype(np.uint32) << np.uint32(4 * _tau(e))
    codes = _pad_to(words.astype("<u4").tobytes(), _align256(NB * G * 1024))
    gs = _pad_to(_scale_region(np.asarray(group_scales, dtype=np.int8), G, N, np.int8),
                 _align256(NB * ((G + 7) // 8) * 128))
    cs = _pad_to(np.asarray(chan_scales, dtype=np.float16).tobytes(), _align256(2 * N))
    out = codes + gs + cs
    assert len(out) == packed_bytes(FMT_W4A8, K, N)
    return out


# --------------------------------------------------------------------------- W2W4
def _bitmap_mask(bitmap: np.ndarray, G: int, N: int) -> np.ndarray:
    bitmap = np.asarray(bitmap, dtype=np.uint32)
    n = np.arange(N)
    return ((bitmap[:G, n // 32] >> (n % 32).astype(np.uint32)) & 1).astype(bool)


def _two_bit_words(plane: np.ndarray) -> np.ndarray:
    """``[G][NB][64][4][8]`` 2-bit values -> ``[G][NB][64][2]`` u32 words."""
    out = np.zeros(plane.shape[:3] + (2,), dtype=np.uint32)
    for s in range(2):
        for p in range(8):
            e = _sigma_inv(p)
            out[..., s] |= plane[..., 2 * s, e].astype(np.uint32) << np.uint32(4 * p)
            out[..., s] |= plane[..., 2 * s + 1, e].astype(np.uint32) << np.uint32(4 * p + 2)
    return out


def blob_w2w4(codes_u8: np.ndarray, bitmap: np.ndarray, scales: np.ndarray) -> bytes:
    codes_u8 = np.asarray(codes_u8, dtype=np.uint8)
    K, N = codes_u8.shape
    _check_shape(K, N)
    G, NB = K // GROUP, N // 16
    G8 = (G + 7) // 8
    mask = _bitmap_mask(bitmap, G, N)                      # [G][N]
    q = _codes_by_lane(codes_u8, K, N)                     # [G][NB][64][4][8]
    base = _two_bit_words(q & np.uint8(3))                 # [G][NB][64][2]
    high = _two_bit_words((q >> np.uint8(2)) & np.uint8(3))
    # descriptors in chunk order g*NB + b
    m_gb = mask.reshape(G, NB, 16)                          # [G][NB][16]
    cnt = m_gb.sum(axis=2).ravel()
    off = np.concatenate([[0], np.cumsum(cnt)[:-1]]).astype(np.uint32)
    bits = (m_gb.astype(np.uint32) << np.arange(16, dtype=np.uint32)).sum(axis=2).ravel()
    desc = np.stack([off, bits.astype(np.uint32)], axis=1).astype("<u4")
    n4 = int(cnt.sum())
    # high plane: quarter pieces of 4-bit groups in (g, b, c) order
    hi_words = high.reshape(G, NB, 4, 16, 2).transpose(0, 1, 3, 2, 4)   # g, b, c, h, s
    sel = hi_words[m_gb]                                    # [n4][4][2] in (g, b, c) order
    hbytes = sel.astype("<u4").tobytes()
    out = (_pad_to(base.astype("<u4").tobytes(), _align256(NB * G * 512))
           + _pad_to(desc.tobytes(), _align256(NB * G * 8))
           + _pad_to(_scale_region(np.asarray(scales, dtype=np.float16), G, N, np.float16),
                     _align256(NB * G8 * 256))
           + _pad_to(hbytes, _align256(32 * n4)))
    assert len(out) == packed_bytes(FMT_W2W4, K, N, n4)
    return out


# --------------------------------------------------------------------------- decoding
def decode_w4a16(blob: bytes, K: int, N: int):
    """Inverse of ``blob_w4a16``: returns (codes uint8[K][N], scales fp16[G][N])."""
    G, NB = K // GROUP, N // 16
    G8 = (G + 7) // 8
    raw = np.frombuffer(blob, dtype=np.uint8)
    words = raw[:NB * G * 1024].view("<u4").reshape(G, NB, 64, 4)
    q = np.zeros((G, NB, 64, 4, 8), dtype=np.uint8)
    for e in range(8):
        q[..., e] = (words >> np.uint32(4 * _sigma(e))) & 0xF
    codes = q.reshape(G, NB, 4, 16, 4, 8).transpose(0, 4, 2, 5, 1, 3).reshape(K, N)
    s0 = _align256(NB * G * 1024)
    sc = raw[s0:s0 + NB * G8 * 256].view(np.float16).reshape(NB, G8, 16, 8)
    scales = sc.transpose(1, 3, 0, 2).reshape(G8 * 8, N)[:G]
    return codes, scales
