"""Reference GEMMs on the CPU: explicit dequantization, then an fp64 matmul.

The methods on the pages (MARLIN's W4A16 kernel, OdysseyLLM's W4A8 FastGEMM,
the 2-bit page's mixed 2/4-bit kernel with asynchronous dequantization) all
compute the ordinary product of the activations with the dequantized weights;
they make it fast, they do not change its value. So the oracle is that
definition written out:

    W[k, n] = (q[k, n] - z) * s[k // 128, n]          (W4A16, mixed 2/4-bit)
    C       = A @ W                                    (fp64 accumulation)

and for W4A8 the exact integer accumulator

    acc[m, n] = sum_k A_i8[m, k] * q[k, n] * s_g[k // 128, n]
    C[m, n]   = acc[m, n] * a_scale[m] * s_c[n]

Readings where the pages are silent (each listed in the design notes):
zero point 8 for 4-bit and 2 for 2-bit codes, not stored; groups are 128
consecutive k of one column; dequantization is (q - z) * s, never q*s - z*s.

fp64 is exact for every dequantized weight (a 5-bit integer times an 11-bit
significand) and its matmul rounding (~K * 2**-53 relative) is far below fp16
resolution. For W4A8 every product and partial sum is an integer below 2**53, so
the fp64 matmul is exact and is returned as int64.
"""

from __future__ import annotations

import numpy as np

GROUP = 128


# --------------------------------------------------------------------------- unpacking
def unpack_u4(qw: np.ndarray) -> np.ndarray:
    """``uint32[K/8][N]`` -> ``int64[K][N]``; nibble j of word r is k = 8r + j."""
    qw = np.asarray(qw, dtype=np.uint32)
    Kq, N = qw.shape
    out = np.empty((Kq, 8, N), dtype=np.int64)
    for j in range(8):
        out[:, j, :] = (qw >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(Kq * 8, N)


def unpack_s4(qw: np.ndarray) -> np.ndarray:
    """Two's-complement int4 nibbles -> ``int64`` values in [-8, 7]."""
    u = unpack_u4(qw)
    return np.where(u >= 8, u - 16, u)


def bitmap_to_mask(bitmap: np.ndarray, N: int) -> np.ndarray:
    """``uint32[G][ceil(N/32)]`` -> ``bool[G][N]``; bit n%32 of word n//32."""
    bitmap = np.asarray(bitmap, dtype=np.uint32)
    n = np.arange(N)
    return ((bitmap[:, n // 32] >> (n % 32).astype(np.uint32)) & np.uint32(1)).astype(bool)


# --------------------------------------------------------------------------- W4A16
def dequant_w4a16(qw: np.ndarray, scales: np.ndarray, zero: int = 8) -> np.ndarray:
    """fp64 ``W[k, n] = (q[k, n] - zero) * s[k // 128, n]``."""
    q = unpack_u4(qw)
    K = q.shape[0]
    s = np.asarray(scales).astype(np.float64)
    return (q - zero).astype(np.float64) * s[np.arange(K) // GROUP, :]


def gemm_w4a16(A: np.ndarray, qw: np.ndarray, scales: np.ndarray,
               cols: np.ndarray | None = None, slab: int = 2048) -> np.ndarray:
    """fp64 ``C = A @ dequant(W)``; optionally only the listed output columns.

    The K dimension is processed in slabs of ``slab`` rows (a multiple of 128)
    only to bound memory for large layers; each slab's product is added in
    order, which changes nothing beyond fp64 rounding.
    """
    A64 = np.asarray(A).astype(np.float64)
    qw = np.asarray(qw)
    scales = np.asarray(scales)
    if cols is not None:
        qw = qw[:, cols]
        scales = scales[:, cols]
    K = qw.shape[0] * 8
    N = qw.shape[1]
    C = np.zeros((A64.shape[0], N), dtype=np.float64)
    for k0 in range(0, K, slab):
        k1 = min(K, k0 + slab)
        W = dequant_w4a16(qw[k0 // 8:k1 // 8], scales[k0 // GROUP:(k1 + GROUP - 1) // GROUP])
        C += A64[:, k0:k1] @ W
    return C


# --------------------------------------------------------------------------- 2:4 sparse W4A16
def sparse24_violations(qw: np.ndarray, zero: int = 8) -> int:
    """Number of runs of 4 consecutive k of one column (k = 4j .. 4j+3) holding
    more than two nonzero weights, i.e. more than two codes other than the
    zero point. The MARLIN abstract extends its kernel to 2:4 sparsity: at most
    two of every four consecutive weights along K are nonzero. Such weights are
    an ordinary W4A16 matrix whose pruned entries hold the zero point, so the
    2:4 GEMM's value is ``gemm_w4a16`` on the dense codes; this function checks
    the structure the sparse kernel relies on."""
    q = unpack_u4(qw)
    K, N = q.shape
    nz = (q != zero).reshape(K // 4, 4, N).sum(axis=1)
    return int((nz > 2).sum())


# --------------------------------------------------------------------------- bit-plane W_b A8
def bipolar_value(u: np.ndarray, bits: int) -> np.ndarray:
    """Value of a b-bit bipolar integer with stored bits u_i (0/1): every bit
    plane i contributes +2^i or -2^i, so w = sum_i 2^i (2 u_i - 1) =
    2 U - (2^b - 1) with U the bits read as an unsigned integer: the odd
    integers -(2^b - 1) .. 2^b - 1, symmetric about zero (the bipolar-INT format
    of the arbitrary-precision Tensor Core page's abstract)."""
    if not 1 <= bits <= 8:
        raise ValueError("bits must be 1..8")
    return 2 * np.asarray(u).astype(np.int64) - (2 ** bits - 1)


def gemm_bitplane_a8(A_i8: np.ndarray, codes_u8: np.ndarray, bits: int, a_scale: np.ndarray,
                     chan_scales: np.ndarray, cols: np.ndarray | None = None):
    """W_b A8 GEMM on bipolar-INT weights with a per-column fp16 scale and
    int8 activations with a per-row fp16 scale:

        acc[m, n] = sum_k A[m, k] * (2 U[k, n] - (2^b - 1))   (exact, int64)
        C[m, n]   = acc[m, n] * a_scale[m] * s_c[n]           (fp64)

    ``codes_u8`` holds U (only its low ``bits`` bits). Every product and partial
    sum is an integer below 2^53 in magnitude, so the fp64 matmul is exact."""
    U = np.asarray(codes_u8).astype(np.int64) & (2 ** bits - 1)
    sc = np.asarray(chan_scales).astype(np.float64)
    if cols is not None:
        U = U[:, cols]
        sc = sc[cols]
    W = bipolar_value(U, bits).astype(np.float64)
    acc = (np.asarray(A_i8).astype(np.float64) @ W).astype(np.int64)
    C = acc.astype(np.float64) * np.asarray(a_scale).astype(np.float64)[:, None] * sc[None, :]
    return acc, C


# --------------------------------------------------------------------------- W4 general grid
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 values given as their 16-bit patterns -> fp64 (exact).

    A bfloat16 number is the upper half of an IEEE binary32 number with the
    same sign, exponent and leading 7 fraction bits, so widening the pattern to
    32 bits with zero low bits gives the binary32 number exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def act_to_f64(x: np.ndarray, act: str) -> np.ndarray:
    """Activations or scales in the activation type -> fp64 (exact): fp16
    arrays as they are, bf16 as uint16 bit patterns."""
    if act == "fp16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if act == "bf16":
        return bf16_to_f64(x)
    raise ValueError(f"unknown activation type {act!r}")


def dequant_w4g(qw: np.ndarray, scales: np.ndarray, zeros: np.ndarray | None,
                group_size: int, act: str = "fp16") -> np.ndarray:
    """fp64 ``W[k, n] = (q[k, n] - z[g, n]) * s[g, n]`` with ``g = k // group_size``.

    The quantization grid variants of the 4-bit weight GEMM: the 2-bit page's
    abstract and the Atom review's method section both quantize weights by
    groups without fixing the group length, so the group is any number of
    consecutive k of one column (64, 128, ..., K for one scale per column);
    ``zeros`` holds one stored integer zero point 0..15 per (group, column),
    or None for the implicit zero point 8; the scales are in the activation
    type. Every product is exact in fp64 (a 5-bit integer times a significand
    of at most 11 bits)."""
    q = unpack_u4(qw)
    K, N = q.shape
    if group_size <= 0 or K % group_size:
        raise ValueError("group_size must divide K")
    g = np.arange(K) // group_size
    s = act_to_f64(scales, act)
    if s.shape != (K // group_size, N):
        raise ValueError(f"scales shape {s.shape} != {(K // group_size, N)}")
    if zeros is None:
        z = np.full((K // group_size, N), 8, dtype=np.int64)
    else:
        z = np.asarray(zeros).astype(np.int64)
        if z.shape != s.shape:
            raise ValueError("zeros shape must match scales")
    return (q - z[g, :]).astype(np.float64) * s[g, :]


def gemm_w4g(A: np.ndarray, qw: np.ndarray, scales: np.ndarray, zeros: np.ndarray | None,
             group_size: int, act: str = "fp16", cols: np.ndarray | None = None) -> np.ndarray:
    """fp64 ``C = A @ dequant_w4g(...)`` (A in the activation type: an fp16
    array, or bf16 bit patterns as uint16); optionally only the listed columns."""
    qw = np.asarray(qw)
    scales = np.asarray(scales)
    if cols is not None:
        qw = qw[:, cols]
        scales = scales[:, cols]
        zeros = None if zeros is None else np.asarray(zeros)[:, cols]
    return act_to_f64(A, act) @ dequant_w4g(qw, scales, zeros, group_size, act)


# --------------------------------------------------------------------------- W4A8
def w4a8_weights_int(qw: np.ndarray, group_scales: np.ndarray) -> np.ndarray:
    """Integer weights ``q[k, n] * s_g[k // 128, n]`` as int64."""
    q = unpack_s4(qw)
    K = q.shape[0]
    sg = np.asarray(group_scales).astype(np.int64)
    return q * sg[np.arange(K) // GROUP, :]


def w4a8_acc(A_i8: np.ndarray, qw: np.ndarray, group_scales: np.ndarray,
             cols: np.ndarray | None = None, slab: int = 2048) -> np.ndarray:
    """Exact ``acc[m, n] = sum_k A[m, k] * q[k, n] * s_g[k // 128, n]`` (int64)."""
    A64 = np.asarray(A_i8).astype(np.float64)
    qw = np.asarray(qw)
    group_scales = np.asarray(group_scales)
    if cols is not None:
        qw = qw[:, cols]
        group_scales = group_scales[:, cols]
    K = qw.shape[0] * 8
    N = qw.shape[1]
    acc = np.zeros((A64.shape[0], N), dtype=np.float64)
    for k0 in range(0, K, slab):
        k1 = min(K, k0 + slab)
        Wi = w4a8_weights_int(qw[k0 // 8:k1 // 8],
                              group_scales[k0 // GROUP:(k1 + GROUP - 1) // GROUP])
        # every term and partial sum is an integer of magnitude < 2**53: exact
        acc += A64[:, k0:k1] @ Wi.astype(np.float64)
    return acc.astype(np.int64)


def w4a8_out(acc: np.ndarray, a_scale: np.ndarray, chan_scales: np.ndarray,
             cols: np.ndarray | None = None) -> np.ndarray:
    """fp64 ``C[m, n] = acc[m, n] * a_scale[m] * s_c[n]``."""
    sc = np.asarray(chan_scales).astype(np.float64)
    if cols is not None:
        sc = sc[cols]
    return (np.asarray(acc).astype(np.float64) * np.asarray(a_scale).astype(np.float64)[:, None]
            * sc[None, :])


def gemm_w4a8(A_i8, qw, group_scales, a_scale, chan_scales, cols=None):
    acc = w4a8_acc(A_i8, qw, group_scales, cols=cols)
    return acc, w4a8_out(acc, a_scale, chan_scales, cols=cols)


def quantize_a8(A: np.ndarray):
    """Per-token (per-row) dynamic int8 quantization of fp16 activations, the
    input side of the W4A8 GEMM (the Atom review's method section adapts the
    activation quantization parameters to each activation matrix at inference
    time; the OdysseyLLM abstract's W4A8 GEMM consumes int8 activations).

    The pages give no formula; the reading taken here is symmetric absmax:

        a_s[m]   = fp16(amax_m / 127),  amax_m = max_k |A[m, k]|   (fp32 division,
                                                                  one RNE rounding)
        q[m, k]  = clamp(rint(fp32(A[m, k]) / fp32(a_s[m])), -127, 127)
                   (fp32 division, round half to even)

    A row whose a_s is zero (all zeros, or so small that amax/127 rounds to fp16
    zero) quantizes to zeros. Inputs must be finite. Returns (q int8[M][K],
    a_s fp16[M]).
    """
    A32 = np.asarray(A, dtype=np.float16).astype(np.float32)
    amax = np.abs(A32).max(axis=1) if A32.shape[1] else np.zeros(A32.shape[0], np.float32)
    a_s = (amax / np.float32(127.0)).astype(np.float32).astype(np.float16)
    s32 = a_s.astype(np.float32)
    q = np.zeros(A32.shape, dtype=np.float32)
    nz = s32 > 0
    q[nz] = np.rint(A32[nz] / s32[nz, None])
    return np.clip(q, -127, 127).astype(np.int8), a_s


# --------------------------------------------------------------------------- mixed 2/4-bit
def dequant_w2w4(codes_u8: np.ndarray, bitmap: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp64 ``W[k, n] = (q[k, n] - z[g, n]) * s[g, n]`` with ``g = k // 128`` and
    ``z = 8`` for 4-bit groups (bitmap bit set), ``z = 2`` for 2-bit groups."""
    q = np.asarray(codes_u8).astype(np.int64)
    K, N = q.shape
    g = np.arange(K) // GROUP
    mask = bitmap_to_mask(bitmap, N)
    z = np.where(mask, 8, 2)[g, :]
    s = np.asarray(scales).astype(np.float64)[g, :]
    return (q - z).astype(np.float64) * s


def gemm_w2w4(A: np.ndarray, codes_u8: np.ndarray, bitmap: np.ndarray, scales: np.ndarray,
              cols: np.ndarray | None = None) -> np.ndarray:
    """fp64 ``C = A @ dequant_w2w4(...)``, optionally for selected columns."""
    codes_u8 = np.asarray(codes_u8)
    scales = np.asarray(scales)
    bitmap = np.asarray(bitmap)
    N = codes_u8.shape[1]
    if cols is not None:
        mask = bitmap_to_mask(bitmap, N)[:, cols]
        codes_u8 = codes_u8[:, cols]
        scales = scales[:, cols]
        W = _dequant_w2w4_mask(codes_u8, mask, scales)
    else:
        W = dequant_w2w4(codes_u8, bitmap, scales)
    return np.asarray(A).astype(np.float64) @ W


def _dequant_w2w4_mask(codes_u8, mask, scales):
    q = np.asarray(codes_u8).astype(np.int64)
    g = np.arange(q.shape[0]) // GROUP
    z = np.where(mask, 8, 2)[g, :]
    return (q - z).astype(np.float64) * np.asarray(scales).astype(np.float64)[g, :]


# --------------------------------------------------------------------------- bookkeeping
def bits_per_weight_w2w4(bitmap: np.ndarray, K: int, N: int) -> float:
    """Average stored bits per weight of the mixed format: 2 base bits for every
    weight, 2 more for weights of 4-bit groups, one fp16 scale and one bitmap bit
    per group of 128."""
    n4 = int(bitmap_to_mask(bitmap, N).sum())
    G = (K // GROUP) * N
    bits = 2 * K * N + 2 * GROUP * n4 + 16 * G + G
    return bits / (K * N)
