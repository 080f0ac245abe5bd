"""Seeded generators for the quantized-GEMM workloads.

Every tensor is drawn from its own ``numpy`` generator, seeded from a
``SeedSequence`` of (seed, workload kind, shape, tensor id). Weight tensors do
not depend on M, so one weight set serves a whole sweep over batch sizes.

Canonical formats (the bytes both the oracle and the GPU library read):

* 4-bit codes: ``uint32[K/8][N]``; nibble ``j`` (bits 4j..4j+3) of word
  ``[r][n]`` is the code of weight ``(k = 8r + j, n)``. W4A16 codes are
  unsigned 0..15; W4A8 codes are two's-complement int4 in -8..7.
* mixed 2/4-bit codes: ``uint8[K][N]``, one code per byte (0..15 or 0..3).
* group scales: one value per (group of 128 consecutive k, column n):
  ``float16[K/128][N]`` (W4A16, mixed) or ``int8[K/128][N]`` (W4A8).
* precision bitmap: ``uint32[K/128][ceil(N/32)]``; bit ``n % 32`` of word
  ``[g][n // 32]`` is 1 when group (g, n) holds 4-bit codes.

Value distributions follow the workloads of the MARLIN paper (4-bit weights,
fp16 activations, batched decode), OdysseyLLM's W4A8 setting, and the
"Enabling Fast 2-bit LLM on GPUs" page (a small fraction of large-range groups
kept at 4 bits); the numeric ranges are this library's stated workload recipe.
"""

from __future__ import annotations

import numpy as np

GROUP = 128

_KIND_W4A16 = 1
_KIND_W4A8 = 2
_KIND_W2W4 = 3
_KIND_W4G = 4
_KIND_SP24 = 5
_KIND_BP = 6


def rng_for(seed: int, *tags: int) -> np.random.Generator:
    """Independent generator for one tensor, keyed by ``(seed, *tags)``."""
    return np.random.default_rng(np.random.SeedSequence([int(seed)] + [int(t) for t in tags]))


def pack_nibbles_u32(codes: np.ndarray) -> np.ndarray:
    """Pack ``uint8[K][N]`` codes (low 4 bits used) into ``uint32[K/8][N]``.

    Nibble j of output word [r][n] receives codes[8r + j][n].
    """
    codes = np.asarray(codes)
    K, N = codes.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    c = (codes.astype(np.uint32) & np.uint32(0xF)).reshape(K // 8, 8, N)
    out = np.zeros((K // 8, N), dtype=np.uint32)
    for j in range(8):
        out |= c[:, j, :] << np.uint32(4 * j)
    return out


def _fp16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32).astype(np.float16)


def _fp16_uniform(rng: np.random.Generator, lo: float, hi: float, shape) -> np.ndarray:
    return rng.uniform(lo, hi, size=shape).astype(np.float16)


def w4a16_problem(M: int, K: int, N: int, seed: int = 0, weights: bool = True,
                  activations: bool = True) -> dict:
    """W4A16 workload: fp16 A ~ N(0,1); uint4 codes uniform 0..15 (zero point 8);
    fp16 scales uniform in [0.005, 0.02], one per (group of 128 k, column)."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    out = {"M": M, "K": K, "N": N, "zero": 8}
    if activations:
        out["A"] = _fp16_normal(rng_for(seed, _KIND_W4A16, 0, M, K), (M, K))
    if weights:
        q = rng_for(seed, _KIND_W4A16, 1, K, N).integers(0, 16, size=(K, N), dtype=np.uint8)
        out["codes"] = pack_nibbles_u32(q)
        out["scales"] = _fp16_uniform(rng_for(seed, _KIND_W4A16, 2, K, N), 0.005, 0.02,
                                      (K // GROUP, N))
    return out


def w4a8_problem(M: int, K: int, N: int, seed: int = 0) -> dict:
    """W4A8 workload: int8 A uniform in [-127, 127] with a per-token fp16 scale
    uniform in [0.01, 0.03]; signed int4 weights uniform in [-8, 7]; int8 group
    scales uniform in [1, 16] per (group of 128 k, column); fp16 per-column scale
    uniform in [5e-4, 1e-3]."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    A = rng_for(seed, _KIND_W4A8, 0, M, K).integers(-127, 128, size=(M, K), dtype=np.int16)
    a_scale = _fp16_uniform(rng_for(seed, _KIND_W4A8, 1, M, K), 0.01, 0.03, (M,))
    q = rng_for(seed, _KIND_W4A8, 2, K, N).integers(-8, 8, size=(K, N), dtype=np.int16)
    s_g = rng_for(seed, _KIND_W4A8, 3, K, N).integers(1, 17, size=(K // GROUP, N), dtype=np.int16)
    s_c = _fp16_uniform(rng_for(seed, _KIND_W4A8, 4, K, N), 5e-4, 1e-3, (N,))
    return {
        "M": M, "K": K, "N": N,
        "A": A.astype(np.int8),
        "a_scale": a_scale,
        # two's-complement nibbles: the low 4 bits of the int16 value
        "codes": pack_nibbles_u32((q & 0xF).astype(np.uint8)),
        "group_scales": s_g.astype(np.int8),
        "chan_scales": s_c,
    }


def select_4bit_groups(latent: np.ndarray, frac: float = 0.10) -> np.ndarray:
    """Choose which (group, column) pairs keep 4-bit codes.

    Following the 2-bit page's recipe of giving 4 bits only to a small fraction of
    groups with the largest weight range: rank groups by (max - min) of their 128
    latent values, keep the ``round(frac * G * N)`` largest, ties broken toward the
    lower linear index ``g * N + n``. Returns ``bool[G][N]``.
    """
    K, N = latent.shape
    G = K // GROUP
    blk = latent.reshape(G, GROUP, N)
    rng_ = (blk.max(axis=1) - blk.min(axis=1)).astype(np.float64).ravel()
    n4 = int(round(frac * G * N))
    # stable sort on -range keeps the lower linear index first among equal ranges
    order = np.argsort(-rng_, kind="stable")
    mask = np.zeros(G * N, dtype=bool)
    mask[order[:n4]] = True
    return mask.reshape(G, N)


def bitmap_from_mask(mask: np.ndarray) -> np.ndarray:
    """``bool[G][N]`` -> ``uint32[G][ceil(N/32)]`` with bit n%32 of word n//32."""
    G, N = mask.shape
    W = (N + 31) // 32
    out = np.zeros((G, W), dtype=np.uint32)
    for n in range(N):
        out[:, n // 32] |= mask[:, n].astype(np.uint32) << np.uint32(n % 32)
    return out


def w2w4_problem(M: int, K: int, N: int, seed: int = 0, frac4: float = 0.10,
                 mask: np.ndarray | None = None) -> dict:
    """Mixed 2/4-bit workload: fp16 A ~ N(0,1); groups of 128 k per column; the
    ``frac4`` fraction of groups with the largest latent range get 4-bit codes
    uniform in 0..15 (zero point 8), the rest 2-bit codes uniform in 0..3 (zero
    point 2); fp16 scales uniform in [0.005, 0.02]. ``mask`` overrides the
    selection (``bool[K/128][N]``)."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    G = K // GROUP
    A = _fp16_normal(rng_for(seed, _KIND_W2W4, 0, M, K), (M, K))
    if mask is None:
        latent = rng_for(seed, _KIND_W2W4, 1, K, N).standard_normal(size=(K, N), dtype=np.float32)
        mask = select_4bit_groups(latent, frac4)
    mask = np.asarray(mask, dtype=bool)
    r = rng_for(seed, _KIND_W2W4, 2, K, N)
    c4 = r.integers(0, 16, size=(K, N), dtype=np.uint8)
    c2 = (c4 & np.uint8(3))  # independent low bits of a uniform 0..15 draw are uniform 0..3
    wide = np.repeat(mask, GROUP, axis=0)
    codes = np.where(wide, c4, c2).astype(np.uint8)
    scales = _fp16_uniform(rng_for(seed, _KIND_W2W4, 3, K, N), 0.005, 0.02, (G, N))
    return {
        "M": M, "K": K, "N": N,
        "A": A,
        "codes": codes,
        "scales": scales,
        "mask": mask,
        "bitmap": bitmap_from_mask(mask),
    }


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns: the upper half of the binary32 pattern after
    adding 0x7FFF plus the lowest kept bit."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def w4g_problem(M: int, K: int, N: int, group_size: int = 128, zeros: bool = False,
                act: str = "fp16", seed: int = 0, weights: bool = True,
                activations: bool = True) -> dict:
    """4-bit weights on a general quantization grid: A ~ N(0,1) in the activation
    type (fp16 array, or bf16 bit patterns as uint16); uint4 codes uniform 0..15;
    one scale per (group of ``group_size`` consecutive k, column), uniform in
    [0.005, 0.02] in the activation type; with ``zeros`` a stored zero point per
    (group, column) uniform in 0..15 (asymmetric grids), else the implicit 8."""
    if group_size <= 0 or K % group_size:
        raise ValueError("group_size must divide K")
    if act not in ("fp16", "bf16"):
        raise ValueError("act must be fp16 or bf16")
    tag = (_KIND_W4G, group_size, int(zeros), 0 if act == "fp16" else 1)
    out = {"M": M, "K": K, "N": N, "group_size": group_size, "act": act}
    cvt = (lambda x: x.astype(np.float16)) if act == "fp16" else to_bf16_bits
    if activations:
        out["A"] = cvt(rng_for(seed, *tag, 0, M, K).standard_normal(size=(M, K), dtype=np.float32))
    if weights:
        q = rng_for(seed, *tag, 1, K, N).integers(0, 16, size=(K, N), dtype=np.uint8)
        out["codes"] = pack_nibbles_u32(q)
        G = K // group_size
        out["scales"] = cvt(rng_for(seed, *tag, 2, K, N).uniform(0.005, 0.02, size=(G, N)).astype(np.float32))
        out["zeros"] = (rng_for(seed, *tag, 3, K, N).integers(0, 16, size=(G, N), dtype=np.uint8)
                        if zeros else None)
    return out


def w4a16_sp24_problem(M: int, K: int, N: int, seed: int = 0, weights: bool = True,
                       activations: bool = True) -> dict:
    """2:4 structured-sparse W4A16 workload (the MARLIN abstract's sparse
    extension): fp16 A ~ N(0,1); in every run of 4 consecutive k of a column
    two positions, chosen uniformly among the 6 pairs, keep a uint4 code uniform
    in 0..15, and the other two hold the zero point 8 (weight exactly 0); fp16
    scales uniform in [0.005, 0.02] per (group of 128 k, column). Codes are
    returned dense, in the W4A16 canonical packing."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    out = {"M": M, "K": K, "N": N, "zero": 8}
    if activations:
        out["A"] = _fp16_normal(rng_for(seed, _KIND_SP24, 0, M, K), (M, K))
    if weights:
        r = rng_for(seed, _KIND_SP24, 1, K, N)
        pairs = np.array([(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)])
        choice = r.integers(0, 6, size=(K // 4, N))
        kept = np.zeros((K // 4, 4, N), dtype=bool)
        jj, nn = np.meshgrid(np.arange(K // 4), np.arange(N), indexing="ij")
        kept[jj, pairs[choice, 0], nn] = True
        kept[jj, pairs[choice, 1], nn] = True
        vals = r.integers(0, 16, size=(K // 4, 4, N), dtype=np.uint8)
        q = np.where(kept, vals, np.uint8(8)).reshape(K, N)
        out["codes"] = pack_nibbles_u32(q)
        out["scales"] = _fp16_uniform(rng_for(seed, _KIND_SP24, 2, K, N), 0.005, 0.02, (K // GROUP, N))
    return out


def bitplane_problem(M: int, K: int, N: int, bits: int, seed: int = 0) -> dict:
    """W_b A8 workload on bipolar-INT weights: int8 A uniform in [-127, 127] with
    a per-row fp16 scale uniform in [0.01, 0.03]; b-bit codes U uniform in
    0 .. 2^b - 1 (value 2U - (2^b - 1)); a per-column fp16 scale uniform in
    [0.05, 0.1] / (2^b - 1), so every weight lies within +-0.1."""
    if not 1 <= bits <= 8:
        raise ValueError("bits must be 1..8")
    return {
        "M": M, "K": K, "N": N, "bits": bits,
        "A": rng_for(seed, _KIND_BP, bits, 0, M, K).integers(-127, 128, size=(M, K), dtype=np.int8),
        "a_scale": _fp16_uniform(rng_for(seed, _KIND_BP, bits, 1, M, K), 0.01, 0.03, (M,)),
        "codes": rng_for(seed, _KIND_BP, bits, 2, K, N).integers(0, 2 ** bits, size=(K, N), dtype=np.uint8),
        "chan_scales": (rng_for(seed, _KIND_BP, bits, 3, K, N).uniform(0.05, 0.1, size=(N,))
                        / (2 ** bits - 1)).astype(np.float16),
    }
