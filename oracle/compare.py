"""Tolerance rule for fp16 outputs of the quantized GEMMs.

With e = C_gpu (fp16, widened exactly) - C_ref (fp64), a result passes when

    max |e|              <= 2e-3 * sqrt(K) * rms(C_ref)
    ||e||_F / ||C_ref||_F <= 1e-3

The GPU rounds each dequantized weight or each per-group partial product once,
accumulates in fp32 and rounds the output to fp16 once; the expected relative
Frobenius error of that chain is about 3e-4, so the bound leaves roughly a 3x
margin. Integer results (W4A8 accumulators, repacked bytes) are compared for
equality elsewhere, not with this rule.
"""

from __future__ import annotations

import numpy as np


def fp16_ulp_distance(a16: np.ndarray, b16: np.ndarray) -> np.ndarray:
    """Distance in units of fp16 representable values (monotone integer map)."""
    def key(x):
        u = np.asarray(x, dtype=np.float16).view(np.uint16).astype(np.int64)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + u)
    return np.abs(key(a16) - key(b16))


def check_fp16(C_gpu: np.ndarray, C_ref: np.ndarray, K: int,
               max_coef: float = 2e-3, fro_bound: float = 1e-3) -> dict:
    """Apply the output tolerance rule; returns the measured figures and ``ok``."""
    g = np.asarray(C_gpu).astype(np.float64)
    r = np.asarray(C_ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    e = g - r
    finite = bool(np.all(np.isfinite(g)))
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    max_err = float(np.max(np.abs(e))) if e.size else 0.0
    ref_norm = float(np.linalg.norm(r))
    rel_fro = float(np.linalg.norm(e) / ref_norm) if ref_norm > 0 else float(np.linalg.norm(e))
    bound = max_coef * np.sqrt(K) * rms
    ulp = fp16_ulp_distance(np.asarray(C_gpu, dtype=np.float16), r.astype(np.float16))
    return {
        "ok": finite and max_err <= bound and rel_fro <= fro_bound,
        "finite": finite,
        "max_err": max_err,
        "bound": float(bound),
        "rel_fro": rel_fro,
        "rms_ref": rms,
        "max_ulp": int(ulp.max()) if ulp.size else 0,
    }


def check_bf16(C_gpu_bits: np.ndarray, C_ref: np.ndarray, K: int,
               max_coef: float = 2e-3, fro_bound: float = 4e-3) -> dict:
    """Tolerance rule for bf16 outputs (given as uint16 bit patterns).

    bf16 keeps 8 significant bits, so its unit roundoff is u = 2**-8 against
    2**-11 for fp16; the single output rounding alone gives a relative
    Frobenius error of about u / sqrt(12) / 1.5 * 2 ~ 1.5e-3 for values spread
    over a binade. The rule keeps the fp16 rule's accumulation allowance and
    adds the rounding of the largest output to the max-error bound, and bounds
    the relative Frobenius error by 4e-3 (a margin of about 2.7x):

        max |e|               <= 2e-3 * sqrt(K) * rms(C_ref) + u * max |C_ref|
        ||e||_F / ||C_ref||_F <= 4e-3
    """
    from .ref import bf16_to_f64
    g = bf16_to_f64(C_gpu_bits)
    r = np.asarray(C_ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    e = g - r
    finite = bool(np.all(np.isfinite(g)))
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    max_err = float(np.max(np.abs(e))) if e.size else 0.0
    ref_norm = float(np.linalg.norm(r))
    rel_fro = float(np.linalg.norm(e) / ref_norm) if ref_norm > 0 else float(np.linalg.norm(e))
    bound = max_coef * np.sqrt(K) * rms + 2.0 ** -8 * (float(np.max(np.abs(r))) if r.size else 0.0)
    return {
        "ok": finite and max_err <= bound and rel_fro <= fro_bound,
        "finite": finite,
        "max_err": max_err,
        "bound": float(bound),
        "rel_fro": rel_fro,
        "rms_ref": rms,
    }
