"""Seeded synthetic inputs for the quantized-weight GEMM workloads.

This module only draws random tensors and packs them into the canonical input
formats that both the CPU oracle and the GPU library read. It holds none of the
GEMM's arithmetic (no dequantization, no products, no reductions over K).
"""

from .gen import (  # noqa: F401
    GROUP,
    rng_for,
    pack_nibbles_u32,
    w4a16_problem,
    w4a8_problem,
    w2w4_problem,
    select_4bit_groups,
    bitmap_from_mask,
)
