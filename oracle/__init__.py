"""CPU oracle for the quantized-weight GEMM (test infrastructure only).

This package is the plain, slow, obviously correct definition of what the GPU
library computes. It is used by ``tests/``, by ``__graft_entry__.smoke()`` and by
the ``cpu_baseline`` leg of ``bench.py`` -- never by the library itself, which
fails loudly if its HIP build is missing.

* ``oracle.ref``     -- dequantize-then-matmul in fp64 (and exact integers for
                        W4A8), following the MARLIN abstract's problem statement
                        (fp16 activations times 4-bit weights, batched), the
                        OdysseyLLM abstract (W4A8) and the 2-bit page's mixed
                        2/4-bit groups; the 4-bit GEMM on a general grid
                        (group length 64 .. K, stored zero points, fp16 or bf16
                        activations); the 2:4 structure check of sparse
                        W4A16 (whose GEMM is the W4A16 definition on the
                        dense codes); the bit-plane W_b A8 GEMM on
                        bipolar-INT weights (b = 1..8); plus the per-token
                        dynamic int8
                        activation quantization that feeds W4A8.
* ``oracle.layout``  -- an independent implementation of the repacked weight
                        blob byte layout, for byte-exact checks of the GPU repack.
* ``oracle.compare`` -- the fp16 and bf16 output tolerance rules.

Every function here is pinned by ``tests/test_oracle_*.py`` against values that
do not come from the oracle itself (exact rational brute force, closed forms,
hand-derived golden files, invariants). Nothing here shares code with the HIP
library; inputs come from the separate ``synth`` module.
"""

from . import compare, layout, ref  # noqa: F401
