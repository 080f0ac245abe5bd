"""Output columns at which full-size layers are compared with the oracle.

One column from every 16-column block (the blob's chunk width and the narrowest
tile of any kernel), at an offset inside the block that varies from block to
block, plus the first and last columns of the layer. Every column tile, every
column wave and every lane position of a 16-column block therefore appears in
the comparison.
"""

import numpy as np


def block_cols(N: int, seed: int, per_block: int = 1) -> np.ndarray:
    rng = np.random.default_rng(seed)
    nb = N // 16
    offs = np.stack([rng.permutation(16)[:per_block] for _ in range(nb)])
    cols = (np.arange(nb)[:, None] * 16 + offs).ravel()
    return np.unique(np.concatenate([cols, [0, 15, N - 16, N - 1]]))
