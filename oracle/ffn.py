"""fp64 oracle for the blockwise feedforward -- TEST INFRASTRUCTURE ONLY.

The feedforward half of a blockwise transformer layer ("Ring Attention with
Blockwise Transformers for Near-Infinite Context" close-reading notes, §2.2:
the feedforward is computed block by block so that its largest activation is
one block of the 4h-wide intermediate).  The pages name neither the
activation nor the bias terms; the reading taken here is the common
two-layer form y = GELU(x W1^T + b1) W2^T + b2 with the exact GELU
z * Phi(z) and weights stored [out][in].

``ffn_forward`` is that definition on all rows at once; ``ffn_blockwise``
takes the pages' route (row blocks one after another) and exists to pin the
definition against it.
"""
from __future__ import annotations

import math

import numpy as np

_erf = np.vectorize(math.erf, otypes=[np.float64])


def gelu(z: np.ndarray) -> np.ndarray:
    """Exact GELU, z * Phi(z) = z/2 * (1 + erf(z / sqrt(2)))."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def ffn_forward(x, w1, b1, w2, b2) -> np.ndarray:
    """y = GELU(x W1^T + b1) W2^T + b2 in float64 (b1, b2 may be None)."""
    x, w1, w2 = (np.asarray(t, dtype=np.float64) for t in (x, w1, w2))
    h = x @ w1.T
    if b1 is not None:
        h = h + np.asarray(b1, dtype=np.float64)
    y = gelu(h) @ w2.T
    if b2 is not None:
        y = y + np.asarray(b2, dtype=np.float64)
    return y


def ffn_blockwise(x, w1, b1, w2, b2, chunk_rows: int) -> np.ndarray:
    """The same, one block of rows at a time (only a block's intermediate exists at once)."""
    x = np.asarray(x)
    return np.concatenate([ffn_forward(x[r:r + chunk_rows], w1, b1, w2, b2)
                           for r in range(0, x.shape[0], chunk_rows)])
