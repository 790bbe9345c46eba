"""fp64 oracle for long-context decode -- TEST INFRASTRUCTURE ONLY.

Decode is the inference use of the method ("Ring Attention with Blockwise
Transformers for Near-Infinite Context" close-reading notes, §3.1 and §3.5:
each host holds one block of the context; a query block meets every block and
the per-block statistics are combined by rescaling): a few new query rows, at
global positions q_pos0 + i, attend to every key of the context, block j's
key t sitting at position j * block_len + t, with a key visible iff its
position is <= the query's.

``decode_forward`` is that definition written out (dense fp64 attention over
the concatenated blocks with explicit positions).  ``decode_by_partials``
takes the ring's route instead -- one normalised partial per host's block,
folded together with the log-sum-exp merge -- and exists to pin the
definition and the merge against each other.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .dense import attention_fwd
from .ring import merge_partials


def _positions(q_len: int, q_pos0: int, block_len: int, n_blocks: int):
    q_pos = q_pos0 + np.arange(q_len, dtype=np.int64)
    k_pos = np.arange(n_blocks * block_len, dtype=np.int64)
    return q_pos, k_pos


def decode_forward(q: np.ndarray, k_blocks: Sequence[np.ndarray], v_blocks: Sequence[np.ndarray],
                   q_pos0: int) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention of ``q [q_len, Hq, d]`` over all blocks (each ``[c, Hkv, d]``).

    Returns ``out [q_len, Hq, d]`` and ``lse [Hq, q_len]`` in float64; a row
    with no visible key has out 0 and lse -inf.
    """
    c = k_blocks[0].shape[0]
    q_pos, k_pos = _positions(q.shape[0], q_pos0, c, len(k_blocks))
    k = np.concatenate([np.asarray(b) for b in k_blocks])
    v = np.concatenate([np.asarray(b) for b in v_blocks])
    return attention_fwd(q, k, v, causal=True, q_pos=q_pos, k_pos=k_pos)


def decode_by_partials(q: np.ndarray, k_blocks: Sequence[np.ndarray], v_blocks: Sequence[np.ndarray],
                       q_pos0: int) -> Tuple[np.ndarray, np.ndarray]:
    """The ring's route: one partial per block (its own key positions), merged in block order."""
    c = k_blocks[0].shape[0]
    q_pos = q_pos0 + np.arange(q.shape[0], dtype=np.int64)
    out = lse = None
    for j, (kb, vb) in enumerate(zip(k_blocks, v_blocks)):
        k_pos = np.arange(j * c, (j + 1) * c, dtype=np.int64)
        o_j, l_j = attention_fwd(q, kb, vb, causal=True, q_pos=q_pos, k_pos=k_pos)
        out, lse = (o_j, l_j) if out is None else merge_partials(out, lse, o_j, l_j)
    return out, lse
