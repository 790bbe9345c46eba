"""Plain fp64 CPU oracle for the ring-attention step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The HIP library never calls it, and it shares
no code with the HIP path (the seeded input generator in ``workloads.py``
holds no attention arithmetic and is the only thing both sides use).

Sources (cited by page title and section):

* "精读笔记 · Ring Attention with Blockwise Transformers for Near-Infinite
  Context" (llm-papers-study close-reading notes), §2.1 (blockwise attention
  without materialising the score matrix), §3.1 (a query block may meet the
  key/value blocks in any order as long as per-block statistics are combined
  by rescaling), §3.2 (ring of hosts: each forwards the block it is using and
  receives the previous host's), §3.5 (Algorithm 1 and its 4-GPU walk-through).
* "Ring Attention 与序列并行" (wj-mcat agent handbook), "Ring Attention 核心机制"
  (online-softmax accumulation over the rotated blocks).
* "什么是环形注意力（Ring Attention）？" (aiboss88 wiki), "边界与常见误解": the
  method is exact attention, not an approximation.

Because the method is exact, the reference for its output is the plain
definition softmax(Q K^T / sqrt(d)) V, written out in fp64 (``dense``).  The
blockwise/online form (``ring``) follows the pages' steps and exists to pin
the definition against the pages' invariants.
"""
from .dense import (attention_fwd, attention_bwd, attention_bwd_keys, brute_force_fwd, positions_for_block,
                    sampled_rows_fwd)
from .ring import (ring_steps, simulate_ring, ring_forward, online_block_forward,
                   merge_partials, merge_partials_scalar, zigzag_positions, visible_pairs_per_rank)
from .decode import decode_forward, decode_by_partials
from .ffn import ffn_blockwise, ffn_forward, gelu

__all__ = [
    "attention_fwd", "attention_bwd", "attention_bwd_keys", "brute_force_fwd", "positions_for_block",
    "sampled_rows_fwd", "ring_steps", "simulate_ring", "ring_forward",
    "online_block_forward", "merge_partials", "merge_partials_scalar",
    "decode_forward", "decode_by_partials", "zigzag_positions", "visible_pairs_per_rank",
    "ffn_forward", "ffn_blockwise", "gelu",
]
