"""The ring schedule and the blockwise online-softmax form of attention, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

These functions follow the pages' description of the method step by step and
are used to pin the dense oracle against the pages' invariants; they are not
a second implementation of the HIP path.

* Ring schedule -- close-reading notes on "Ring Attention with Blockwise
  Transformers for Near-Infinite Context", §3.2 and the §3.5 walk-through:
  hosts form a ring; in every round a host computes with the K/V block it
  currently holds, forwards that block to the next host and receives the
  previous host's.  In round 0 each host uses its own block, so host r holds
  block (r - s) mod D in round s.  With a causal mask (not on the pages; taken
  from the workload definition) rounds whose block lies wholly in the future
  (j > r) contribute nothing and are dropped.
* Online accumulation -- same notes, §3.1, and "Ring Attention 与序列并行"
  (wj-mcat handbook), "Ring Attention 核心机制": a query block can absorb the
  K/V blocks in any order provided the running per-row statistics (row max m
  and row sum l) rescale what was accumulated so far.
* Merging two finished partials -- the same statistic in log form: a partial
  is (O_a, lse_a) with O_a normalised; combining two gives
  lse = log(e^lse_a + e^lse_b) and O = e^(lse_a-lse) O_a + e^(lse_b-lse) O_b.
  (One news page says the partial outputs are simply summed; that is only true
  of unnormalised numerators, so the rescaled form above is the reading taken.)
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


def ring_steps(rank: int, n_blocks: int, causal: bool) -> List[int]:
    """Sequence-block ids a rank computes with, in ring order (round s -> (rank - s) mod D)."""
    steps = []
    for s in range(n_blocks):
        j = (rank - s) % n_blocks
        if causal and j > rank:
            continue
        steps.append(j)
    return steps


def simulate_ring(n_hosts: int) -> List[List[int]]:
    """Pass block ids around a ring of hosts; returns ``used[round][host]``.

    Each host starts with its own block; after computing in a round it sends
    the block it used to host (r + 1) mod n and takes what host r - 1 sent.
    """
    holding = list(range(n_hosts))
    used = []
    for _ in range(n_hosts):
        used.append(list(holding))
        nxt = [0] * n_hosts
        for r in range(n_hosts):
            nxt[(r + 1) % n_hosts] = holding[r]
        holding = nxt
    return used


def online_block_forward(state, q: np.ndarray, k_blk: np.ndarray, v_blk: np.ndarray, *,
                         causal: bool, q_pos: np.ndarray, k_pos: np.ndarray):
    """Fold one K/V block into the running (m, l, acc) of every (head, query row).

    ``state`` is ``(m [Hq, n], l [Hq, n], acc [n, Hq, d])`` or ``None`` to start.
    """
    n, hq, d = q.shape
    hkv = k_blk.shape[1]
    group = hq // hkv
    scale = 1.0 / math.sqrt(d)
    if state is None:
        m = np.full((hq, n), -np.inf)
        l = np.zeros((hq, n))
        acc = np.zeros((n, hq, d))
    else:
        m, l, acc = (x.copy() for x in state)
    for h in range(hq):
        g = h // group
        s = (np.asarray(q[:, h, :], np.float64) @ np.asarray(k_blk[:, g, :], np.float64).T) * scale
        if causal:
            s = np.where(k_pos[None, :] <= q_pos[:, None], s, -np.inf)
        m_new = np.maximum(m[h], s.max(axis=1))
        ok = np.isfinite(m_new)
        m_ref = np.where(ok, m_new, 0.0)
        alpha = np.where(np.isfinite(m[h]), np.exp(m[h] - m_ref), 0.0)
        p = np.where(ok[:, None], np.exp(s - m_ref[:, None]), 0.0)
        l[h] = alpha * l[h] + p.sum(axis=1)
        acc[:, h, :] = alpha[:, None] * acc[:, h, :] + p @ np.asarray(v_blk[:, g, :], np.float64)
        m[h] = m_new
    return m, l, acc


def finish_online(state) -> Tuple[np.ndarray, np.ndarray]:
    """Normalise a running state into (out [n, Hq, d], lse [Hq, n]); empty rows -> (0, -inf)."""
    m, l, acc = state
    ok = l > 0
    lsafe = np.where(ok, l, 1.0)
    out = np.where(ok.T[:, :, None], acc / lsafe.T[:, :, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(ok, m + np.log(lsafe), -np.inf)
    return out, lse


def ring_forward(q: np.ndarray, k_blocks: Sequence[np.ndarray], v_blocks: Sequence[np.ndarray],
                 order: Sequence[int], *, causal: bool, q_pos: np.ndarray, block_len: int):
    """One rank's share computed block by block in the given order with online softmax."""
    state = None
    for j in order:
        k_pos = np.arange(j * block_len, (j + 1) * block_len, dtype=np.int64)
        state = online_block_forward(state, q, k_blocks[j], v_blocks[j], causal=causal,
                                     q_pos=q_pos, k_pos=k_pos)
    return finish_online(state)


def merge_partials(out_a: np.ndarray, lse_a: np.ndarray, out_b: np.ndarray, lse_b: np.ndarray):
    """Combine two normalised partials ``(out [n, Hq, d], lse [Hq, n])`` over disjoint key sets."""
    lse = np.logaddexp(lse_a, lse_b)
    ok = np.isfinite(lse)
    ref = np.where(ok, lse, 0.0)
    wa = np.where(ok & np.isfinite(lse_a), np.exp(lse_a - ref), 0.0)
    wb = np.where(ok & np.isfinite(lse_b), np.exp(lse_b - ref), 0.0)
    out = wa.T[:, :, None] * out_a + wb.T[:, :, None] * out_b
    return out, lse


def merge_partials_scalar(o_a: float, l_a: float, o_b: float, l_b: float) -> Tuple[float, float]:
    """Scalar form of the merge (for hand-checkable tests)."""
    if l_a == -math.inf and l_b == -math.inf:
        return 0.0, -math.inf
    mx = max(l_a, l_b)
    lse = mx + math.log(math.exp(l_a - mx) + math.exp(l_b - mx))
    return math.exp(l_a - lse) * o_a + math.exp(l_b - lse) * o_b, lse


def zigzag_positions(block: int, n_blocks: int, block_len: int) -> np.ndarray:
    """Global positions of the rows of block ``block`` in the zig-zag layout.

    The sequence is cut into 2D chunks of block_len/2 tokens; block b holds
    chunk b then chunk 2D-1-b, so that under a causal mask every rank pairs an
    early and a late chunk (the load-balancing reading of "Ring Attention
    with Blockwise Transformers for Near-Infinite Context" close-reading
    notes, §3.5: the per-host work of the plain causal split is uneven).
    """
    h = block_len // 2
    first = np.arange(block * h, (block + 1) * h, dtype=np.int64)
    late = 2 * n_blocks - 1 - block
    second = np.arange(late * h, (late + 1) * h, dtype=np.int64)
    return np.concatenate([first, second])


def visible_pairs_per_rank(n_blocks: int, block_len: int, zigzag: bool) -> List[int]:
    """Causal (query, key) pairs each rank's queries see over the whole ring (brute count)."""
    pos = [zigzag_positions(b, n_blocks, block_len) if zigzag else
           np.arange(b * block_len, (b + 1) * block_len, dtype=np.int64) for b in range(n_blocks)]
    allk = np.sort(np.concatenate(pos))
    return [int(np.sum(np.searchsorted(allk, p, side="right"))) for p in pos]

