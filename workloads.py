"""Seeded synthetic inputs and workload shapes for the ring-attention step.

This module is shared by the tests, the oracle-side checks, ``bench.py`` and
``__graft_entry__.smoke()``.  It holds only *data preparation*: workload
shapes and a seeded normal generator with bf16 round-to-nearest-even.  It
contains none of the attention arithmetic, so neither the oracle nor the HIP
path depends on the other through it.

Generation recipe (the same on every machine):

* Every tensor block is drawn from its own numpy PCG64 stream, seeded with
  ``[seed, tensor_id, block_id]`` where ``tensor_id`` is 0 for Q, 1 for K,
  2 for V, 3 for dO.  Block ``j`` of a tensor covers sequence positions
  ``j*block_len .. (j+1)*block_len - 1`` and has shape
  ``[block_len, heads_of_that_tensor, head_dim]`` (token-major).
* Values are iid N(0, 1) drawn in float32, then (for bf16 workloads) rounded
  to bfloat16 with round-to-nearest-even.  Both sides see exactly those
  rounded values; the oracle upcasts them to float64.
* A per-block stream means a rank's share can be generated without drawing
  the whole sequence, which keeps the 512k-token workload cheap to build.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one ring-attention workload (batch 1, token-major layout)."""

    name: str
    seq_len: int          # total sequence length S
    n_blocks: int         # ring size D (number of sequence blocks)
    heads: int            # query heads Hq
    kv_heads: int         # key/value heads Hkv
    head_dim: int         # d
    causal: bool
    ranks: Tuple[int, ...]  # which ranks' shares one pass computes
    dtype: str            # "bf16" or "f32"
    backward: bool        # whether the pass includes the backward step
    seed: int
    description: str = ""
    q_len: int = 0        # decode workloads: new query rows placed after the whole context
    zigzag: bool = False  # block b holds sequence chunks b and 2D-1-b (load-balanced causal layout)

    @property
    def block_len(self) -> int:
        return self.seq_len // self.n_blocks

    @property
    def is_decode(self) -> bool:
        return self.q_len > 0

    def kv_bytes(self) -> int:
        """Bytes of every K and V block (each read once by a decode step)."""
        esize = 2 if self.dtype == "bf16" else 4
        return 2 * self.seq_len * self.kv_heads * self.head_dim * esize

    def visible_pairs(self, rank: int) -> int:
        """Unmasked (query, key) pairs of one rank's share (decode: every query sees every key)."""
        if self.is_decode:
            return self.q_len * self.seq_len
        c = self.block_len
        if not self.causal:
            return c * self.seq_len
        # blocks j < rank are fully visible, block j == rank is the diagonal
        return rank * c * c + c * (c + 1) // 2

    def fwd_flop(self) -> float:
        """Algorithmic forward FLOP: 4 * d * Hq per visible pair (QK^T and PV)."""
        pairs = sum(self.visible_pairs(r) for r in self.ranks)
        return 4.0 * self.head_dim * self.heads * pairs

    def bwd_flop(self) -> float:
        """Algorithmic backward FLOP: 2.5x the forward (five contractions)."""
        return 2.5 * self.fwd_flop()


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_noncausal_f32", 1024, 4, 1, 1, 64, False, (0, 1, 2, 3), "f32", False, 1,
                 "one rank's 256-token Q block against 4 K/V blocks, fp32"),
        Workload("noncausal_64k_h16_d64", 65536, 8, 16, 16, 64, False, (0,), "bf16", False, 2,
                 "hidden 1024 as 16 heads x 64, one rank against 8 blocks of 8192"),
        Workload("causal_128k_h32_d128", 131072, 16, 32, 32, 128, True, tuple(range(16)), "bf16", True, 3,
                 "causal full sequence, every rank's share, 16 blocks of 8192"),
        Workload("causal_128k_h32_d128_zigzag", 131072, 16, 32, 32, 128, True, tuple(range(16)), "bf16", True, 3,
                 "the causal 128k workload in the zig-zag layout (chunks b and 31-b of 4096 per block)",
                 zigzag=True),
        Workload("decode_512k_gqa32x8_q4", 524288, 8, 32, 8, 128, False, (0,), "bf16", False, 6,
                 "decode: 4 new query rows after a 512k-token context held as 8 blocks of 65536, GQA 32/8",
                 q_len=4),
        Workload("causal_512k_gqa32x8_rank7", 524288, 8, 32, 8, 128, True, (7,), "bf16", False, 4,
                 "rank 7's share at 512k tokens, GQA 32/8, 8 blocks of 65536"),
        Workload("bwd_causal_32k_h32_d128", 32768, 4, 32, 32, 128, True, (0, 1, 2, 3), "bf16", True, 5,
                 "backward, causal, every rank's share, 4 blocks of 8192"),
    ]
}


@dataclasses.dataclass(frozen=True)
class FfnWorkload:
    """Blockwise feedforward on one rank's block: y = GELU(x W1^T + b1) W2^T + b2."""

    name: str
    rows: int        # tokens of the block
    hidden: int      # h (= heads x head_dim of the attention it follows)
    ffn: int         # intermediate width (4h)
    chunk_rows: int  # rows per feedforward block
    seed: int
    description: str = ""

    def flop(self) -> float:
        """Two GEMMs of 2 * rows * hidden * ffn flop each."""
        return 4.0 * self.rows * self.hidden * self.ffn


FFN_WORKLOADS: Dict[str, FfnWorkload] = {
    w.name: w
    for w in [
        FfnWorkload("ffn_block8192_h4096_f16384", 8192, 4096, 16384, 2048, 7,
                    "one rank's 8192-token block of the causal 128k workload (h = 32 x 128), 4h intermediate, "
                    "blocks of 2048 rows"),
    ]
}


def gen_ffn(w: FfnWorkload):
    """Seeded ffn inputs: x ~ N(0,1), W1 ~ N(0, 1/hidden), W2 ~ N(0, 1/ffn) (bf16-rounded),
    b1, b2 ~ N(0, 0.1^2) in fp32 -- unit-scale activations at every layer."""
    x = gen_small(w.seed, (w.rows, w.hidden), "bf16", 1.0, 0)
    w1 = gen_small(w.seed, (w.ffn, w.hidden), "bf16", 1.0 / np.sqrt(w.hidden), 1)
    w2 = gen_small(w.seed, (w.hidden, w.ffn), "bf16", 1.0 / np.sqrt(w.ffn), 2)
    b1 = gen_small(w.seed, (w.ffn,), "f32", 0.1, 3)
    b2 = gen_small(w.seed, (w.hidden,), "f32", 0.1, 4)
    return x, w1, b1, w2, b2


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of already-bf16-exact float32 values (for device upload)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def gen_block(seed: int, tensor: str, block: int, block_len: int, heads: int, head_dim: int,
              dtype: str) -> np.ndarray:
    """One seeded block ``[block_len, heads, head_dim]`` as float32 values.

    For ``dtype == "bf16"`` the values are already rounded to bf16.
    """
    rng = np.random.default_rng([seed, TENSOR_IDS[tensor], block])
    x = rng.standard_normal((block_len, heads, head_dim), dtype=np.float32)
    if dtype == "bf16":
        x = bf16_round(x)
    return x


def gen_small(seed: int, shape: Tuple[int, ...], dtype: str = "f32", scale: float = 1.0,
              stream: int = 0) -> np.ndarray:
    """A small seeded N(0, scale^2) tensor for unit tests (float32 values)."""
    rng = np.random.default_rng([seed, 100 + stream])
    x = (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)
    if dtype == "bf16":
        x = bf16_round(x)
    return x


def ranks_q_blocks(w: Workload, ranks: List[int] | None = None) -> Dict[int, np.ndarray]:
    ranks = list(w.ranks if ranks is None else ranks)
    return {r: gen_block(w.seed, "q", r, w.block_len, w.heads, w.head_dim, w.dtype) for r in ranks}
