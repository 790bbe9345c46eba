"""GPU parity: long-context decode (few query rows against every block) vs the fp64 oracle.

Small shapes cover ragged blocks, grouped heads up to the 32-row limit,
queries whose causal cut falls inside a block and rows with no visible key;
a composition test folds per-block decode results with ring_attn_merge (the
ring's route); the full-size case is the 512k-token GQA decode workload that
bench.py times.
"""
import numpy as np
import pytest
import torch

import long_context_exact_ring_amd as ra
import oracle
from tests.gpu_util import compare, dev, log, require_gpu
from workloads import WORKLOADS, bf16_round, gen_block, gen_small

pytestmark = pytest.mark.gpu

# (head_dim, heads, kv_heads, block_len, n_blocks, q_len, q_pos0 ("end" = after the context))
CASES = [
    (128, 32, 8, 1000, 4, 1, "end"),   # GQA 4, ragged blocks, one new token
    (128, 8, 8, 512, 3, 4, "end"),     # MHA, four new tokens
    (64, 4, 1, 700, 2, 8, 650),        # group 4 x 8 rows = 32; causal cut inside block 0
    (128, 2, 2, 33, 5, 3, 0),          # first positions: row 0 sees one key, later rows a few
    (128, 16, 1, 256, 1, 2, "end"),    # group 16 x 2 rows = 32, a ring of one
    (64, 2, 2, 5000, 2, 1, 7777),      # long blocks, cut inside block 1
    (128, 8, 2, 64, 64, 2, 3000),      # the most blocks one call takes (64), cut inside block 46
    (128, 32, 8, 700, 3, 20, "end"),   # group 4 x 20 rows: passes of 8, 8 and 4 rows
    (64, 8, 1, 300, 2, 9, 250),        # group 8 x 9 rows: passes of 4, 4, 1; causal cut in block 0
]


def _case_inputs(seed, d, hq, hkv, c, D, q_len):
    q = bf16_round(gen_small(seed, (q_len, hq, d), "f32", 1.0, 0))
    k = [bf16_round(gen_small(seed, (c, hkv, d), "f32", 1.0, 10 + j)) for j in range(D)]
    v = [bf16_round(gen_small(seed, (c, hkv, d), "f32", 1.0, 40 + j)) for j in range(D)]
    return q, k, v


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_vs_oracle(case):
    require_gpu()
    d, hq, hkv, c, D, q_len, pos = case
    log(f"decode case {case}")
    q, k, v = _case_inputs(71, d, hq, hkv, c, D, q_len)
    q_pos0 = D * c if pos == "end" else pos
    o, l = ra.decode(dev(q, "bf16"), [dev(x, "bf16") for x in k], [dev(x, "bf16") for x in v], q_pos0=q_pos0)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_forward(q.astype(np.float64), [x.astype(np.float64) for x in k],
                                         [x.astype(np.float64) for x in v], q_pos0)
    compare("out", o, o_ref, "bf16")
    compare("lse", l, l_ref, "bf16")


def test_per_block_decode_merged_by_ring_attn_merge():
    """The ring's route on the device: decode against each block alone (each host's partial,
    every key visible), fold the partials with ring_attn_merge, compare with one call."""
    require_gpu()
    d, hq, hkv, c, D, q_len = 128, 8, 2, 768, 4, 4
    q, k, v = _case_inputs(79, d, hq, hkv, c, D, q_len)
    qd = dev(q, "bf16")
    kd = [dev(x, "bf16") for x in k]
    vd = [dev(x, "bf16") for x in v]
    big = 10 * D * c
    o_all, l_all = ra.decode(qd, kd, vd, q_pos0=big)
    o_acc, l_acc = ra.decode(qd, kd[:1], vd[:1], q_pos0=big)
    for j in range(1, D):
        o_j, l_j = ra.decode(qd, kd[j:j + 1], vd[j:j + 1], q_pos0=big)
        ra.merge(o_acc, l_acc, o_j, l_j, out=o_acc, lse=l_acc)  # in place
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_forward(q.astype(np.float64), [x.astype(np.float64) for x in k],
                                         [x.astype(np.float64) for x in v], big)
    compare("merged out", o_acc, o_ref, "bf16")
    compare("merged lse", l_acc, l_ref, "bf16")
    compare("single-call out", o_all, o_ref, "bf16")
    assert torch.allclose(o_acc, o_all, atol=2e-5, rtol=0)


def test_full_decode_512k_gqa():
    require_gpu()
    w = WORKLOADS["decode_512k_gqa32x8_q4"]
    log(f"workload {w.name}")
    c = w.block_len
    k = [gen_block(w.seed, "k", j, c, w.kv_heads, w.head_dim, w.dtype) for j in range(w.n_blocks)]
    v = [gen_block(w.seed, "v", j, c, w.kv_heads, w.head_dim, w.dtype) for j in range(w.n_blocks)]
    q = gen_block(w.seed, "q", 0, w.q_len, w.heads, w.head_dim, w.dtype)
    o, l = ra.decode(dev(q, "bf16"), [dev(x, "bf16") for x in k], [dev(x, "bf16") for x in v], q_pos0=w.seq_len)
    torch.cuda.synchronize()
    heads = [0, 5, 17, 31]
    kvh = sorted({h // (w.heads // w.kv_heads) for h in heads})
    qs = q[:, heads]
    ks = [x[:, [h // (w.heads // w.kv_heads) for h in heads]] for x in k]
    vs = [x[:, [h // (w.heads // w.kv_heads) for h in heads]] for x in v]
    # one K/V column per sampled head (repeat-interleaved), so the oracle runs as MHA on 4 heads
    o_ref, l_ref = oracle.decode_forward(qs.astype(np.float64), [x.astype(np.float64) for x in ks],
                                         [x.astype(np.float64) for x in vs], w.seq_len)
    log(f"  heads {heads} (K/V heads {kvh})")
    compare("out", o[:, heads], o_ref, "bf16")
    compare("lse", l[heads], l_ref, "bf16")
