"""GPU parity: the zig-zag (load-balanced causal) layout, forward and backward.

The whole sequence is drawn once; block b of the ring is chunk b followed by
chunk 2D-1-b.  Every rank runs the zig-zag forward and backward; results are
put back in sequence order and compared with dense fp64 causal attention.
The per-rank launch counts show the balance: every rank runs the same
number of steps.  Without a mask the layout is only a permutation of the
sequence, and the results equal plain attention.

The shapes include large gradients: under the causal mask key 0 collects
weight from every row of every grouped head, so a 4-way group over 600 rows
puts |dV| near 6.5, and with one token per chunk and a shared K/V head dQ has
so few terms that each rounded dS counts.  Rounding P and dS to bf16 for the
matrix core would cost 1.0e-2 to 1.1e-2 on those shapes (an fp64 emulation
of that rounding); the backward rounds them to half precision instead.
"""
import numpy as np
import pytest
import torch

import long_context_exact_ring_amd as ra
import oracle
from tests.gpu_util import compare, dev, log, require_gpu
from workloads import gen_small

pytestmark = pytest.mark.gpu

# (head_dim, heads, kv_heads, block_len, n_blocks)
CASES = [
    (128, 4, 4, 512, 4),
    (128, 4, 2, 200, 3),   # chunks of 100 tokens: ragged tiles, GQA 2
    (64, 2, 2, 66, 5),     # chunks of 33 tokens
    (128, 2, 2, 2, 4),     # one token per chunk
    (64, 6, 2, 64, 4),     # group 3 (not a divisor of the wave count), chunks of 32
    (128, 4, 1, 200, 3),   # GQA 4 over 600 tokens: |dV| 6.5 on key 0
    (128, 2, 1, 2, 4),     # one token per chunk, shared K/V head: few dQ terms
    (128, 6, 2, 128, 4),   # group 3, head_dim 128, chunks of 64: |dV| 7.3
]


def _seq(seed, S, hq, hkv, d):
    q = gen_small(seed, (S, hq, d), "bf16", 1.0, 0)
    k = gen_small(seed, (S, hkv, d), "bf16", 1.0, 1)
    v = gen_small(seed, (S, hkv, d), "bf16", 1.0, 2)
    do = gen_small(seed, (S, hq, d), "bf16", 1.0, 3)
    return q, k, v, do


# without a mask every query chunk sees both key chunks of every block, so each round runs as
# whole-block sub-problems on both sides
NONCAUSAL_CASES = [(128, 4, 2, 200, 3, False), (64, 2, 2, 66, 4, False)]


@pytest.mark.parametrize("case", [c + (True,) for c in CASES] + NONCAUSAL_CASES,
                         ids=lambda c: "-".join(map(str, c)))
def test_zigzag_fwd_bwd_all_ranks(case):
    require_gpu()
    d, hq, hkv, c, D, causal = case
    log(f"zigzag case {case}")
    S = c * D
    q, k, v, do = _seq(83, S, hq, hkv, d)
    pos = [oracle.zigzag_positions(b, D, c) for b in range(D)]
    kb = [dev(k[p], "bf16") for p in pos]
    vb = [dev(v[p], "bf16") for p in pos]
    dkb = [torch.zeros((c, hkv, d), dtype=torch.float32, device="cuda") for _ in range(D)]
    dvb = [torch.zeros((c, hkv, d), dtype=torch.float32, device="cuda") for _ in range(D)]
    out = np.zeros((S, hq, d))
    lse = np.zeros((hq, S))
    dq = np.zeros((S, hq, d))
    for r in range(D):
        qd, dod = dev(q[pos[r]], "bf16"), dev(do[pos[r]], "bf16")
        o, l = ra.fwd(qd, kb, vb, causal=causal, rank=r, zigzag=True)
        g, _, _ = ra.bwd(qd, kb, vb, o, dod, l, causal=causal, rank=r, dk_blocks=dkb, dv_blocks=dvb, zigzag=True)
        torch.cuda.synchronize()
        out[pos[r]] = o.cpu().numpy()
        lse[:, pos[r]] = l.cpu().numpy()
        dq[pos[r]] = g.cpu().numpy()
    dk = np.zeros((S, hkv, d))
    dv = np.zeros((S, hkv, d))
    for b in range(D):
        dk[pos[b]] = dkb[b].cpu().numpy()
        dv[pos[b]] = dvb[b].cpu().numpy()
    dq_ref, dk_ref, dv_ref, o_ref, l_ref = oracle.attention_bwd(q, k, v, do, causal=causal)
    compare("out", out, o_ref, "bf16")
    compare("lse", lse, l_ref, "bf16")
    compare("dq", dq, dq_ref, "bf16")
    compare("dk", dk, dk_ref, "bf16")
    compare("dv", dv, dv_ref, "bf16")


def test_zigzag_every_rank_runs_the_same_steps():
    require_gpu()
    d, hq, hkv, c, D = 128, 2, 2, 256, 4
    q, k, v, _ = _seq(89, c * D, hq, hkv, d)
    pos = [oracle.zigzag_positions(b, D, c) for b in range(D)]
    kb = [dev(k[p], "bf16") for p in pos]
    vb = [dev(v[p], "bf16") for p in pos]
    counts = []
    for r in range(D):
        ra.ring_attn_profile_enable(True)
        try:
            ra.ring_attn_profile_read()
            ra.fwd(dev(q[pos[r]], "bf16"), kb, vb, causal=True, rank=r, zigzag=True)
            torch.cuda.synchronize()
            recs, _, _ = ra.ring_attn_profile_read()
        finally:
            ra.ring_attn_profile_enable(False)
        counts.append(recs["fwd_step"][1])
    log(f"  zig-zag forward launches per rank: {counts}")
    # Chunk pairs (query chunk qc, key chunk kc) that attend: kc <= qc.  Block b holds chunks
    # b and 2D-1-b.  Every rank has 2D+1 of them (3 in its diagonal round, 2 in every other).
    # A query half that sees both key halves off the diagonal runs them as one sub-problem;
    # sub-problems of the two query halves share a launch when their key spans match.
    zz = lambda b, half: b if half == 0 else 2 * D - 1 - b
    pairs, launches = [], []
    for r in range(D):
        n_launch = 0
        for j in range(D):
            subs = []
            for u in (0, 1):
                live = [zz(j, v) <= zz(r, u) for v in (0, 1)]
                diag = [zz(j, v) == zz(r, u) for v in (0, 1)]
                pairs.append((r, sum(live)))
                subs.append([2] if all(live) and not any(diag) else [1 for v in (0, 1) if live[v]])
            # greedy pairing in order: the i-th sub-problems of the two halves pair if both exist
            # and span the same number of key halves
            a, b = subs
            i = k = 0
            while i < len(a) or k < len(b):
                if i < len(a) and k < len(b) and a[i] == b[k]:
                    i, k = i + 1, k + 1
                elif i < len(a):
                    i += 1
                else:
                    k += 1
                n_launch += 1
        launches.append(n_launch)
    assert [sum(n for rr, n in pairs if rr == r) for r in range(D)] == [2 * D + 1] * D
    assert launches == [D + 1] * D  # one launch per round, two in the diagonal round
    assert counts == launches


def test_zigzag_rejects_odd_block_len():
    require_gpu()
    d, h, c, D = 128, 2, 33, 2
    x = dev(gen_small(1, (c, h, d), "bf16", 1.0, 0), "bf16")
    with pytest.raises(ra.RingAttnError, match="even"):
        ra.fwd(x, [x, x], [x, x], causal=True, rank=0, zigzag=True)
