"""GPU parity over a seeded sweep of random small shapes (forward and backward, every rank).

Each case draws head_dim, the head grouping, a ragged block length, the ring size,
the mask and the layout (contiguous or zig-zag) from a fixed seed, runs every
rank's forward and backward through the library, and compares out, lse, dQ, dK
and dV with the fp64 oracle over the whole sequence (dK/dV summed over the ranks).
The shapes stay small, so the oracle covers every element.
"""
import numpy as np
import pytest
import torch

import long_context_exact_ring_amd as ra
import oracle
from tests.gpu_util import compare, dev, log, require_gpu
from workloads import gen_small

pytestmark = pytest.mark.gpu


def _cases(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 3]))
        group = int(rng.choice([1, 2, 3, 4, 8]))
        zigzag = bool(rng.random() < 0.3)
        c = int(rng.integers(1, 161))
        if zigzag:
            c += c % 2  # the zig-zag layout halves every block
        D = int(rng.integers(1, 6))
        causal = True if zigzag else bool(rng.random() < 0.6)
        out.append((i, d, hkv * group, hkv, c, D, causal, zigzag))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "-".join(map(str, c)))
def test_random_shape_fwd_bwd_all_ranks(case):
    require_gpu()
    i, d, hq, hkv, c, D, causal, zigzag = case
    log(f"sweep case {case}")
    S = c * D
    q = gen_small(300 + i, (S, hq, d), "bf16", 1.0, 0)
    k = gen_small(300 + i, (S, hkv, d), "bf16", 1.0, 1)
    v = gen_small(300 + i, (S, hkv, d), "bf16", 1.0, 2)
    do = gen_small(300 + i, (S, hq, d), "bf16", 1.0, 3)
    # rows of block b in sequence order (zig-zag: chunk b, then chunk 2D-1-b)
    pos = [oracle.zigzag_positions(b, D, c) if zigzag else np.arange(b * c, (b + 1) * c) for b in range(D)]
    kb = [dev(k[p], "bf16") for p in pos]
    vb = [dev(v[p], "bf16") for p in pos]
    dkb = [torch.zeros((c, hkv, d), dtype=torch.float32, device="cuda") for _ in range(D)]
    dvb = [torch.zeros((c, hkv, d), dtype=torch.float32, device="cuda") for _ in range(D)]
    outs, lses, dqs = [], [], []
    for r in range(D):
        qd, dod = dev(q[pos[r]], "bf16"), dev(do[pos[r]], "bf16")
        o, l = ra.fwd(qd, kb, vb, causal=causal, rank=r, zigzag=zigzag)
        g, _, _ = ra.bwd(qd, kb, vb, o, dod, l, causal=causal, rank=r, dk_blocks=dkb, dv_blocks=dvb, zigzag=zigzag)
        outs.append(o), lses.append(l), dqs.append(g)
    torch.cuda.synchronize()
    order = np.argsort(np.concatenate(pos))  # back to sequence order
    dq_ref, dk_ref, dv_ref, o_ref, l_ref = oracle.attention_bwd(q, k, v, do, causal=causal)
    compare("out", torch.cat(outs, 0)[order], o_ref, "bf16")
    compare("lse", torch.cat(lses, 1)[:, order], l_ref, "bf16")
    compare("dq", torch.cat(dqs, 0)[order], dq_ref, "bf16")
    compare("dk", torch.cat(dkb, 0)[order], dk_ref, "bf16")
    compare("dv", torch.cat(dvb, 0)[order], dv_ref, "bf16")
