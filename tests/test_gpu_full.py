"""GPU parity at the workloads' full sizes, in the launch configuration bench.py uses.

Every workload's GPU result is computed in full; the fp64 oracle is evaluated
on sampled query rows and heads (each sampled output is exact attention over
all of that row's visible keys), and for the backward on whole heads.
"""
import numpy as np
import pytest
import torch

import long_context_exact_ring_amd as ra
import oracle
from tests.gpu_util import compare, log, require_gpu
from workloads import WORKLOADS, bf16_bits, gen_block

pytestmark = pytest.mark.gpu


def up(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(bf16_bits(x).view("int16")).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def kv_blocks(w, nblk=None):
    nblk = w.n_blocks if nblk is None else nblk
    k = [gen_block(w.seed, "k", j, w.block_len, w.kv_heads, w.head_dim, w.dtype) for j in range(nblk)]
    v = [gen_block(w.seed, "v", j, w.block_len, w.kv_heads, w.head_dim, w.dtype) for j in range(nblk)]
    return k, v


def sample_rows(c, n_random=12, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, c // 2, c - 2, c - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, c, n_random)]).astype(np.int64))


def check_fwd_sampled(w, rank, out, lse, kblk, vblk, heads):
    c = w.block_len
    group = w.heads // w.kv_heads
    kvh = [h // group for h in heads]
    q = gen_block(w.seed, "q", rank, c, w.heads, w.head_dim, w.dtype)
    rows = sample_rows(c, seed=rank)
    nvis = rank + 1 if w.causal else w.n_blocks
    k = np.concatenate([kb[:, kvh] for kb in kblk[:nvis]])
    v = np.concatenate([vb[:, kvh] for vb in vblk[:nvis]])
    o_ref, l_ref = oracle.sampled_rows_fwd(q[rows][:, heads], rank * c + rows, k, v, causal=w.causal)
    o = out[torch.from_numpy(rows).cuda()][:, heads]
    l = lse[heads][:, torch.from_numpy(rows).cuda()]
    compare(f"{w.name} rank {rank} out", o, o_ref, w.dtype)
    compare(f"{w.name} rank {rank} lse", l, l_ref, w.dtype)


def test_full_noncausal_64k_h16_d64():
    require_gpu()
    w = WORKLOADS["noncausal_64k_h16_d64"]
    log(f"workload {w.name}")
    kblk, vblk = kv_blocks(w)
    kb = [up(x, w.dtype) for x in kblk]
    vb = [up(x, w.dtype) for x in vblk]
    q = up(gen_block(w.seed, "q", 0, w.block_len, w.heads, w.head_dim, w.dtype), w.dtype)
    out, lse = ra.fwd(q, kb, vb, causal=False, rank=0)
    torch.cuda.synchronize()
    check_fwd_sampled(w, 0, out, lse, kblk, vblk, heads=list(range(w.heads)))


def test_full_causal_128k_all_ranks():
    require_gpu()
    w = WORKLOADS["causal_128k_h32_d128"]
    log(f"workload {w.name}")
    kblk, vblk = kv_blocks(w)
    kb = [up(x, w.dtype) for x in kblk]
    vb = [up(x, w.dtype) for x in vblk]
    results = {}
    for r in w.ranks:  # every rank's share, as the bench step runs them
        q = up(gen_block(w.seed, "q", r, w.block_len, w.heads, w.head_dim, w.dtype), w.dtype)
        results[r] = ra.fwd(q, kb, vb, causal=True, rank=r)
    torch.cuda.synchronize()
    for r in (0, 7, 15):
        check_fwd_sampled(w, r, *results[r], kblk, vblk, heads=[0, 17, 31])


def test_full_causal_512k_gqa_rank7():
    require_gpu()
    w = WORKLOADS["causal_512k_gqa32x8_rank7"]
    log(f"workload {w.name}")
    kblk, vblk = kv_blocks(w)
    kb = [up(x, w.dtype) for x in kblk]
    vb = [up(x, w.dtype) for x in vblk]
    q = up(gen_block(w.seed, "q", 7, w.block_len, w.heads, w.head_dim, w.dtype), w.dtype)
    out, lse = ra.fwd(q, kb, vb, causal=True, rank=7)
    torch.cuda.synchronize()
    check_fwd_sampled(w, 7, out, lse, kblk, vblk, heads=[0, 5, 31])


def test_full_backward_causal_32k():
    require_gpu()
    w = WORKLOADS["bwd_causal_32k_h32_d128"]
    log(f"workload {w.name}")
    c, D = w.block_len, w.n_blocks
    kblk, vblk = kv_blocks(w)
    kb = [up(x, w.dtype) for x in kblk]
    vb = [up(x, w.dtype) for x in vblk]
    qs = [gen_block(w.seed, "q", r, c, w.heads, w.head_dim, w.dtype) for r in range(D)]
    dos = [gen_block(w.seed, "do", r, c, w.heads, w.head_dim, w.dtype) for r in range(D)]
    dkb = [torch.zeros((c, w.kv_heads, w.head_dim), dtype=torch.float32, device="cuda") for _ in range(D)]
    dvb = [torch.zeros((c, w.kv_heads, w.head_dim), dtype=torch.float32, device="cuda") for _ in range(D)]
    dq = []
    for r in range(D):
        qd, dod = up(qs[r], w.dtype), up(dos[r], w.dtype)
        o, l = ra.fwd(qd, kb, vb, causal=True, rank=r)
        g, _, _ = ra.bwd(qd, kb, vb, o, dod, l, causal=True, rank=r, dk_blocks=dkb, dv_blocks=dvb)
        dq.append(g)
    torch.cuda.synchronize()
    dq = torch.cat(dq, 0)
    dk, dv = torch.cat(dkb, 0), torch.cat(dvb, 0)
    heads = [0, 31]  # whole heads: every row and every key of those heads
    q = np.concatenate(qs)[:, heads]
    do = np.concatenate(dos)[:, heads]
    k = np.concatenate(kblk)[:, heads]
    v = np.concatenate(vblk)[:, heads]
    dq_ref, dk_ref, dv_ref, _, _ = oracle.attention_bwd(q, k, v, do, causal=True)
    compare("dq", dq[:, heads], dq_ref, w.dtype)
    compare("dk", dk[:, heads], dk_ref, w.dtype)
    compare("dv", dv[:, heads], dv_ref, w.dtype)


def test_full_causal_128k_zigzag_sampled():
    """The zig-zag layout at full size: ranks 0 and 15, sampled rows and heads, against
    dense fp64 attention over every key at its zig-zag position."""
    require_gpu()
    w = WORKLOADS["causal_128k_h32_d128_zigzag"]
    log(f"workload {w.name}")
    c, D = w.block_len, w.n_blocks
    kblk, vblk = kv_blocks(w)
    kb = [up(x, w.dtype) for x in kblk]
    vb = [up(x, w.dtype) for x in vblk]
    kpos = np.concatenate([oracle.zigzag_positions(j, D, c) for j in range(D)])
    order = np.argsort(kpos)
    heads = [0, 31]
    k = np.concatenate(kblk)[order][:, heads]
    v = np.concatenate(vblk)[order][:, heads]
    for r in (0, 15):
        q = gen_block(w.seed, "q", r, c, w.heads, w.head_dim, w.dtype)
        out, lse = ra.fwd(up(q, w.dtype), kb, vb, causal=True, rank=r, zigzag=True)
        torch.cuda.synchronize()
        rows = sample_rows(c, seed=r)
        qpos = oracle.zigzag_positions(r, D, c)[rows]
        o_ref, l_ref = oracle.sampled_rows_fwd(q[rows][:, heads], qpos, k, v, causal=True, k_pos=kpos[order])
        compare(f"zigzag rank {r} out", out[torch.from_numpy(rows).cuda()][:, heads], o_ref, w.dtype)
        compare(f"zigzag rank {r} lse", lse[heads][:, torch.from_numpy(rows).cuda()], l_ref, w.dtype)
