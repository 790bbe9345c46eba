"""GPU parity at the workloads' full sizes, in the launch configuration bench.py uses.

Every workload's GPU result is computed in full; the fp64 oracle is evaluated
on sampled query rows and heads (each sampled output is exact attention over
all of that row's visible keys), and for the backward on whole heads.
"""
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

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


def check_fwd_rows_all_heads(w, rank, out, lse, kblk, vblk, rows):
    """Every head of the chosen rows of one rank against the oracle, one oracle call per head
    (side by side on the host's cores)."""
    c = w.block_len
    group = w.heads // w.kv_heads
    q = gen_block(w.seed, "q", rank, c, w.heads, w.head_dim, w.dtype)[rows]
    nvis = rank + 1 if w.causal else w.n_blocks
    k_all = np.concatenate(kblk[:nvis])
    v_all = np.concatenate(vblk[:nvis])

    def ref(h):
        g = h // group
        return oracle.sampled_rows_fwd(q[:, [h]], rank * c + rows, k_all[:, [g]], v_all[:, [g]], causal=w.causal)

    refs = _pool(ref, list(range(w.heads)))
    o_ref = np.concatenate([r[0] for r in refs], axis=1)
    l_ref = np.concatenate([r[1] for r in refs], axis=0)
    idx = torch.from_numpy(rows).cuda()
    compare(f"{w.name} rank {rank} out ({rows.size} rows x {w.heads} heads)", out[idx], o_ref, w.dtype)
    compare(f"{w.name} rank {rank} lse", lse[:, idx], l_ref, w.dtype)


def test_full_noncausal_64k_h16_d64():
    """Every head at the first and last 64 rows and every 64th row of the query block."""
    require_gpu()
    w = WORKLOADS["noncausal_64k_h16_d64"]
    log(f"workload {w.name}")
    kblk, vblk = kv_blocks(w)
    kb = [up(x, w.dtype) for x in kblk]
    vb = [up(x, w.dtype) for x in vblk]
    q = up(gen_block(w.seed, "q", 0, w.block_len, w.heads, w.head_dim, w.dtype), w.dtype)
    out, lse = ra.fwd(q, kb, vb, causal=False, rank=0)
    torch.cuda.synchronize()
    c = w.block_len
    rows = np.unique(np.concatenate([np.arange(64), np.arange(c - 64, c), np.arange(0, c, 64)])).astype(np.int64)
    check_fwd_rows_all_heads(w, 0, out, lse, kblk, vblk, rows)


def dense_rows(c):
    """First and last 64 rows plus every 16th row of a query block."""
    return np.unique(np.concatenate([np.arange(64), np.arange(c - 64, c), np.arange(0, c, 16)])).astype(np.int64)


def _pool(fn, items):
    """Independent oracle calls side by side: numpy's matrix products and elementwise
    loops release the GIL, so one thread per core, each with a single-threaded BLAS."""
    workers = max(1, min(16, os.cpu_count() or 1))
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))


def test_full_causal_128k_all_ranks():
    """The headline workload's forward, as bench.py runs it: every rank's share against
    the oracle on every head, at the first and last 64 rows and every 16th row."""
    require_gpu()
    w = WORKLOADS["causal_128k_h32_d128"]
    log(f"workload {w.name}")
    t0 = time.time()
    c = w.block_len
    kblk, vblk = kv_blocks(w)
    kb = [up(x, w.dtype) for x in kblk]
    vb = [up(x, w.dtype) for x in vblk]
    rows = dense_rows(c)
    got = {}
    for r in w.ranks:  # every rank's share, as the bench step runs them
        q = up(gen_block(w.seed, "q", r, w.block_len, w.heads, w.head_dim, w.dtype), w.dtype)
        out, lse = ra.fwd(q, kb, vb, causal=True, rank=r)
        idx = torch.from_numpy(rows).cuda()
        got[r] = (out[idx].cpu(), lse[:, idx].cpu())
    torch.cuda.synchronize()
    k_all, v_all = np.concatenate(kblk), np.concatenate(vblk)

    qs = {r: gen_block(w.seed, "q", r, c, w.heads, w.head_dim, w.dtype)[rows] for r in w.ranks}

    def ref(task):  # one rank and one head (MHA: K/V head = query head)
        r, h = task
        nvis = (r + 1) * c
        return oracle.sampled_rows_fwd(qs[r][:, [h]], r * c + rows, k_all[:nvis, [h]], v_all[:nvis, [h]],
                                       causal=True)

    tasks = [(r, h) for r in reversed(w.ranks) for h in range(w.heads)]  # longest first
    refs = dict(zip(tasks, _pool(ref, tasks)))
    for r in w.ranks:
        o_ref = np.concatenate([refs[(r, h)][0] for h in range(w.heads)], axis=1)
        l_ref = np.concatenate([refs[(r, h)][1] for h in range(w.heads)], axis=0)
        compare(f"{w.name} rank {r} out ({rows.size} rows x {w.heads} heads)", got[r][0], o_ref, w.dtype)
        compare(f"{w.name} rank {r} lse", got[r][1], l_ref, w.dtype)
    log(f"  {time.time() - t0:.1f}s")


def test_full_backward_causal_128k():
    """The headline workload's backward, as bench.py runs it (forward and backward of every
    rank, dK/dV accumulated over the ranks).  dQ: sampled rows of every rank, every head.
    dK/dV: heads 0 and 31 at sampled keys of blocks 0 (seen by every row), 7 and 15,
    against the oracle's own forward over all 131072 rows of those heads."""
    require_gpu()
    w = WORKLOADS["causal_128k_h32_d128"]
    log(f"workload {w.name} backward")
    t0 = time.time()
    c, D, H, d = w.block_len, w.n_blocks, w.heads, w.head_dim
    kblk, vblk = kv_blocks(w)
    kb = [up(x, w.dtype) for x in kblk]
    vb = [up(x, w.dtype) for x in vblk]
    qs = [gen_block(w.seed, "q", r, c, H, d, w.dtype) for r in range(D)]
    dos = [gen_block(w.seed, "do", r, c, H, d, w.dtype) for r in range(D)]
    dkb = [torch.zeros((c, w.kv_heads, d), dtype=torch.float32, device="cuda") for _ in range(D)]
    dvb = [torch.zeros((c, w.kv_heads, d), dtype=torch.float32, device="cuda") for _ in range(D)]
    qrows = {r: sample_rows(c, n_random=4, seed=100 + r) for r in range(D)}
    dq_got = {}
    for r in range(D):
        qd, dod = up(qs[r], w.dtype), up(dos[r], w.dtype)
        o, l = ra.fwd(qd, kb, vb, causal=True, rank=r)
        g, _, _ = ra.bwd(qd, kb, vb, o, dod, l, causal=True, rank=r, dk_blocks=dkb, dv_blocks=dvb)
        dq_got[r] = g[torch.from_numpy(qrows[r]).cuda()].cpu()
    torch.cuda.synchronize()
    heads = [0, 31]
    keys = np.array([0, 1, 17, c // 2, c - 1, 7 * c, 7 * c + 4095, D * c - 2, D * c - 1], dtype=np.int64)
    dk_got = torch.cat(dkb, 0)[torch.from_numpy(keys).cuda()][:, heads].cpu()
    dv_got = torch.cat(dvb, 0)[torch.from_numpy(keys).cuda()][:, heads].cpu()
    k_all, v_all = np.concatenate(kblk), np.concatenate(vblk)

    def dq_ref(r):
        rows = qrows[r]
        nvis = (r + 1) * c
        g, _, _, _, _ = oracle.attention_bwd(qs[r][rows], k_all[:nvis], v_all[:nvis], dos[r][rows], causal=True,
                                             q_pos=r * c + rows)
        return g

    for r, ref in zip(range(D), _pool(dq_ref, list(range(D)))):
        compare(f"dq rank {r} ({qrows[r].size} rows x {H} heads)", dq_got[r], ref, w.dtype)

    # dK/dV at the chosen keys sum over every row of the head: split the rows into ranges
    # (each range's sum is exact), add the ranges' contributions
    q_h = np.concatenate(qs)[:, heads]
    do_h = np.concatenate(dos)[:, heads]
    k_h, v_h = k_all[:, heads], v_all[:, heads]
    step = 8192

    def dkdv_part(task):  # one row range of one head
        r0, i = task
        r1 = min(D * c, r0 + step)
        return oracle.attention_bwd_keys(q_h[r0:r1, [i]], k_h[:, [i]], v_h[:, [i]], do_h[r0:r1, [i]], causal=True,
                                         keys=keys, q_pos=np.arange(r0, r1))

    tasks = [(r0, i) for r0 in reversed(range(0, D * c, step)) for i in range(len(heads))]  # longest first
    parts = dict(zip(tasks, _pool(dkdv_part, tasks)))
    dk_ref = np.concatenate([np.sum([parts[(r0, i)][0] for r0 in range(0, D * c, step)], axis=0)
                             for i in range(len(heads))], axis=1)
    dv_ref = np.concatenate([np.sum([parts[(r0, i)][1] for r0 in range(0, D * c, step)], axis=0)
                             for i in range(len(heads))], axis=1)
    compare(f"dk heads {heads} at {keys.size} keys", dk_got, dk_ref, w.dtype)
    compare(f"dv heads {heads} at {keys.size} keys", dv_got, dv_ref, w.dtype)
    log(f"  {time.time() - t0:.1f}s")


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
    # every head at the first and last 64 rows and every 512th row (each sees up to all 524288 keys)
    c = w.block_len
    rows = np.unique(np.concatenate([np.arange(64), np.arange(c - 64, c), np.arange(0, c, 512)])).astype(np.int64)
    check_fwd_rows_all_heads(w, 7, out, lse, kblk, vblk, rows)


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


def test_full_backward_causal_128k_zigzag():
    """The zig-zag layout's backward at full size, as its bench workload runs it (forward and
    backward of every rank, dK/dV accumulated over the ranks).  dQ: sampled rows of every rank,
    every head.  dK/dV: heads 0 and 31 at keys of both chunks of blocks 0, 7 and 15, against the
    oracle over all 131072 rows at their zig-zag positions."""
    require_gpu()
    w = WORKLOADS["causal_128k_h32_d128_zigzag"]
    log(f"workload {w.name} backward")
    t0 = time.time()
    c, D, H, d = w.block_len, w.n_blocks, w.heads, w.head_dim
    kblk, vblk = kv_blocks(w)
    kb = [up(x, w.dtype) for x in kblk]
    vb = [up(x, w.dtype) for x in vblk]
    qs = [gen_block(w.seed, "q", r, c, H, d, w.dtype) for r in range(D)]
    dos = [gen_block(w.seed, "do", r, c, H, d, w.dtype) for r in range(D)]
    dkb = [torch.zeros((c, w.kv_heads, d), dtype=torch.float32, device="cuda") for _ in range(D)]
    dvb = [torch.zeros((c, w.kv_heads, d), dtype=torch.float32, device="cuda") for _ in range(D)]
    qrows = {r: sample_rows(c, n_random=4, seed=200 + r) for r in range(D)}
    dq_got = {}
    for r in range(D):
        qd, dod = up(qs[r], w.dtype), up(dos[r], w.dtype)
        o, l = ra.fwd(qd, kb, vb, causal=True, rank=r, zigzag=True)
        g, _, _ = ra.bwd(qd, kb, vb, o, dod, l, causal=True, rank=r, dk_blocks=dkb, dv_blocks=dvb, zigzag=True)
        dq_got[r] = g[torch.from_numpy(qrows[r]).cuda()].cpu()
    torch.cuda.synchronize()

    # the whole sequence in position order: block b's rows sit at zigzag_positions(b)
    pos = np.concatenate([oracle.zigzag_positions(j, D, c) for j in range(D)])
    order = np.argsort(pos)  # order[p] = row (in block-concatenated order) at position p
    k_pos = np.arange(D * c, dtype=np.int64)
    k_all = np.concatenate(kblk)[order]
    v_all = np.concatenate(vblk)[order]

    def dq_ref(r):
        rows = qrows[r]
        g, _, _, _, _ = oracle.attention_bwd(qs[r][rows], k_all, v_all, dos[r][rows], causal=True,
                                             q_pos=oracle.zigzag_positions(r, D, c)[rows], k_pos=k_pos)
        return g

    for r, ref in zip(range(D), _pool(dq_ref, list(range(D)))):
        compare(f"zigzag dq rank {r} ({qrows[r].size} rows x {H} heads)", dq_got[r], ref, w.dtype)

    heads = [0, 31]
    h2 = c // 2
    kidx = np.array([b * c + t for b in (0, 7, 15) for t in (0, 1, h2 - 1, h2, h2 + 1, c - 1)], dtype=np.int64)
    dk_got = torch.cat(dkb, 0)[torch.from_numpy(kidx).cuda()][:, heads].cpu()
    dv_got = torch.cat(dvb, 0)[torch.from_numpy(kidx).cuda()][:, heads].cpu()
    keys = pos[kidx]  # the chosen keys' positions = their indices in position order
    q_h = np.concatenate(qs)[order][:, heads]
    do_h = np.concatenate(dos)[order][:, heads]
    k_h, v_h = k_all[:, heads], v_all[:, heads]
    step = 8192

    def dkdv_part(task):  # one row range (in position order) of one head
        r0, i = task
        r1 = min(D * c, r0 + step)
        return oracle.attention_bwd_keys(q_h[r0:r1, [i]], k_h[:, [i]], v_h[:, [i]], do_h[r0:r1, [i]], causal=True,
                                         keys=keys, q_pos=np.arange(r0, r1), k_pos=k_pos)

    tasks = [(r0, i) for r0 in reversed(range(0, D * c, step)) for i in range(len(heads))]  # longest first
    parts = dict(zip(tasks, _pool(dkdv_part, tasks)))
    dk_ref = np.concatenate([np.sum([parts[(r0, i)][0] for r0 in range(0, D * c, step)], axis=0)
                             for i in range(len(heads))], axis=1)
    dv_ref = np.concatenate([np.sum([parts[(r0, i)][1] for r0 in range(0, D * c, step)], axis=0)
                             for i in range(len(heads))], axis=1)
    compare(f"zigzag dk heads {heads} at {keys.size} keys", dk_got, dk_ref, w.dtype)
    compare(f"zigzag dv heads {heads} at {keys.size} keys", dv_got, dv_ref, w.dtype)
    log(f"  {time.time() - t0:.1f}s")
