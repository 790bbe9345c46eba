"""CPU pins for the fp64 oracle: it is checked against things other than itself.

Each test names what fixes the expected value: brute force with exactly
rounded sums, a library routine (torch's fp64 CPU attention and autograd) on
the special case D = 1, closed forms, invariants the pages state (blockwise
online accumulation equals dense attention in any block order; the ring walk
of the four-GPU example), finite differences for the backward, and gradient
identities that follow from softmax rows summing to one.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.ring import finish_online, online_block_forward
from workloads import gen_small

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(seed, shape, scale=1.0, stream=0):
    return gen_small(seed, shape, "f32", scale, stream).astype(np.float64)


def qkv(seed, n, m, hq, hkv, d, scale=1.0):
    return (rand(seed, (n, hq, d), scale, 0), rand(seed, (m, hkv, d), scale, 1),
            rand(seed, (m, hkv, d), 1.0, 2))


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2), (3, 1)])
def test_dense_equals_brute_force(causal, hq, hkv):
    n, m, d = 5, 7, 3
    q, k, v = qkv(11, n, m, hq, hkv, d, scale=1.5)
    q_pos = np.arange(2, 2 + n)            # rows 2..6 of a 7-key sequence
    o, lse = oracle.attention_fwd(q, k, v, causal=causal, q_pos=q_pos)
    ob, lb = oracle.brute_force_fwd(q, k, v, causal=causal, q_pos=q_pos)
    np.testing.assert_allclose(o, ob, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, lb, atol=1e-13, rtol=0)


def test_empty_rows_give_zero_and_neg_inf():
    q, k, v = qkv(3, 4, 6, 2, 2, 4)
    # queries at positions 0..3, keys at 10..15: every row fully masked
    o, lse = oracle.attention_fwd(q, k, v, causal=True, q_pos=np.arange(4), k_pos=np.arange(10, 16))
    assert np.all(o == 0.0) and np.all(lse == -np.inf)
    ob, lb = oracle.brute_force_fwd(q, k, v, causal=True, q_pos=np.arange(4), k_pos=np.arange(10, 16))
    assert np.all(ob == 0.0) and np.all(lb == -np.inf)


# ------------------------------------------------------ library special case
def _torch_sdpa(q, k, v, causal):
    group = q.shape[1] // k.shape[1]
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(np.repeat(k, group, axis=1)).permute(1, 0, 2)[None]
    tv = torch.from_numpy(np.repeat(v, group, axis=1)).permute(1, 0, 2)[None]
    return tq, tk, tv


@pytest.mark.parametrize("causal", [False, True])
def test_dense_equals_torch_sdpa_fp64(causal):
    q, k, v = qkv(5, 96, 96, 4, 2, 32)
    o, _ = oracle.attention_fwd(q, k, v, causal=causal)
    tq, tk, tv = _torch_sdpa(q, k, v, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_equals_torch_autograd_fp64(causal):
    q, k, v = qkv(6, 80, 80, 4, 2, 16)
    do = rand(7, (80, 4, 16))
    dq, dk, dv, o, _ = oracle.attention_bwd(q, k, v, do, causal=causal)
    tq = torch.from_numpy(q.copy()).requires_grad_()
    tk = torch.from_numpy(k.copy()).requires_grad_()
    tv = torch.from_numpy(v.copy()).requires_grad_()
    group = 2
    out = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(1, 0, 2)[None], tk.repeat_interleave(group, dim=1).permute(1, 0, 2)[None],
        tv.repeat_interleave(group, dim=1).permute(1, 0, 2)[None], is_causal=causal)
    (out[0].permute(1, 0, 2) * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(o, out[0].permute(1, 0, 2).detach().numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12, rtol=0)


# --------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_uniform_values_give_constant_output(causal):
    q, k, _ = qkv(8, 40, 40, 2, 1, 16, scale=3.0)
    vrow = rand(9, (1, 1, 16))
    v = np.broadcast_to(vrow, (40, 1, 16)).copy()
    o, _ = oracle.attention_fwd(q, k, v, causal=causal)
    np.testing.assert_allclose(o, np.broadcast_to(vrow, o.shape), atol=1e-14, rtol=0)


def test_single_key_gives_its_value():
    q, k, v = qkv(10, 6, 1, 3, 3, 8)
    o, lse = oracle.attention_fwd(q, k, v, causal=False)
    np.testing.assert_array_equal(o, np.broadcast_to(v[0][None], o.shape))
    expect = np.einsum("nhd,hd->hn", q, k[0]) / math.sqrt(8)
    np.testing.assert_allclose(lse, expect, atol=1e-14, rtol=0)


def test_causal_first_row_sees_one_key():
    q, k, v = qkv(12, 16, 16, 2, 2, 8)
    o, lse = oracle.attention_fwd(q, k, v, causal=True)
    np.testing.assert_array_equal(o[0], v[0])
    np.testing.assert_allclose(lse[:, 0], np.sum(q[0] * k[0], axis=1) / math.sqrt(8), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(causal):
    _, k, v = qkv(13, 24, 24, 2, 2, 8)
    q = np.zeros((24, 2, 8))
    o, lse = oracle.attention_fwd(q, k, v, causal=causal)
    for i in range(24):
        nvis = i + 1 if causal else 24
        np.testing.assert_allclose(o[i], v[:nvis].mean(axis=0), atol=1e-14, rtol=0)
        np.testing.assert_allclose(lse[:, i], math.log(nvis), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_changes_only_lse(causal):
    q, k, v = qkv(14, 30, 30, 2, 2, 8)
    u = rand(15, (2, 8))
    o1, l1 = oracle.attention_fwd(q, k, v, causal=causal)
    o2, l2 = oracle.attention_fwd(q, k + u[None], v, causal=causal)
    np.testing.assert_allclose(o2, o1, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l2, l1 + np.einsum("nhd,hd->hn", q, u) / math.sqrt(8), atol=1e-12)


def test_gqa_equals_repeated_kv_mha():
    q, k, v = qkv(16, 20, 28, 8, 2, 8)
    for causal in (False, True):
        o_g, l_g = oracle.attention_fwd(q, k, v, causal=causal, q_pos=np.arange(8, 28))
        o_m, l_m = oracle.attention_fwd(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1),
                                        causal=causal, q_pos=np.arange(8, 28))
        np.testing.assert_array_equal(o_g, o_m)
        np.testing.assert_array_equal(l_g, l_m)


# ----------------------------------------- the pages' invariants (blockwise)
def _split(m, rng):
    cuts = np.sort(rng.choice(np.arange(1, m), size=3, replace=False))
    return [0, *cuts.tolist(), m]


@pytest.mark.parametrize("causal", [False, True])
def test_online_blockwise_equals_dense_any_order(causal):
    rng = np.random.default_rng(0)
    q, k, v = qkv(17, 33, 57, 4, 2, 16, scale=2.0)
    q_pos = np.arange(24, 57)
    o_ref, l_ref = oracle.attention_fwd(q, k, v, causal=causal, q_pos=q_pos)
    bounds = _split(57, rng)                 # uneven blocks
    blocks = list(zip(bounds[:-1], bounds[1:]))
    for trial in range(4):
        order = rng.permutation(len(blocks)) if (trial or not causal) else np.arange(len(blocks))
        state = None
        for b in order:
            a, e = blocks[b]
            state = online_block_forward(state, q, k[a:e], v[a:e], causal=causal, q_pos=q_pos,
                                         k_pos=np.arange(a, e))
        o, l = finish_online(state)
        np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
        np.testing.assert_allclose(l, l_ref, atol=1e-12, rtol=0)


def test_noncausal_result_independent_of_block_order():
    q, k, v = qkv(18, 16, 64, 2, 2, 8)
    kb = [k[i * 16:(i + 1) * 16] for i in range(4)]
    vb = [v[i * 16:(i + 1) * 16] for i in range(4)]
    outs = []
    for order in ([0, 1, 2, 3], [3, 2, 1, 0], [2, 0, 3, 1]):
        outs.append(oracle.ring_forward(q, kb, vb, order, causal=False, q_pos=np.arange(16),
                                        block_len=16))
    for o, l in outs[1:]:
        np.testing.assert_allclose(o, outs[0][0], atol=1e-12, rtol=0)
        np.testing.assert_allclose(l, outs[0][1], atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_ring_over_all_ranks_equals_full_attention(causal):
    D, c, hq, hkv, d = 4, 12, 4, 2, 8
    q, k, v = qkv(19, D * c, D * c, hq, hkv, d)
    o_ref, l_ref = oracle.attention_fwd(q, k, v, causal=causal)
    kb = [k[j * c:(j + 1) * c] for j in range(D)]
    vb = [v[j * c:(j + 1) * c] for j in range(D)]
    for r in range(D):
        steps = oracle.ring_steps(r, D, causal)
        qp = oracle.positions_for_block(r, c)
        o, l = oracle.ring_forward(q[r * c:(r + 1) * c], kb, vb, steps, causal=causal, q_pos=qp,
                                   block_len=c)
        np.testing.assert_allclose(o, o_ref[r * c:(r + 1) * c], atol=1e-12, rtol=0)
        np.testing.assert_allclose(l, l_ref[:, r * c:(r + 1) * c], atol=1e-12, rtol=0)


# ---------------------------------------------------------------------- merge
def _partial(seed, n=9, hq=3, d=5):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, hq, d)), rng.standard_normal((hq, n)) * 3


def test_merge_commutative_associative_identity():
    a, b, c = _partial(1), _partial(2), _partial(3)
    ab = oracle.merge_partials(*a, *b)
    ba = oracle.merge_partials(*b, *a)
    np.testing.assert_allclose(ab[0], ba[0], atol=1e-14)
    np.testing.assert_allclose(ab[1], ba[1], atol=1e-14)
    l = oracle.merge_partials(*ab, *c)
    r = oracle.merge_partials(*a, *oracle.merge_partials(*b, *c))
    np.testing.assert_allclose(l[0], r[0], atol=1e-13)
    np.testing.assert_allclose(l[1], r[1], atol=1e-13)
    empty = (np.zeros_like(a[0]), np.full_like(a[1], -np.inf))
    e = oracle.merge_partials(*a, *empty)
    np.testing.assert_array_equal(e[0], a[0])
    np.testing.assert_array_equal(e[1], a[1])
    ee = oracle.merge_partials(*empty, *empty)
    assert np.all(ee[0] == 0) and np.all(ee[1] == -np.inf) and not np.any(np.isnan(ee[0]))


def test_merge_scalar_hand_values():
    # two single-key partials with scores 0 and log 3: weights 1/4 and 3/4
    o, lse = oracle.merge_partials_scalar(1.0, 0.0, 5.0, math.log(3.0))
    assert abs(o - (0.25 * 1.0 + 0.75 * 5.0)) < 1e-15
    assert abs(lse - math.log(4.0)) < 1e-15
    vo, vl = oracle.merge_partials(np.array([[[1.0]]]), np.array([[0.0]]),
                                   np.array([[[5.0]]]), np.array([[math.log(3.0)]]))
    assert abs(vo[0, 0, 0] - o) < 1e-15 and abs(vl[0, 0] - lse) < 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_merging_per_block_partials_equals_full(causal):
    D, c = 4, 10
    q, k, v = qkv(20, c, D * c, 2, 1, 8)
    qp = oracle.positions_for_block(2, c)
    o_ref, l_ref = oracle.attention_fwd(q, k, v, causal=causal, q_pos=qp)
    acc = None
    for j in oracle.ring_steps(2, D, causal):
        part = oracle.attention_fwd(q, k[j * c:(j + 1) * c], v[j * c:(j + 1) * c], causal=causal,
                                    q_pos=qp, k_pos=oracle.positions_for_block(j, c))
        acc = part if acc is None else oracle.merge_partials(*acc, *part)
    np.testing.assert_allclose(acc[0], o_ref, atol=1e-13)
    np.testing.assert_allclose(acc[1], l_ref, atol=1e-13)


# ---------------------------------------------------------------- ring schedule
def _golden_walkthrough():
    rows = []
    with open(os.path.join(GOLDEN, "ring_walkthrough_4gpu.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                kind, rnd, host, blk = line.split()
                rows.append((kind, int(rnd), int(host), int(blk)))
    return rows


def test_ring_simulator_matches_four_gpu_walkthrough():
    used = oracle.simulate_ring(4)
    for kind, rnd, host, blk in _golden_walkthrough():
        if kind == "use":
            assert used[rnd - 1][host] == blk
        else:  # the block a host sends in round r is what the next host uses in round r+1
            assert used[rnd][(host + 1) % 4] == blk
    for host in range(4):
        assert sorted(used[r][host] for r in range(4)) == [0, 1, 2, 3]


@pytest.mark.parametrize("D", [1, 2, 4, 8, 16])
def test_ring_steps_follow_the_simulator(D):
    used = oracle.simulate_ring(D)
    for r in range(D):
        assert oracle.ring_steps(r, D, False) == [used[s][r] for s in range(D)]
        causal = oracle.ring_steps(r, D, True)
        assert causal == [j for j in (used[s][r] for s in range(D)) if j <= r]
        assert causal[0] == r and len(causal) == r + 1


# ------------------------------------------------------------------- backward
def _loss(q, k, v, do, causal, group_kv=None):
    o, _ = oracle.attention_fwd(q, k, v, causal=causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal,hq,hkv", [(False, 2, 2), (True, 2, 2), (True, 2, 1)])
def test_backward_finite_differences(causal, hq, hkv):
    # 2 query heads, 64 tokens, head_dim 128 (the backward workload's head size)
    n, d = 64, 128
    q, k, v = qkv(21, n, n, hq, hkv, d)
    do = rand(22, (n, hq, d))
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, causal=causal)
    rng = np.random.default_rng(23)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(3):
            u = rng.standard_normal(x.shape)
            args = {"q": q, "k": k, "v": v}
            args[name] = x + h * u
            lp = _loss(args["q"], args["k"], args["v"], do, causal)
            args[name] = x - h * u
            lm = _loss(args["q"], args["k"], args["v"], do, causal)
            fd = (lp - lm) / (2 * h)
            an = float(np.sum(g * u))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    # a few single coordinates too
    for idx in [(0, 0, 0), (n - 1, hq - 1, d - 1), (17, 0, 63)]:
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            j = (idx[0], min(idx[1], x.shape[1] - 1), idx[2])
            xp = x.copy(); xp[j] += h
            xm = x.copy(); xm[j] -= h
            args_p = {"q": q, "k": k, "v": v, name: xp}
            args_m = {"q": q, "k": k, "v": v, name: xm}
            fd = (_loss(args_p["q"], args_p["k"], args_p["v"], do, causal)
                  - _loss(args_m["q"], args_m["k"], args_m["v"], do, causal)) / (2 * h)
            assert abs(fd - g[j]) <= 1e-6 * max(1.0, abs(g[j])), (name, j, fd, g[j])


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    q, k, v = qkv(24, 48, 48, 4, 2, 16)
    do = rand(25, (48, 4, 16))
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, causal=causal)
    # softmax rows sum to one: sum_t dV_t = sum_i dO_i (per K/V head, summed over its group)
    np.testing.assert_allclose(dv.sum(axis=0), do.reshape(48, 2, 2, 16).sum(axis=(0, 2)), atol=1e-10)
    # ... and sum_t dS_it = 0, hence sum_t dK_t = 0
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-10)
    # uniform V: the output does not depend on Q or K
    vu = np.broadcast_to(v[:1], v.shape).copy()
    dq2, dk2, _, _, _ = oracle.attention_bwd(q, k, vu, do, causal=causal)
    np.testing.assert_allclose(dq2, 0.0, atol=1e-10)
    np.testing.assert_allclose(dk2, 0.0, atol=1e-10)


def test_backward_single_key_has_zero_dq():
    q, k, v = qkv(26, 5, 1, 2, 2, 8)
    do = rand(27, (5, 2, 8))
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, causal=False)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv[0], do.sum(axis=0), atol=1e-14)


@pytest.mark.parametrize("causal,hq,hkv", [(False, 2, 2), (True, 4, 2), (True, 3, 1)])
def test_backward_at_chosen_keys_equals_full_backward(causal, hq, hkv):
    """attention_bwd_keys (dK/dV at a few keys, over every row) agrees with the columns
    of the full analytic backward, which finite differences pin; causal keys include
    key 0 (seen by every row) and the last key (seen by one row)."""
    n, d = 70, 16
    q, k, v = qkv(41, n, n, hq, hkv, d)
    do = rand(42, (n, hq, d))
    _, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, causal=causal)
    keys = np.array([0, 1, 33, 34, 68, 69])
    dk_s, dv_s = oracle.attention_bwd_keys(q, k, v, do, causal=causal, keys=keys)
    np.testing.assert_allclose(dk_s, dk[keys], atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv_s, dv[keys], atol=1e-12, rtol=0)


def test_backward_at_chosen_keys_finite_differences():
    """dK/dV at chosen keys against central differences of L = sum(O * dO) with respect
    to those keys' rows alone (causal, grouped heads)."""
    n, hq, hkv, d = 40, 2, 1, 32
    q, k, v = qkv(43, n, n, hq, hkv, d)
    do = rand(44, (n, hq, d))
    keys = np.array([0, 19, 39])
    dk_s, dv_s = oracle.attention_bwd_keys(q, k, v, do, causal=True, keys=keys)
    rng = np.random.default_rng(45)
    h = 1e-6
    for name, x, g in (("k", k, dk_s), ("v", v, dv_s)):
        for _ in range(3):
            u = np.zeros_like(x)
            u[keys] = rng.standard_normal((keys.size,) + x.shape[1:])
            args = {"q": q, "k": k, "v": v}
            args[name] = x + h * u
            lp = _loss(args["q"], args["k"], args["v"], do, True)
            args[name] = x - h * u
            lm = _loss(args["q"], args["k"], args["v"], do, True)
            fd = (lp - lm) / (2 * h)
            an = float(np.sum(g * u[keys]))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


# ------------------------------------------------------------ zig-zag layout
@pytest.mark.parametrize("D", [1, 2, 4, 8])
def test_zigzag_positions_partition_the_sequence(D):
    c = 6
    pos = np.concatenate([oracle.zigzag_positions(b, D, c) for b in range(D)])
    assert np.array_equal(np.sort(pos), np.arange(D * c))


@pytest.mark.parametrize("D", [2, 4, 16])
def test_zigzag_balances_causal_work(D):
    c = 8
    flat = oracle.visible_pairs_per_rank(D, c, zigzag=False)
    zz = oracle.visible_pairs_per_rank(D, c, zigzag=True)
    # contiguous: rank r sees r*c*c + c(c+1)/2 pairs; zig-zag: the same count for every rank
    assert flat == [r * c * c + c * (c + 1) // 2 for r in range(D)]
    assert len(set(zz)) == 1 and sum(zz) == sum(flat)


def test_zigzag_ring_equals_dense_attention():
    """Every rank's zig-zag share, computed block by block along the ring with online
    softmax at the chunks' true positions, equals dense causal attention."""
    D, c, hq, hkv, d = 4, 6, 2, 1, 4
    S = D * c
    q, k, v = qkv(17, S, S, hq, hkv, d)
    o_ref, l_ref = oracle.attention_fwd(q, k, v, causal=True)
    for r in range(D):
        qp = oracle.zigzag_positions(r, D, c)
        state = None
        for j in oracle.ring_steps(r, D, causal=False):
            kp = oracle.zigzag_positions(j, D, c)
            state = online_block_forward(state, q[qp], k[kp], v[kp], causal=True, q_pos=qp, k_pos=kp)
        o, l = finish_online(state)
        np.testing.assert_allclose(o, o_ref[qp], atol=1e-12, rtol=0)
        np.testing.assert_allclose(l, l_ref[:, qp], atol=1e-12, rtol=0)
