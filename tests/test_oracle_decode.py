"""Pins of the decode oracle (CPU, fp64).

The decode definition (few query rows at given global positions against the
whole blocked context, causal by position) is pinned to scalar brute force,
to the ring's route (per-block partials folded by the log-sum-exp merge), to
closed forms, and to the special cases where positions make it plain
attention.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import gen_small


def blocks(seed, n_blocks, c, hkv, d):
    k = [gen_small(seed, (c, hkv, d), "f32", 1.0, 10 + j).astype(np.float64) for j in range(n_blocks)]
    v = [gen_small(seed, (c, hkv, d), "f32", 1.0, 40 + j).astype(np.float64) for j in range(n_blocks)]
    return k, v


def query(seed, q_len, hq, d, scale=1.0):
    return gen_small(seed, (q_len, hq, d), "f32", scale, 0).astype(np.float64)


@pytest.mark.parametrize("q_pos0", [0, 4, 9, 11, 30])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (3, 1)])
def test_decode_equals_brute_force(q_pos0, hq, hkv):
    # 3 blocks of 4 keys (positions 0..11), 3 query rows from q_pos0
    k, v = blocks(5, 3, 4, hkv, 3)
    q = query(5, 3, hq, 3, scale=1.3)
    o, lse = oracle.decode_forward(q, k, v, q_pos0)
    ob, lb = oracle.brute_force_fwd(q, np.concatenate(k), np.concatenate(v), causal=True,
                                    q_pos=q_pos0 + np.arange(3), k_pos=np.arange(12))
    np.testing.assert_allclose(o, ob, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, lb, atol=1e-13, rtol=0)


@pytest.mark.parametrize("q_pos0", [3, 17, 100])
def test_ring_partials_merged_equal_the_definition(q_pos0):
    k, v = blocks(7, 5, 8, 2, 4)
    q = query(7, 4, 4, 4)
    o, lse = oracle.decode_forward(q, k, v, q_pos0)
    om, lm = oracle.decode_by_partials(q, k, v, q_pos0)
    np.testing.assert_allclose(om, o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lm, lse, atol=1e-12, rtol=0)


def test_query_after_the_context_is_plain_attention():
    k, v = blocks(9, 4, 6, 1, 5)
    q = query(9, 2, 1, 5)
    o, lse = oracle.decode_forward(q, k, v, q_pos0=10_000)
    o2, l2 = oracle.attention_fwd(q, np.concatenate(k), np.concatenate(v), causal=False)
    np.testing.assert_allclose(o, o2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, l2, atol=1e-13, rtol=0)


def test_first_position_sees_only_key_zero():
    k, v = blocks(11, 2, 5, 1, 4)
    q = query(11, 1, 1, 4)
    o, lse = oracle.decode_forward(q, k, v, q_pos0=0)
    np.testing.assert_allclose(o[0, 0], v[0][0, 0], atol=1e-15, rtol=0)
    assert math.isclose(lse[0, 0], float(q[0, 0] @ k[0][0, 0]) / 2.0, abs_tol=1e-14)  # 1/sqrt(4) = 1/2


def test_uniform_values_and_zero_query_closed_forms():
    k, v = blocks(13, 3, 4, 1, 3)
    vv = [np.broadcast_to(np.array([1.5, -2.0, 0.25]), b.shape).copy() for b in v]
    q = query(13, 2, 1, 3)
    o, _ = oracle.decode_forward(q, k, vv, q_pos0=6)
    np.testing.assert_allclose(o, np.broadcast_to([1.5, -2.0, 0.25], o.shape), atol=1e-14, rtol=0)
    # zero query: uniform weights over the visible keys -> mean of visible values, lse = ln(count)
    q0 = np.zeros((2, 1, 3))
    o, lse = oracle.decode_forward(q0, k, v, q_pos0=6)
    allv = np.concatenate(v)
    np.testing.assert_allclose(o[0, 0], allv[:7, 0].mean(axis=0), atol=1e-14, rtol=0)
    np.testing.assert_allclose(o[1, 0], allv[:8, 0].mean(axis=0), atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse[0], [math.log(7), math.log(8)], atol=1e-14, rtol=0)


def test_planted_position_mistake_is_caught(monkeypatch):
    """Shift the query positions by one inside the oracle: the brute-force pin must fail."""
    import oracle.decode as dec

    real = dec._positions
    monkeypatch.setattr(dec, "_positions", lambda q_len, q_pos0, c, nb: real(q_len, q_pos0 + 1, c, nb))
    k, v = blocks(5, 3, 4, 2, 3)
    q = query(5, 3, 4, 3, scale=1.3)
    o, _ = oracle.decode_forward(q, k, v, 4)
    ob, _ = oracle.brute_force_fwd(q, np.concatenate(k), np.concatenate(v), causal=True,
                                   q_pos=4 + np.arange(3), k_pos=np.arange(12))
    assert np.max(np.abs(o - ob)) > 1e-3
