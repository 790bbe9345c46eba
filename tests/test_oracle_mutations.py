"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch them.

Each mutation patches one piece of the fp64 oracle in place for the duration
of a test, then evaluates pins that do not depend on the patched code path
(brute force, torch fp64 attention, closed forms, finite differences).  A
mutation that slips through every pin would mean the pins are too weak.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.dense as dense
from workloads import gen_small


def rand(seed, shape, scale=1.0, stream=0):
    return gen_small(seed, shape, "f32", scale, stream).astype(np.float64)


def pins_fwd_error():
    """Largest error of the dense oracle across the forward pins."""
    errs = []
    q, k, v = rand(1, (6, 4, 3), 1.5, 0), rand(1, (6, 2, 3), 1.5, 1), rand(1, (6, 2, 3), 1.0, 2)
    for causal in (False, True):
        o, l = oracle.attention_fwd(q, k, v, causal=causal)
        ob, lb = oracle.brute_force_fwd(q, k, v, causal=causal)
        errs += [np.max(np.abs(o - ob)), np.max(np.abs(l - lb))]
        tq = torch.from_numpy(q).permute(1, 0, 2)[None]
        tk = torch.from_numpy(np.repeat(k, 2, axis=1)).permute(1, 0, 2)[None]
        tv = torch.from_numpy(np.repeat(v, 2, axis=1)).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
        errs.append(np.max(np.abs(o - ref[0].permute(1, 0, 2).numpy())))
    # single key: lse is the scaled score
    o1, l1 = oracle.attention_fwd(q, k[:1], v[:1], causal=False)
    errs.append(np.max(np.abs(l1 - np.einsum("nhd,hd->hn", q, np.repeat(k[0], 2, axis=0)) / math.sqrt(3))))
    return max(errs)


def pins_bwd_error():
    n, d = 12, 4
    q, k, v = rand(2, (n, 2, d), 1, 0), rand(2, (n, 1, d), 1, 1), rand(2, (n, 1, d), 1, 2)
    do = rand(3, (n, 2, d))
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, causal=True)
    rng = np.random.default_rng(4)
    worst = 0.0
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        u = rng.standard_normal(x.shape)
        a = {"q": q, "k": k, "v": v}
        a[name] = x + 1e-6 * u
        lp = np.sum(oracle.attention_fwd(a["q"], a["k"], a["v"], causal=True)[0] * do)
        a[name] = x - 1e-6 * u
        lm = np.sum(oracle.attention_fwd(a["q"], a["k"], a["v"], causal=True)[0] * do)
        worst = max(worst, abs((lp - lm) / 2e-6 - np.sum(g * u)))
    return worst


def test_unmutated_oracle_passes_the_pins():
    assert pins_fwd_error() < 1e-12
    assert pins_bwd_error() < 1e-6


def _wrong_scale(qh, kg, scale, causal, q_pos, k_pos):
    return _ORIG_SCORES(qh, kg, scale * scale * 2.0, causal, q_pos, k_pos)


def _mask_off_by_one(qh, kg, scale, causal, q_pos, k_pos):
    return _ORIG_SCORES(qh, kg, scale, causal, q_pos - 1, k_pos)


def _transposed_scores(qh, kg, scale, causal, q_pos, k_pos):
    s = (qh @ kg.T) * scale
    s = s[:, ::-1]  # keys in reverse: a mis-indexed operand
    if causal:
        s = np.where(k_pos[None, :] <= q_pos[:, None], s, -np.inf)
    return s


_ORIG_SCORES = dense._scores


@pytest.mark.parametrize("mutant", [_wrong_scale, _mask_off_by_one, _transposed_scores])
def test_forward_mutations_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(dense, "_scores", mutant)
    assert pins_fwd_error() > 1e-6


def test_gqa_head_map_mutation_is_caught(monkeypatch):
    orig = dense.attention_fwd

    def interleaved_map(q, k, v, *, causal, q_pos=None, k_pos=None):
        # wrong grouping: head h uses K/V head h % Hkv instead of h // group
        hq, hkv = q.shape[1], k.shape[1]
        idx = [h % hkv for h in range(hq)]
        return orig(q, k[:, idx], v[:, idx], causal=causal, q_pos=q_pos, k_pos=k_pos)

    monkeypatch.setattr(oracle, "attention_fwd", interleaved_map)
    assert pins_fwd_error() > 1e-6


def test_backward_mutation_dropped_delta_is_caught(monkeypatch):
    orig_sum = np.sum

    def zero_delta(a, axis=None, **kw):
        r = orig_sum(a, axis=axis, **kw)
        if axis == 1 and getattr(a, "ndim", 0) == 2:
            return np.zeros_like(r)   # Delta_i dropped from dS = P (dP - Delta)
        return r

    monkeypatch.setattr(dense.np, "sum", zero_delta)
    try:
        err = pins_bwd_error()
    finally:
        monkeypatch.undo()
    assert err > 1e-4


def pins_keys_error():
    """dK/dV at chosen keys (attention_bwd_keys) against central differences of the dense forward."""
    n, d = 12, 4
    q, k, v = rand(5, (n, 2, d), 1, 0), rand(5, (n, 1, d), 1, 1), rand(5, (n, 1, d), 1, 2)
    do = rand(6, (n, 2, d))
    keys = np.array([0, 5, 11])
    dk, dv = oracle.attention_bwd_keys(q, k, v, do, causal=True, keys=keys)
    rng = np.random.default_rng(7)
    worst = 0.0
    for name, x, g in (("k", k, dk), ("v", v, dv)):
        u = np.zeros_like(x)
        u[keys] = rng.standard_normal((keys.size,) + x.shape[1:])
        a = {"q": q, "k": k, "v": v}
        a[name] = x + 1e-6 * u
        lp = np.sum(oracle.attention_fwd(a["q"], a["k"], a["v"], causal=True)[0] * do)
        a[name] = x - 1e-6 * u
        lm = np.sum(oracle.attention_fwd(a["q"], a["k"], a["v"], causal=True)[0] * do)
        worst = max(worst, abs((lp - lm) / 2e-6 - np.sum(g * u[keys])))
    return worst


def test_chosen_key_backward_pins_pass_unmutated():
    assert pins_keys_error() < 1e-6


def test_chosen_key_backward_mutations_are_caught(monkeypatch):
    # a causal mask shifted by one key in the chosen-key scores only (the forward, which the
    # finite differences differentiate, keeps the right mask; the 3-key calls are the chosen keys)
    def mask_off_by_one_at_chosen_keys(qh, kg, scale, causal, q_pos, k_pos):
        if kg.shape[0] == 3:
            return _ORIG_SCORES(qh, kg, scale, causal, q_pos - 1, k_pos)
        return _ORIG_SCORES(qh, kg, scale, causal, q_pos, k_pos)

    monkeypatch.setattr(dense, "_scores", mask_off_by_one_at_chosen_keys)
    assert pins_keys_error() > 1e-4
    monkeypatch.undo()
    # dS without Delta: the row term of the chosen-key backward dropped
    orig_sum = np.sum

    def zero_delta(a, axis=None, **kw):
        r = orig_sum(a, axis=axis, **kw)
        if axis == 1 and getattr(a, "ndim", 0) == 2:
            return np.zeros_like(r)
        return r

    monkeypatch.setattr(dense.np, "sum", zero_delta)
    try:
        err = pins_keys_error()
    finally:
        monkeypatch.undo()
    assert err > 1e-4
