"""Dense fp64 attention: the plain definition the ring step must reproduce exactly.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

The method is exact attention ("什么是环形注意力（Ring Attention）？", aiboss88 wiki,
"边界与常见误解": no approximation; close-reading notes on "Ring Attention with
Blockwise Transformers for Near-Infinite Context", §3.5: after a full turn of the
ring every query block has met every key/value block).  So the oracle for a
rank's share is the textbook definition, per query head h:

    S = Q_h K_g^T / sqrt(d)            g = h // (Hq / Hkv)   (grouped K/V heads)
    P = softmax over the visible keys of each row (causal: key pos <= query pos)
    O = P V_g,   lse = log sum_t exp(S_t)   (natural log)

computed in float64 with a two-pass softmax (row max, then the sum).  The
backward is the analytic gradient of L = sum(O * dO):

    dV = P^T dO,  dP = dO V^T,  Delta_i = sum_t P_it dP_it (= dO_i . O_i),
    dS = P * (dP - Delta),  dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),

with dK, dV of a shared K/V head summed over the query heads of its group.

Readings taken where the pages are silent: scale 1/sqrt(d); causal mask on
global positions with the diagonal included; grouped heads are contiguous
(head h uses K/V head h // (Hq/Hkv)); a row with no visible key has
lse = -inf and output 0.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

_ROW_CHUNK_BYTES = 256 << 20  # bound the fp64 score chunk to ~256 MB


def positions_for_block(block: int, block_len: int) -> np.ndarray:
    """Global sequence positions of the tokens in sequence block ``block``."""
    return np.arange(block * block_len, (block + 1) * block_len, dtype=np.int64)


def _row_chunk(n_keys: int) -> int:
    return max(1, min(4096, _ROW_CHUNK_BYTES // (8 * max(1, n_keys))))


def _scores(qh: np.ndarray, kg: np.ndarray, scale: float, causal: bool,
            q_pos: np.ndarray, k_pos: np.ndarray) -> np.ndarray:
    s = qh @ kg.T
    s *= scale
    if causal and s.size:
        # keys at or before the chunk's first query position are visible to every row,
        # so only the other columns need the per-element test (same values, less work)
        cols = np.nonzero(k_pos > q_pos.min())[0]
        if cols.size:
            s[:, cols] = np.where(k_pos[cols][None, :] <= q_pos[:, None], s[:, cols], -np.inf)
    return s


def _softmax_rows(s: np.ndarray):
    """Two-pass softmax over rows, in place on ``s``; returns (P, lse). Empty rows give
    P = 0, lse = -inf."""
    m = s.max(axis=1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    s -= m_safe[:, None]
    p = np.exp(s, out=s)                     # exp(-inf) = 0 for masked entries
    l = p.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(finite, m_safe + np.log(np.where(finite, l, 1.0)), -np.inf)
    p /= np.where(finite, l, 1.0)[:, None]   # an empty row is all zeros already
    return p, lse


def _visible_prefix(causal: bool, q_pos_chunk: np.ndarray, k_pos: np.ndarray) -> int:
    """Number of leading keys that can be visible to a row chunk.

    With a causal mask a row only sums over keys at positions <= its own
    (the definition's visible set), so keys past the chunk's last position
    contribute exact zeros and are left out.  Requires sorted key positions;
    otherwise every key is kept.
    """
    m = k_pos.shape[0]
    if not causal or m == 0 or np.any(np.diff(k_pos) < 0):
        return m
    return int(np.searchsorted(k_pos, q_pos_chunk.max(), side="right"))


def _defaults(n: int, m: int, q_pos, k_pos):
    if q_pos is None:
        q_pos = np.arange(n, dtype=np.int64)
    if k_pos is None:
        k_pos = np.arange(m, dtype=np.int64)
    return np.asarray(q_pos, dtype=np.int64), np.asarray(k_pos, dtype=np.int64)


def attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool,
                  q_pos: Optional[np.ndarray] = None, k_pos: Optional[np.ndarray] = None
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention of ``q [n, Hq, d]`` over ``k, v [m, Hkv, d]``.

    Returns ``out [n, Hq, d]`` and ``lse [Hq, n]`` in float64.
    """
    n, hq, d = q.shape
    m, hkv, dk = k.shape
    assert dk == d and v.shape == k.shape and hq % hkv == 0
    q_pos, k_pos = _defaults(n, m, q_pos, k_pos)
    group = hq // hkv
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((n, hq, d), dtype=np.float64)
    lse = np.full((hq, n), -np.inf, dtype=np.float64)
    chunk = _row_chunk(m)
    for h in range(hq):
        g = h // group
        kg = np.asarray(k[:, g, :], dtype=np.float64)
        vg = np.asarray(v[:, g, :], dtype=np.float64)
        for r0 in range(0, n, chunk):
            r1 = min(n, r0 + chunk)
            kv = _visible_prefix(causal, q_pos[r0:r1], k_pos)
            if kv == 0:
                continue  # no visible key: out stays 0, lse stays -inf
            qh = np.asarray(q[r0:r1, h, :], dtype=np.float64)
            s = _scores(qh, kg[:kv], scale, causal, q_pos[r0:r1], k_pos[:kv])
            p, lse[h, r0:r1] = _softmax_rows(s)
            out[r0:r1, h, :] = p @ vg[:kv]
    return out, lse


def sampled_rows_fwd(q_rows: np.ndarray, q_pos_rows: np.ndarray, k: np.ndarray, v: np.ndarray,
                     *, causal: bool, k_pos: Optional[np.ndarray] = None):
    """Exact attention for a chosen subset of query rows at global positions ``q_pos_rows``."""
    return attention_fwd(q_rows, k, v, causal=causal, q_pos=q_pos_rows, k_pos=k_pos)


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, *, causal: bool,
                  q_pos: Optional[np.ndarray] = None, k_pos: Optional[np.ndarray] = None):
    """Analytic fp64 gradients of L = sum(O * dout) with respect to q, k, v.

    Returns ``dq [n, Hq, d]``, ``dk [m, Hkv, d]``, ``dv [m, Hkv, d]``, plus the
    forward ``out`` and ``lse`` for convenience.
    """
    n, hq, d = q.shape
    m, hkv, _ = k.shape
    q_pos, k_pos = _defaults(n, m, q_pos, k_pos)
    group = hq // hkv
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros((n, hq, d), dtype=np.float64)
    dk = np.zeros((m, hkv, d), dtype=np.float64)
    dv = np.zeros((m, hkv, d), dtype=np.float64)
    out = np.zeros((n, hq, d), dtype=np.float64)
    lse = np.full((hq, n), -np.inf, dtype=np.float64)
    chunk = _row_chunk(m)
    for h in range(hq):
        g = h // group
        kg = np.asarray(k[:, g, :], dtype=np.float64)
        vg = np.asarray(v[:, g, :], dtype=np.float64)
        for r0 in range(0, n, chunk):
            r1 = min(n, r0 + chunk)
            kv = _visible_prefix(causal, q_pos[r0:r1], k_pos)
            if kv == 0:
                continue  # no visible key: no output, no gradient
            qh = np.asarray(q[r0:r1, h, :], dtype=np.float64)
            doh = np.asarray(dout[r0:r1, h, :], dtype=np.float64)
            s = _scores(qh, kg[:kv], scale, causal, q_pos[r0:r1], k_pos[:kv])
            p, lse[h, r0:r1] = _softmax_rows(s)
            oh = p @ vg[:kv]
            out[r0:r1, h, :] = oh
            dv[:kv, g, :] += p.T @ doh
            dp = doh @ vg[:kv].T
            delta = np.sum(doh * oh, axis=1)
            ds = p * (dp - delta[:, None])
            dq[r0:r1, h, :] = (ds @ kg[:kv]) * scale
            dk[:kv, g, :] += (ds.T @ qh) * scale
    return dq, dk, dv, out, lse


def attention_bwd_keys(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, *, causal: bool,
                       keys: np.ndarray, q_pos: Optional[np.ndarray] = None,
                       k_pos: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """dK and dV at the chosen key indices ``keys`` only, summed over every query row.

    The same definition as ``attention_bwd`` restricted to a few columns of P:
    every row's output and lse come from its full visible key set (the
    forward above), Delta_i = dO_i . O_i, and then for the chosen keys t only
    P_it = exp(S_it - lse_i), dS_it = P_it (dO_i . v_t - Delta_i),
    dV_t = sum_i P_it dO_i, dK_t = sum_i dS_it q_i / sqrt(d) (summed over the
    query heads of a grouped K/V head).  Returns ``dk, dv [len(keys), Hkv, d]``.
    """
    n, hq, d = q.shape
    m, hkv, _ = k.shape
    q_pos, k_pos = _defaults(n, m, q_pos, k_pos)
    keys = np.asarray(keys, dtype=np.int64)
    group = hq // hkv
    scale = 1.0 / math.sqrt(d)
    out, lse = attention_fwd(q, k, v, causal=causal, q_pos=q_pos, k_pos=k_pos)
    dk = np.zeros((keys.size, hkv, d), dtype=np.float64)
    dv = np.zeros((keys.size, hkv, d), dtype=np.float64)
    chunk = _row_chunk(keys.size)
    for h in range(hq):
        g = h // group
        kt = np.asarray(k[keys, g, :], dtype=np.float64)
        vt = np.asarray(v[keys, g, :], dtype=np.float64)
        for r0 in range(0, n, chunk):
            r1 = min(n, r0 + chunk)
            qh = np.asarray(q[r0:r1, h, :], dtype=np.float64)
            doh = np.asarray(dout[r0:r1, h, :], dtype=np.float64)
            s = _scores(qh, kt, scale, causal, q_pos[r0:r1], k_pos[keys])
            l = lse[h, r0:r1]
            ok = np.isfinite(l)  # rows with no visible key contribute nothing
            p = np.where(ok[:, None], np.exp(s - np.where(ok, l, 0.0)[:, None]), 0.0)
            delta = np.sum(doh * out[r0:r1, h, :], axis=1)
            ds = p * (doh @ vt.T - delta[:, None])
            dv[:, g, :] += p.T @ doh
            dk[:, g, :] += (ds.T @ qh) * scale
    return dk, dv


def brute_force_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool,
                    q_pos=None, k_pos=None):
    """Scalar triple loops with exactly-rounded sums (math.fsum); tiny inputs only."""
    n, hq, d = q.shape
    m, hkv, _ = k.shape
    q_pos, k_pos = _defaults(n, m, q_pos, k_pos)
    group = hq // hkv
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((n, hq, d), dtype=np.float64)
    lse = np.full((hq, n), -np.inf, dtype=np.float64)
    for h in range(hq):
        g = h // group
        for i in range(n):
            keys = [t for t in range(m) if (not causal) or k_pos[t] <= q_pos[i]]
            if not keys:
                continue
            sc = {t: math.fsum(float(q[i, h, e]) * float(k[t, g, e]) for e in range(d)) * scale
                  for t in keys}
            mx = max(sc.values())
            w = {t: math.exp(sc[t] - mx) for t in keys}
            z = math.fsum(w.values())
            lse[h, i] = mx + math.log(z)
            for e in range(d):
                out[i, h, e] = math.fsum(w[t] * float(v[t, g, e]) for t in keys) / z
    return out, lse
