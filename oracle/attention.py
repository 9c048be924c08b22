"""Plain float64 attention forward over the oracle's pool (test infrastructure only).

Definition followed (FlashAttention page, section 1: scaled dot-product
self-attention, where the extracted text lost the formula and keeps only "d_k
is the feature dimension"; read as softmax(Q K^T / sqrt(d_k)) V with the scale
a parameter):

  S[i, t] = scale * sum_c Q[i, c] K[t, c]                 (full score matrix)
  S[i, t] = -inf  where t > pos_i  (causal; pos_i = ctx - q_len + i)
  m_i = max_t S[i, t];  E = exp(S - m_i);  l_i = sum_t E   (safe softmax, the
        same page's core-principle section)
  P = E / l_i;  O = P V;  LSE_i = m_i + ln l_i

A row with no visible key has O = 0 and LSE = -inf.  Chunked queries align to
the end of the context (bottom-right), the reading the pages leave open.

``online_softmax_pages`` restates the "core modules" chapter, section 2.1
design two (running max m and exp-sum l, correcting the accumulated O as each
new K block arrives); it exists only so the tests can pin that recurrence
against the two-pass definition.  ``lse_merge`` combines partial results of
disjoint key ranges from their logsumexps.
"""
from __future__ import annotations

import numpy as np
import torch

from .pool import OraclePool, gather_kv


def _f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def attention_two_pass(Q, K, V, scale: float, positions=None, causal: bool = True,
                       return_probs: bool = False):
    """Q [n_q, d], K/V [n_k, d] (float64); positions[i] is query i's position.
    Returns O [n_q, d], LSE [n_q] (and P [n_q, n_k] on request)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    n_q, n_k = Q.shape[0], K.shape[0]
    S = scale * (Q @ K.T)
    if causal:
        pos = np.asarray(positions, dtype=np.int64).reshape(n_q, 1)
        S = np.where(np.arange(n_k).reshape(1, n_k) > pos, -np.inf, S)
    m = S.max(axis=1, keepdims=True) if n_k else np.full((n_q, 1), -np.inf)
    empty = ~np.isfinite(m[:, 0])
    m_safe = np.where(np.isfinite(m), m, 0.0)
    E = np.exp(S - m_safe)
    l = E.sum(axis=1, keepdims=True)
    P = np.divide(E, l, out=np.zeros_like(E), where=l > 0)
    O = P @ V
    with np.errstate(divide="ignore"):
        lse = (m_safe + np.log(l))[:, 0]
    O[empty] = 0.0
    lse[empty] = -np.inf
    return (O, lse, P) if return_probs else (O, lse)


def paged_attention(pool: OraclePool, q, cu_q_lens, ctx_lens, block_table,
                    num_q_heads: int, scale: float, causal: bool = True):
    """Whole call: q [T, Hq, d] -> O [T, Hq, d], LSE [T, Hq] (float64).
    Query head h reads KV head h // (Hq / Hkv)."""
    qf = _f64(q)
    T, Hq, d = qf.shape
    G = num_q_heads // pool.num_kv_heads
    cu = np.asarray(cu_q_lens).astype(np.int64)
    ctx = np.asarray(ctx_lens).astype(np.int64)
    bt = np.asarray(block_table)
    O = np.zeros((T, Hq, d))
    LSE = np.full((T, Hq), -np.inf)
    for b in range(len(ctx)):
        q0, q1 = cu[b], cu[b + 1]
        n_q, c = q1 - q0, ctx[b]
        pos = c - n_q + np.arange(n_q)
        for g in range(pool.num_kv_heads):
            K, V = gather_kv(pool, bt[b], int(c), g)
            for h in range(g * G, (g + 1) * G):
                o, lse = attention_two_pass(qf[q0:q1, h], K, V, scale, pos, causal)
                O[q0:q1, h] = o
                LSE[q0:q1, h] = lse
    return O, LSE


def paged_attention_rows(pool: OraclePool, q, cu_q_lens, ctx_lens, block_table,
                         num_q_heads: int, scale: float, rows, causal: bool = True):
    """Only the listed (query token index, q head) rows: O [n, d], LSE [n]."""
    G = num_q_heads // pool.num_kv_heads
    cu = np.asarray(cu_q_lens).astype(np.int64)
    ctx = np.asarray(ctx_lens).astype(np.int64)
    bt = np.asarray(block_table)
    out_o, out_l = [], []
    cache = {}
    for (t, h) in rows:
        b = int(np.searchsorted(cu, t, side="right") - 1)
        pos = ctx[b] - (cu[b + 1] - cu[b]) + (t - cu[b])
        g = h // G
        if (b, g) not in cache:
            cache = {(b, g): gather_kv(pool, bt[b], int(ctx[b]), g)}
        K, V = cache[(b, g)]
        qrow = _f64(q[t, h]).reshape(1, -1)
        o, lse = attention_two_pass(qrow, K, V, scale, [pos], causal)
        out_o.append(o[0])
        out_l.append(lse[0])
    return np.stack(out_o), np.array(out_l)


def online_softmax_pages(q, K, V, scale: float, page: int = 16, n_visible=None):
    """One query row, keys visited one page at a time in logical order with a
    running max m, running exp-sum l and an unnormalised accumulator,
    rescaled by exp(m_old - m_new) whenever the max grows; divided by l at
    the end.  Returns (O [d], LSE)."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    n = K.shape[0] if n_visible is None else n_visible
    m, l = -np.inf, 0.0
    acc = np.zeros(V.shape[1])
    for j0 in range(0, n, page):
        s = scale * (K[j0:min(n, j0 + page)] @ q)
        m_new = max(m, s.max())
        alpha = np.exp(m - m_new) if np.isfinite(m) else 0.0
        p = np.exp(s - m_new)
        l = alpha * l + p.sum()
        acc = alpha * acc + p @ V[j0:min(n, j0 + page)]
        m = m_new
    if l == 0:
        return np.zeros(V.shape[1]), -np.inf
    return acc / l, m + np.log(l)


def lse_merge(parts):
    """parts: list of (o_s [d] normalised over its own key range, lse_s).
    Empty ranges carry lse_s = -inf and weight 0."""
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    if not np.isfinite(lses).any():
        return np.zeros_like(_f64(parts[0][0])), -np.inf
    M = lses[np.isfinite(lses)].max()
    w = np.where(np.isfinite(lses), np.exp(lses - M), 0.0)
    lse = M + np.log(w.sum())
    o = np.zeros_like(_f64(parts[0][0]))
    for (os_, ls), wi in zip(parts, w):
        if wi > 0:
            o = o + np.exp(ls - lse) * _f64(os_)
    return o, lse
