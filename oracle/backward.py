"""Plain float64 attention backward over the oracle's pool (test infrastructure only).

The FlashAttention page (core-principle section, and its recomputation point)
says the backward pass rebuilds the attention weights from the kept output and
statistics instead of storing the n x n matrix; it gives no formulas.  What
any such backward must produce is the gradient of the forward's definition, so
the oracle is that gradient written out with the full probability matrix P
(no recomputation, no tiling):

  S = scale * Q K^T, masked like the forward;  P = softmax(S) row by row
  O = P V
  dV = P^T dO
  dP = dO V^T
  dS = P * (dP - rowsum(P * dP))        (softmax Jacobian, row by row)
  dQ = scale * dS K
  dK = scale * dS^T Q

Masked entries have P = 0 and pass no gradient; a row with no visible key has
P = 0 everywhere.  For a paged call, dK and dV of a KV head sum over its G
query heads and over every query row that sees the key, and are returned in
the pool's layouts (dK [NB, Hkv, 16, d], dV [NB, Hkv, d, 16]); a physical page
used by several sequences gets the sum of their contributions, pages no
sequence uses stay zero.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, attention_two_pass
from .pool import BLOCK, OraclePool, gather_kv


def attention_backward_dense(Q, K, V, dO, scale: float, positions=None, causal: bool = True):
    """Q, dO [n_q, d]; K, V [n_k, d].  Returns dQ [n_q, d], dK [n_k, d], dV [n_k, d]."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    _, _, P = attention_two_pass(Q, K, V, scale, positions, causal, return_probs=True)
    dV = P.T @ dO
    dP = dO @ V.T
    row = (P * dP).sum(axis=1, keepdims=True)
    dS = P * (dP - row)
    dQ = scale * (dS @ K)
    dK = scale * (dS.T @ Q)
    return dQ, dK, dV


def paged_attention_backward(pool: OraclePool, q, do, cu_q_lens, ctx_lens, block_table,
                             num_q_heads: int, scale: float, causal: bool = True):
    """Whole call: q, do [T, Hq, d] -> dQ [T, Hq, d], dK [NB, Hkv, 16, d],
    dV [NB, Hkv, d, 16] (float64).  Queries align to the end of the context,
    as in the forward."""
    qf, dof = _f64(q), _f64(do)
    T, Hq, d = qf.shape
    Hkv = pool.num_kv_heads
    G = num_q_heads // Hkv
    cu = np.asarray(cu_q_lens).astype(np.int64)
    ctx = np.asarray(ctx_lens).astype(np.int64)
    bt = np.asarray(block_table)
    dQ = np.zeros((T, Hq, d))
    dK = np.zeros((pool.num_blocks, Hkv, BLOCK, d))
    dV = np.zeros((pool.num_blocks, Hkv, d, BLOCK))
    for b in range(len(ctx)):
        q0, q1 = cu[b], cu[b + 1]
        n_q, c = q1 - q0, int(ctx[b])
        pos = c - n_q + np.arange(n_q)
        for g in range(Hkv):
            K, V = gather_kv(pool, bt[b], c, g)
            dk_seq = np.zeros((c, d))
            dv_seq = np.zeros((c, d))
            for h in range(g * G, (g + 1) * G):
                dq, dk, dv = attention_backward_dense(qf[q0:q1, h], K, V, dof[q0:q1, h], scale,
                                                      pos, causal)
                dQ[q0:q1, h] = dq
                dk_seq += dk
                dv_seq += dv
            for t in range(c):
                page, slot = int(bt[b][t // BLOCK]), t % BLOCK
                dK[page, g, slot, :] += dk_seq[t]
                dV[page, g, :, slot] += dv_seq[t]
    return dQ, dK, dV
