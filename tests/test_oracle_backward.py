"""Pins of the float64 backward oracle against things other than itself (CPU).

Each expected value comes from something the backward oracle does not use:
central finite differences of the forward oracle, torch's autograd on a dense
float64 attention written here, invariants of the softmax gradient, or the
single-key special case.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import backward as B
from oracle.attention import attention_two_pass
from oracle.pool import OraclePool, write_kv


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _fd_grads(Q, K, V, G, scale, pos, causal, eps=1e-6):
    """Central differences of L = sum(O * G) through the forward oracle."""
    def loss(q, k, v):
        o, _ = attention_two_pass(q, k, v, scale, pos, causal)
        return float((o * G).sum())
    out = []
    for X, which in ((Q, 0), (K, 1), (V, 2)):
        g = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            args = [Q.copy(), K.copy(), V.copy()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            dn = loss(*args)
            g[idx] = (up - dn) / (2 * eps)
        out.append(g)
    return out


@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_finite_differences(causal):
    rng = np.random.default_rng(3)
    n_q, n_k, d = 3, 7, 5
    Q, K, V, G = _rand(rng, n_q, d), _rand(rng, n_k, d), _rand(rng, n_k, d), _rand(rng, n_q, d)
    pos = np.array([4, 5, 6])           # a chunk at the end of a 7-token context
    scale = 0.37
    dq, dk, dv = B.attention_backward_dense(Q, K, V, G, scale, pos, causal)
    fq, fk, fv = _fd_grads(Q, K, V, G, scale, pos, causal)
    for a, f in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.abs(a - f).max() < 1e-8


@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_torch_autograd(causal):
    rng = np.random.default_rng(4)
    n_q, n_k, d = 20, 45, 16
    Q, K, V, G = _rand(rng, n_q, d), _rand(rng, n_k, d), _rand(rng, n_k, d), _rand(rng, n_q, d)
    pos = np.arange(n_k - n_q, n_k)
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv = B.attention_backward_dense(Q, K, V, G, scale, pos, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    s = scale * tq @ tk.T
    if causal:
        mask = torch.arange(n_k).view(1, -1) > torch.tensor(pos).view(-1, 1)
        s = s.masked_fill(mask, float("-inf"))
    o = torch.softmax(s, dim=1) @ tv
    (o * torch.tensor(G)).sum().backward()
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(a - t.grad.numpy()).max() < 1e-11


def test_backward_invariants():
    """Rows of dS sum to zero, so the key gradients of one query head sum to
    zero; rows of P sum to one, so the value gradients sum to the summed dO.
    With one key, P = 1: no gradient reaches Q or K and dV is the summed dO."""
    rng = np.random.default_rng(5)
    n_q, n_k, d = 9, 30, 8
    Q, K, V, G = _rand(rng, n_q, d), _rand(rng, n_k, d), _rand(rng, n_k, d), _rand(rng, n_q, d)
    pos = np.arange(n_k - n_q, n_k)
    dq, dk, dv = B.attention_backward_dense(Q, K, V, G, 0.3, pos, True)
    assert np.abs(dk.sum(axis=0)).max() < 1e-12
    assert np.abs(dv.sum(axis=0) - G.sum(axis=0)).max() < 1e-12
    dq1, dk1, dv1 = B.attention_backward_dense(Q[:1], K[:1], V[:1], G[:1], 0.3, [0], True)
    assert np.abs(dq1).max() == 0 and np.abs(dk1).max() == 0
    assert np.abs(dv1 - G[:1]).max() == 0


def _src_tokens(wl, b):
    start = sum(wl.ctx_lens[:b])
    return (wl.k_src[start:start + wl.ctx_lens[b]].to(torch.float64).numpy(),
            wl.v_src[start:start + wl.ctx_lens[b]].to(torch.float64).numpy())


def test_paged_backward_scatters_into_the_pool_layouts():
    """The paged call equals the dense backward of each sequence's own tokens
    (taken from the write order, bypassing pool and table), summed over the
    query heads of a KV head and placed at (physical page, slot) -- K token-major,
    V feature-major; untouched pages stay zero."""
    wl = workloads.small("prefill", kv_dtype="f32", q_dtype="f32", num_q_heads=4,
                         num_kv_heads=2, head_dim=8, ctx_lens=(37, 20), q_lens=(5, 20), seed=9)
    pool = OraclePool(wl.num_blocks, 2, 8, "f32")
    write_kv(pool, wl.k_src, wl.v_src, wl.slot_mapping)
    call = wl.calls[0]
    rng = np.random.default_rng(6)
    do = rng.standard_normal(tuple(call.q.shape))
    dq, dk, dv = B.paged_attention_backward(pool, call.q, do, call.cu_q_lens, call.ctx_lens,
                                            call.block_table, 4, wl.scale, True)
    cu = call.cu_q_lens.tolist()
    touched = set()
    for b in range(2):
        K, V = _src_tokens(wl, b)
        c, n_q = wl.ctx_lens[b], cu[b + 1] - cu[b]
        pos = np.arange(c - n_q, c)
        for g in range(2):
            dks, dvs = np.zeros((c, 8)), np.zeros((c, 8))
            for h in (2 * g, 2 * g + 1):
                q = call.q[cu[b]:cu[b + 1], h].to(torch.float64).numpy()
                a, k_, v_ = B.attention_backward_dense(q, K[:, g], V[:, g],
                                                       do[cu[b]:cu[b + 1], h], wl.scale, pos)
                assert np.abs(dq[cu[b]:cu[b + 1], h] - a).max() < 1e-12
                dks += k_
                dvs += v_
            for t in range(c):
                p = int(call.block_table[b, t // 16])
                touched.add(p)
                assert np.abs(dk[p, g, t % 16] - dks[t]).max() < 1e-12
                assert np.abs(dv[p, g, :, t % 16] - dvs[t]).max() < 1e-12
    for p in range(wl.num_blocks):
        if p not in touched:
            assert not dk[p].any() and not dv[p].any()


def test_backward_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the backward oracle (on the CPU) and check
    that a pin above fails for each: the softmax row term dropped, the scale
    left off dK, and dV taken from O instead of dO."""
    real = B.attention_backward_dense

    def fd_fails():
        try:
            test_backward_matches_finite_differences(True)
        except AssertionError:
            return True
        return False

    def no_row_term(Q, K, V, dO, scale, positions=None, causal=True):
        _, _, P = attention_two_pass(Q, K, V, scale, positions, causal, return_probs=True)
        dS = P * (dO @ np.asarray(V).T)
        return scale * dS @ K, scale * dS.T @ Q, P.T @ dO

    def unscaled_dk(*a, **k):
        dq, dk, dv = real(*a, **k)
        return dq, dk / a[4], dv

    def dv_from_o(Q, K, V, dO, scale, positions=None, causal=True):
        dq, dk, _ = real(Q, K, V, dO, scale, positions, causal)
        O, _, P = attention_two_pass(Q, K, V, scale, positions, causal, return_probs=True)
        return dq, dk, P.T @ O

    for wrong in (no_row_term, unscaled_dk, dv_from_o):
        monkeypatch.setattr(B, "attention_backward_dense", wrong)
        assert fd_fails(), wrong.__name__
    monkeypatch.setattr(B, "attention_backward_dense", real)
    assert not fd_fails()
