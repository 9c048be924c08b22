"""Pins of the float64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: brute force, a closed form, a
library routine in a special case, an invariant the pages state, or the fp8
format's bit definition.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import fp8_e4m3
from oracle.pool import OraclePool, write_kv, gather_kv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pool_for(wl):
    p = OraclePool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
    write_kv(p, wl.k_src, wl.v_src, wl.slot_mapping)
    return p


def _run(wl, call, pool=None, causal=True):
    pool = pool or _pool_for(wl)
    return oracle.paged_attention(pool, call.q, call.cu_q_lens, call.ctx_lens,
                                  call.block_table, wl.num_q_heads, wl.scale, causal)


def _src_tokens(wl, b):
    """Logical tokens of sequence b straight from the written-token order
    (no prefix sharing): the pool and block table are bypassed."""
    assert wl.shared_prefix == 0
    start = sum(wl.ctx_lens[:b])
    k = wl.k_src[start:start + wl.ctx_lens[b]].to(torch.float64)
    v = wl.v_src[start:start + wl.ctx_lens[b]].to(torch.float64)
    return k, v


# ---------------------------------------------------------------- P-a brute force
def test_brute_force_tiny():
    """Per-element pure-Python sums on tiny inputs (3 pages, d=4, 2 q heads
    sharing 1 KV head), read straight from the token order."""
    wl = workloads.small("prefill", kv_dtype="f32", q_dtype="f32", num_q_heads=2,
                         num_kv_heads=1, head_dim=4, ctx_lens=(40, 7),
                         q_lens=(5, 7), seed=3)
    call = wl.calls[0]
    O, L = _run(wl, call)
    q = call.q.to(torch.float64).tolist()
    cu = call.cu_q_lens.tolist()
    for b in range(2):
        k, v = _src_tokens(wl, b)
        k, v = k.tolist(), v.tolist()
        n_q, ctx = cu[b + 1] - cu[b], wl.ctx_lens[b]
        for i in range(n_q):
            pos = ctx - n_q + i
            for h in range(2):
                qi = q[cu[b] + i][h]
                s = [wl.scale * sum(qi[c] * k[t][0][c] for c in range(4)) for t in range(pos + 1)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                den = sum(e)
                for c in range(4):
                    num = sum(e[t] * v[t][0][c] for t in range(pos + 1))
                    assert abs(O[cu[b] + i, h, c] - num / den) < 1e-12
                assert abs(L[cu[b] + i, h] - (m + math.log(den))) < 1e-12


def test_golden_two_keys():
    """Hand-derived closed form stored under tests/golden."""
    with open(os.path.join(GOLDEN, "two_keys_closed_form.json")) as f:
        g = json.load(f)
    wl = workloads.small("prefill", kv_dtype="f32", q_dtype="f32", num_q_heads=1,
                         num_kv_heads=1, head_dim=4, ctx_lens=(2,), seed=0)
    wl.k_src = torch.tensor(g["k"], dtype=torch.float32).reshape(2, 1, 4)
    wl.v_src = torch.tensor(g["v"], dtype=torch.float32).reshape(2, 1, 4)
    wl.calls[0].q = torch.tensor(g["q"], dtype=torch.float32).reshape(2, 1, 4)
    wl.scale = g["scale"]
    O, L = _run(wl, wl.calls[0])
    # q holds 2 ln 2 rounded to float32 (relative error <= 2^-24), which moves
    # the score by < 5e-8 and the outputs by less than 1e-7.
    np.testing.assert_allclose(O[:, 0], np.array(g["expected_o"]), rtol=0, atol=1e-7)
    np.testing.assert_allclose(L[:, 0], np.array(g["expected_lse"]), rtol=0, atol=1e-7)
    assert O[0, 0].tolist() == g["expected_o"][0] and L[0, 0] == g["expected_lse"][0]


# ---------------------------------------------------------------- P-b, P-c
def test_rows_sum_to_one():
    rng = np.random.default_rng(0)
    Q, K, V = rng.standard_normal((50, 16)), rng.standard_normal((70, 16)), rng.standard_normal((70, 16))
    pos = 20 + np.arange(50)
    _, _, P = oracle.attention_two_pass(Q, K, V, 0.25, pos, True, return_probs=True)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
    assert (P[np.arange(70)[None, :] > pos[:, None]] == 0).all()


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "fp8"])
def test_constant_v(kv_dtype):
    """V identical for every token -> every output row equals that constant."""
    wl = workloads.small("prefill", kv_dtype=kv_dtype, q_dtype="f32" if kv_dtype == "f32" else "bf16",
                         num_q_heads=4, num_kv_heads=2, head_dim=8, ctx_lens=(33, 50),
                         q_lens=(9, 50), seed=5)
    c = torch.linspace(-2.0, 2.0, 8)
    wl.v_src = c.reshape(1, 1, 8).expand_as(wl.v_src).contiguous().to(wl.v_src.dtype)
    O, _ = _run(wl, wl.calls[0])
    expect = wl.v_src[0, 0].to(torch.float64).numpy()
    if kv_dtype == "fp8":   # the constant itself goes through the fp8 code
        pool = _pool_for(wl)
        _, V = gather_kv(pool, wl.block_tables[0], 33, 0)
        expect = V[0]
    np.testing.assert_allclose(O, np.broadcast_to(expect, O.shape), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P-d
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_block_permutation_invariance(kv_dtype):
    """Relabel every physical page (pool bytes moved, table remapped): identical output."""
    wl = workloads.small("prefill", kv_dtype=kv_dtype, num_q_heads=4, num_kv_heads=2,
                         head_dim=16, ctx_lens=(70, 20, 45), q_lens=(70, 5, 1), seed=11)
    call = wl.calls[0]
    O1, L1 = _run(wl, call)
    perm = torch.randperm(wl.num_blocks, generator=torch.Generator().manual_seed(99)).to(torch.int32)
    wl.slot_mapping = perm[(wl.slot_mapping // 16).long()] * 16 + wl.slot_mapping % 16
    bt = call.block_table.clone()
    bt[bt >= 0] = perm[bt[bt >= 0].long()]
    call.block_table = bt
    O2, L2 = _run(wl, call)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


# ---------------------------------------------------------------- P-e
def test_causal_first_row_returns_v0():
    wl = workloads.small("prefill", kv_dtype="f32", q_dtype="f32", num_q_heads=2,
                         num_kv_heads=1, head_dim=64, ctx_lens=(48,), seed=2)
    call = wl.calls[0]
    O, L = _run(wl, call)
    k, v = _src_tokens(wl, 0)
    for h in range(2):
        assert np.array_equal(O[0, h], v[0, 0].numpy())
        q0 = call.q[0, h].to(torch.float64)
        assert abs(L[0, h] - wl.scale * float(q0 @ k[0, 0])) < 1e-12


# ---------------------------------------------------------------- P-f
@pytest.mark.parametrize("chunk", [False, True])
def test_matches_torch_sdpa(chunk):
    """Library special case: PyTorch's CPU scaled_dot_product_attention in float64
    (is_causal for a full prefill; an explicit bottom-right mask for a chunk)."""
    ctx = 77
    n_q = 21 if chunk else ctx
    wl = workloads.small("prefill", kv_dtype="bf16", num_q_heads=6, num_kv_heads=2,
                         head_dim=32, ctx_lens=(ctx,), q_lens=(n_q,), seed=13)
    call = wl.calls[0]
    O, _ = _run(wl, call)
    k, v = _src_tokens(wl, 0)
    q = call.q.to(torch.float64).permute(1, 0, 2)                 # [Hq, n_q, d]
    kk = k.permute(1, 0, 2).repeat_interleave(3, dim=0)           # [Hq, ctx, d]
    vv = v.permute(1, 0, 2).repeat_interleave(3, dim=0)
    if chunk:
        pos = ctx - n_q + torch.arange(n_q)
        mask = torch.arange(ctx)[None, :] <= pos[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, attn_mask=mask, scale=wl.scale)
    else:
        ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True, scale=wl.scale)
    np.testing.assert_allclose(O, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_sampled_rows_match_torch_sdpa():
    """The row-sampling oracle (used at full sizes) against PyTorch's CPU SDPA in
    float64 on a two-sequence chunked batch, rows drawn from both sequences and
    from heads of different KV groups."""
    wl = workloads.small("prefill", kv_dtype="bf16", num_q_heads=4, num_kv_heads=2,
                         head_dim=32, ctx_lens=(45, 70), q_lens=(45, 19), seed=21)
    call = wl.calls[0]
    pool = _pool_for(wl)
    rows = [(0, 0), (44, 3), (45, 1), (50, 2), (63, 3)]
    O, L = oracle.paged_attention_rows(pool, call.q, call.cu_q_lens, call.ctx_lens,
                                       call.block_table, wl.num_q_heads, wl.scale, rows)
    cu = [0, 45, 64]
    for n, (t, h) in enumerate(rows):
        b = 0 if t < 45 else 1
        k, v = _src_tokens(wl, b)
        ctx, n_q = wl.ctx_lens[b], cu[b + 1] - cu[b]
        pos = ctx - n_q + (t - cu[b])
        q = call.q[t, h].to(torch.float64)[None, None]            # [1, 1, d]
        kk, vv = k[:, h // 2][None], v[:, h // 2][None]           # [1, ctx, d]
        mask = (torch.arange(ctx) <= pos)[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, attn_mask=mask, scale=wl.scale)
        np.testing.assert_allclose(O[n], ref[0, 0].numpy(), rtol=0, atol=1e-12)
        s = wl.scale * (k[: pos + 1, h // 2] @ call.q[t, h].to(torch.float64))
        assert abs(L[n] - float(torch.logsumexp(s, 0))) < 1e-12


# ---------------------------------------------------------------- P-g
def test_zero_query_gives_mean_of_visible_v():
    rng = np.random.default_rng(1)
    K, V = rng.standard_normal((40, 8)), rng.standard_normal((40, 8))
    pos = np.array([0, 5, 17, 39])
    O, L = oracle.attention_two_pass(np.zeros((4, 8)), K, V, 0.3, pos, True)
    for i, p in enumerate(pos):
        np.testing.assert_allclose(O[i], V[: p + 1].mean(axis=0), atol=1e-13)
        assert abs(L[i] - math.log(p + 1)) < 1e-13


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(2)
    q = rng.standard_normal(8)
    K, V = rng.standard_normal((30, 8)) * 0.01, rng.standard_normal((30, 8))
    K[12] = 400.0 * q
    O, _ = oracle.attention_two_pass(q[None], K, V, 1.0, [29], True)
    np.testing.assert_allclose(O[0], V[12], atol=1e-12)


def test_no_visible_key_gives_zero_and_minus_inf():
    O, L = oracle.attention_two_pass(np.ones((1, 4)), np.ones((0, 4)), np.ones((0, 4)), 1.0, [0], False)
    assert (O == 0).all() and L[0] == -np.inf


# ---------------------------------------------------------------- P-h
def test_online_recurrence_equals_two_pass():
    """The running-max / running-sum recurrence over 16-token pages equals the
    one-shot softmax (the "core modules" chapter, section 2.1, design two)."""
    rng = np.random.default_rng(3)
    K, V = rng.standard_normal((203, 32)) * 2, rng.standard_normal((203, 32))
    for n_vis in (1, 16, 17, 100, 203):
        q = rng.standard_normal(32) * 3
        o1, l1 = oracle.online_softmax_pages(q, K, V, 0.2, 16, n_vis)
        o2, l2 = oracle.attention_two_pass(q[None], K[:n_vis], V[:n_vis], 0.2, [n_vis - 1], True)
        np.testing.assert_allclose(o1, o2[0], atol=1e-12)
        assert abs(l1 - l2[0]) < 1e-12


# ---------------------------------------------------------------- P-i
def test_lse_merge_of_page_aligned_splits():
    rng = np.random.default_rng(4)
    K, V = rng.standard_normal((300, 16)), rng.standard_normal((300, 16))
    q = rng.standard_normal(16) * 2
    o_ref, l_ref = oracle.attention_two_pass(q[None], K, V, 0.25, [299], True)
    for cuts in ([0, 300], [0, 16, 300], [0, 48, 160, 176, 300], [0, 300, 300, 300]):
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            o, l = oracle.attention_two_pass(q[None], K[a:b], V[a:b], 0.25, [b - a - 1], False)
            parts.append((o[0], l[0]))
        o, l = oracle.lse_merge(parts)
        np.testing.assert_allclose(o, o_ref[0], atol=1e-12)
        assert abs(l - l_ref[0]) < 1e-12
    o, l = oracle.lse_merge([(np.zeros(16), -np.inf)] * 3)
    assert (o == 0).all() and l == -np.inf


# ---------------------------------------------------------------- gather
def test_gather_follows_block_table_and_prefix_sharing():
    """Sequences sharing prefix pages read the same bytes; each page holds the
    16 consecutive logical tokens its table entry names."""
    wl = workloads.build("t", kv_dtype="bf16", q_dtype="bf16", num_q_heads=2, num_kv_heads=2,
                         head_dim=8, ctx_lens=[64, 50, 40], shared_prefix=32,
                         calls=[workloads.Call("decode", [0, 1, 2], [1, 1, 1])], seed=21)
    pool = _pool_for(wl)
    k0, v0 = gather_kv(pool, wl.block_tables[0], 64, 1)
    k1, v1 = gather_kv(pool, wl.block_tables[1], 50, 1)
    assert np.array_equal(k0[:32], k1[:32]) and np.array_equal(v0[:32], v1[:32])
    src = wl.k_src.to(torch.float64).numpy()
    np.testing.assert_array_equal(k0[:32], src[:32, 1])
    np.testing.assert_array_equal(k0[32:], src[32:64, 1])
    np.testing.assert_array_equal(k1[32:], src[64:82, 1])
    # pages nobody wrote are still NaN
    used = set(wl.block_tables[wl.block_tables >= 0].tolist())
    spare = [p for p in range(wl.num_blocks) if p not in used]
    assert len(spare) == 8
    assert (pool.k[spare] == 0x7FC0).all()


# ---------------------------------------------------------------- P-l fp8 codec
def test_fp8_decode_table_matches_torch_float8():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = fp8_e4m3.decode_table()
    nan = np.isnan(t)
    assert (nan == np.isnan(mine)).all() and nan.sum() == 2
    assert np.array_equal(t[~nan], mine[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_fp8_encode_round_to_nearest_even():
    vals = fp8_e4m3.decode_table()[:0x7F]
    # every representable value encodes to itself, both signs
    assert np.array_equal(fp8_e4m3.encode_rne(vals), np.arange(0x7F, dtype=np.uint8))
    assert np.array_equal(fp8_e4m3.encode_rne(-vals[1:]), np.arange(1, 0x7F, dtype=np.uint8) | 0x80)
    # midpoints go to the even code
    mids = (vals[:-1] + vals[1:]) / 2
    codes = fp8_e4m3.encode_rne(mids)
    lo = np.arange(0x7E)
    assert np.array_equal(codes, np.where(lo % 2 == 0, lo, lo + 1))
    # random values agree with torch's (round-to-nearest-even) cast inside the range
    x = np.random.default_rng(5).standard_normal(100000) * 60
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8_e4m3.encode_rne(x), ref)
    assert fp8_e4m3.encode_rne(np.array([-0.0]))[0] == 0x80


def test_fp8_page_quantisation_scale():
    wl = workloads.small("decode", kv_dtype="fp8", num_q_heads=2, num_kv_heads=2,
                         head_dim=16, ctx_lens=(32,), seed=8)
    pool = _pool_for(wl)
    src = wl.k_src.to(torch.float32).numpy()
    for j in range(2):
        p = int(wl.block_tables[0, j])
        amax = np.float32(np.abs(src[16 * j:16 * j + 16]).max())
        assert pool.k_scale[p] == np.float32(amax / np.float32(448))
        assert (np.abs(fp8_e4m3.decode(pool.k[p])) <= 448).all()
        assert (pool.k[p] & 0x7F == 0x7E).sum() >= 1          # amax lands on +-448
        deq = fp8_e4m3.decode(pool.k[p]) * np.float64(pool.k_scale[p])
        # worst case is half an E4M3 step in the top binade [256, 448], i.e. 16
        # code units of size amax/448, plus float32 rounding of x / scale
        err = np.abs(deq - src[16 * j:16 * j + 16].transpose(1, 0, 2))
        assert err.max() <= amax * 16.0 / 448.0 * (1 + 1e-6)


# ---------------------------------------------------------------- pins have teeth
def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle (on the CPU) and check that a pin
    above fails for each: a dropped scale, top-left causal alignment, and K/V
    swapped in the gather."""
    from oracle import attention as A

    def sdpa_fails():
        try:
            test_matches_torch_sdpa(True)
        except AssertionError:
            return True
        return False

    real = A.attention_two_pass
    monkeypatch.setattr(A, "attention_two_pass",
                        lambda Q, K, V, scale, *a, **k: real(Q, K, V, 1.0, *a, **k))
    assert sdpa_fails()
    monkeypatch.setattr(A, "attention_two_pass",
                        lambda Q, K, V, scale, positions=None, causal=True, **k:
                        real(Q, K, V, scale, np.arange(len(positions)), causal, **k))
    assert sdpa_fails()
    monkeypatch.setattr(A, "attention_two_pass", real)
    real_gather = A.gather_kv
    monkeypatch.setattr(A, "gather_kv", lambda *a: real_gather(*a)[::-1])
    assert sdpa_fails()
    monkeypatch.setattr(A, "gather_kv", real_gather)
    assert not sdpa_fails()
