"""Block management on the host (no GPU): the oracle's block model pinned by
the rules it states, and the library's planner (pa_plan_append) compared with
it on random append scenarios.  Also pins of the oracle's fp8 append."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_e4m3
from oracle.blocks import BLOCK, BlockModel, OutOfBlocks
from oracle.pool import OraclePool, append_kv, write_kv

pa = pytest.importorskip("online_softmax_paged_amd")


# ---------------------------------------------------------------- block model pins
def test_model_on_demand_pages_and_copy_on_write():
    m = BlockModel(16)
    tables, ctx = [[], []], [0, 0]
    slots, copies = m.plan_append(tables, ctx, [37, 0])      # 2 full pages + 5 tokens
    assert tables[0] == [0, 1, 2] and ctx == [37, 0] and copies == []
    assert slots == [0 * 16 + i for i in range(16)] + [1 * 16 + i for i in range(16)] + \
        [2 * 16 + i for i in range(5)]
    # sequence 1 shares sequence 0's pages (a common prompt)
    tables[1] = list(tables[0])
    ctx[1] = 37
    for p in tables[1]:
        m.share(p)
    assert m.ref[:3] == [2, 2, 2]
    # sequence 1 writes into the shared partial page: it gets a copy first
    slots, copies = m.plan_append(tables, ctx, [0, 2])
    assert copies == [(2, 3)] and tables[1] == [0, 1, 3] and m.ref[2] == 1 and m.ref[3] == 1
    assert slots == [3 * 16 + 5, 3 * 16 + 6]
    # sequence 0 now owns page 2 alone: it writes in place, and at the page end
    # takes a fresh page
    slots, copies = m.plan_append(tables, ctx, [12, 0])
    assert copies == [] and tables[0] == [0, 1, 2, 4]
    assert slots == [2 * 16 + i for i in range(5, 16)] + [4 * 16 + 0]
    assert ctx == [49, 39]


def test_model_two_sharers_append_in_one_call():
    m = BlockModel(8)
    tables, ctx = [[], []], [0, 0]
    m.plan_append(tables, ctx, [20, 0])
    tables[1], ctx[1] = list(tables[0]), 20
    for p in tables[1]:
        m.share(p)
    slots, copies = m.plan_append(tables, ctx, [1, 1])
    # the first writer copies; the second is then the page's only owner
    assert copies == [(1, 2)] and tables == [[0, 2], [0, 1]]
    assert slots == [2 * 16 + 4, 1 * 16 + 4] and m.ref[:3] == [2, 1, 1]


def test_model_failure_changes_nothing():
    m = BlockModel(3)
    tables, ctx = [[]], [0]
    m.plan_append(tables, ctx, [40])                         # all 3 blocks
    before = (list(m.ref), [list(t) for t in tables], list(ctx))
    with pytest.raises(OutOfBlocks):
        m.plan_append(tables, ctx, [9])                      # needs a 4th page
    assert (m.ref, tables, ctx) == before


# ---------------------------------------------------------------- planner parity
def _c_state(alloc, tables, W):
    bt = torch.full((len(tables), W), -1, dtype=torch.int32)
    for b, t in enumerate(tables):
        bt[b, :len(t)] = torch.tensor(t, dtype=torch.int32)
    return bt


def test_planner_matches_model_on_random_appends():
    rng = np.random.default_rng(5)
    NB, W, B = 64, 12, 5
    m, a = BlockModel(NB), pa.BlockAllocator(NB)
    tables, ctx = [[] for _ in range(B)], [0] * B
    bt = torch.full((B, W), -1, dtype=torch.int32)
    cl = torch.zeros(B, dtype=torch.int32)
    for step in range(40):
        if step in (3, 11, 25):                              # fork: b2 <- b1's pages
            src, dst = rng.choice(B, 2, replace=False)
            for p in tables[dst]:                            # drop dst's own pages
                m.release(p)
                a.decref(p)
            tables[dst], ctx[dst] = list(tables[src]), ctx[src]
            for p in tables[dst]:
                m.share(p)
                a.incref(p)
            bt[dst] = bt[src]
            cl[dst] = cl[src]
        room = [W * BLOCK - c for c in ctx]
        n = [int(min(r, rng.choice([0, 1, 1, 3, 16, 21]))) for r in room]
        try:
            slots_m, copies_m = m.plan_append(tables, ctx, n)
        except OutOfBlocks:
            with pytest.raises(pa.PAError) as e:
                a.plan_append(bt, cl, n)
            assert e.value.status == pa.PA_ERR_OOM
            continue
        slots, csrc, cdst = a.plan_append(bt, cl, n)
        assert slots.tolist() == slots_m
        assert list(zip(csrc.tolist(), cdst.tolist())) == copies_m
        assert cl.tolist() == ctx
        for b in range(B):
            assert bt[b, :len(tables[b])].tolist() == tables[b]
        assert [a.refcount(i) for i in range(NB)] == m.ref
        assert a.num_free() == m.ref.count(0)


def test_planner_errors_change_nothing():
    a = pa.BlockAllocator(4)
    bt = torch.full((2, 3), -1, dtype=torch.int32)           # 48 slots per sequence
    cl = torch.zeros(2, dtype=torch.int32)
    a.plan_append(bt, cl, [20, 0])                           # 2 of 4 blocks
    snap = (bt.clone(), cl.clone(), a.num_free())
    # 40 tokens need 3 pages (2 free); 20 + 29 > 48 slots; a negative count
    for n, status in (([0, 40], pa.PA_ERR_OOM), ([29, 0], pa.PA_ERR_INVALID_ARG),
                      ([-1, 0], pa.PA_ERR_INVALID_ARG)):
        with pytest.raises(pa.PAError) as e:
            a.plan_append(bt, cl, n)
        assert e.value.status == status
        assert torch.equal(bt, snap[0]) and torch.equal(cl, snap[1]) and a.num_free() == snap[2]


# ---------------------------------------------------------------- fp8 append pins
def _fp8_pool(nb=4, hkv=2, d=8):
    return OraclePool(nb, hkv, d, "fp8")


def test_append_into_fresh_pages_equals_write():
    g = torch.Generator().manual_seed(3)
    k, v = torch.randn(23, 2, 8, generator=g), torch.randn(23, 2, 8, generator=g)
    slots = torch.tensor([16 + i for i in range(16)] + [48 + i for i in range(7)], dtype=torch.int32)
    p1, p2 = _fp8_pool(), _fp8_pool()
    write_kv(p1, k, v, slots)
    append_kv(p2, k, v, slots)
    assert np.array_equal(p1.k, p2.k) and np.array_equal(p1.v, p2.v)
    assert np.array_equal(p1.k_scale, p2.k_scale, equal_nan=True)


def test_append_of_smaller_values_keeps_codes_and_scale():
    g = torch.Generator().manual_seed(4)
    k, v = torch.randn(9, 2, 8, generator=g), torch.randn(9, 2, 8, generator=g)
    p = _fp8_pool()
    write_kv(p, k[:6], v[:6], torch.arange(6, dtype=torch.int32))
    k0, v0, s0 = p.k[0].copy(), p.v[0].copy(), (p.k_scale[0], p.v_scale[0])
    amax = min(float(k[:6].abs().max()), float(v[:6].abs().max()))
    small = torch.full((3, 2, 8), amax / 4)
    append_kv(p, small, small, torch.arange(6, 9, dtype=torch.int32))
    assert (p.k_scale[0], p.v_scale[0]) == s0
    assert np.array_equal(p.k[0][:, :6], k0[:, :6]) and np.array_equal(p.v[0][:, :, :6], v0[:, :, :6])


def test_append_reencodes_to_the_nearest_code_by_brute_force():
    g = torch.Generator().manual_seed(6)
    k, v = torch.randn(5, 2, 8, generator=g), torch.randn(5, 2, 8, generator=g)
    p = _fp8_pool()
    write_kv(p, k, v, torch.arange(5, dtype=torch.int32))
    old_codes, s_old = p.k[0][:, :5].copy(), np.float32(p.k_scale[0])
    big = torch.full((1, 2, 8), 3.0 * float(k.abs().max()))  # amax grows 3x
    append_kv(p, big, big, torch.tensor([5], dtype=torch.int32))
    s_new = np.float32(p.k_scale[0])
    assert s_new > s_old
    table = fp8_e4m3.decode_table()
    finite = np.isfinite(table)
    for code_old, code_new in zip(old_codes.reshape(-1), p.k[0][:, :5].reshape(-1)):
        x = np.float32(np.float32(table[code_old]) * s_old)       # the stored value
        y = np.float64(np.float32(x / s_new))
        dist = np.where(finite, np.abs(table - y), np.inf)
        best = np.nonzero(dist == dist.min())[0]
        best = [c for c in best if table[c] != 0 or (c >> 7) == (0 if y >= 0 else 1)] or list(best)
        # ties go to the even code (last mantissa bit 0)
        want = min(best, key=lambda c: (c & 1, c))
        assert table[code_new] == table[want], (code_old, code_new, want)


def test_append_error_bound():
    g = torch.Generator().manual_seed(7)
    p = _fp8_pool(nb=2, hkv=1, d=16)
    ref = np.zeros((16, 16), dtype=np.float64)
    pos = 0
    for scale in (1.0, 0.3, 2.5, 1.0):
        n = 4
        x = torch.randn(n, 1, 16, generator=g) * scale
        append_kv(p, x, x, torch.arange(pos, pos + n, dtype=torch.int32))
        ref[pos:pos + n] = x[:, 0].double().numpy()
        pos += n
    got = fp8_e4m3.decode(p.k[0, 0]) * np.float64(p.k_scale[0])
    amax = np.abs(ref).max()
    # each re-encoding adds at most half a code step at the top of the range
    # (16 code units of the scale at that time); four rounds at most
    assert np.abs(got - ref).max() <= 4 * 16 * amax / 448


# ---------------------------------------------------------------- copy-on-write pins
# The copy a sequence takes before writing into a block it shares (survey page,
# section 3, core principle: shared blocks carry reference counts and are copied
# before a sharer changes them).  What the copy must achieve is fixed without
# looking at oracle.pool.copy_blocks: the destination then holds what the source
# held (all heads, K, V and both fp8 scales), nothing else changes, and
# attention through the copy equals attention through the original.
def _filled_pool(kv_dtype, nb=8, hkv=2, d=8, seed=11):
    g = torch.Generator().manual_seed(seed)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.bfloat16}[kv_dtype]
    p = OraclePool(nb, hkv, d, kv_dtype)
    # every page written whole, each with its own value range (so its own fp8 scales)
    for page in range(nb):
        mag = 0.25 * (page + 1)
        k = (torch.randn(16, hkv, d, generator=g) * mag).to(dt)
        v = (torch.randn(16, hkv, d, generator=g) * (2.0 - 0.2 * page)).to(dt)
        write_kv(p, k, v, torch.arange(page * 16, page * 16 + 16, dtype=torch.int32))
    return p


def _snapshot(p):
    s = [p.k.copy(), p.v.copy()]
    if p.kv_dtype == "fp8":
        s += [p.k_scale.copy(), p.v_scale.copy()]
    return s


def _copy_pins_hold(kv_dtype, copy_fn):
    """True when copy_fn(pool, src, dst) passes every pin of a block copy."""
    p = _filled_pool(kv_dtype)
    src, dst = [1, 5, 0], [6, 2, 7]
    before = _snapshot(p)
    copy_fn(p, src, dst)
    after = _snapshot(p)
    for b_arr, a_arr in zip(before, after):
        for s, d in zip(src, dst):
            if not np.array_equal(a_arr[d], b_arr[s], equal_nan=True):   # byte for byte
                return False
        others = [i for i in range(p.num_blocks) if i not in dst]
        if not np.array_equal(a_arr[others], b_arr[others], equal_nan=True):
            return False
    # attention through a table that names the copies equals the same table on
    # the originals, for a query per sequence over 3 pages
    g = torch.Generator().manual_seed(12)
    q = torch.randn(2, 4, p.head_dim, generator=g, dtype=torch.float64)
    t_src = torch.tensor([[1, 5, 0], [0, 1, 5]], dtype=torch.int32)
    t_dst = torch.tensor([[6, 2, 7], [7, 6, 2]], dtype=torch.int32)
    cu, ctx = torch.tensor([0, 1, 2]), torch.tensor([45, 48])
    o1, l1 = oracle.paged_attention(p, q, cu, ctx, t_src, 4, 0.3, True)
    o2, l2 = oracle.paged_attention(p, q, cu, ctx, t_dst, 4, 0.3, True)
    return np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "fp8"])
def test_copy_blocks_pins(kv_dtype):
    assert _copy_pins_hold(kv_dtype, oracle.pool.copy_blocks)


def test_copy_pins_catch_planted_mistakes():
    """Plausible mistakes in a block copy each fail a pin above: fp8 scales not
    copied, only K copied, only the first KV head copied, source and
    destination swapped."""
    def no_scales(p, src, dst):
        for s, d in zip(src, dst):
            p.k[d], p.v[d] = p.k[s], p.v[s]

    def only_k(p, src, dst):
        for s, d in zip(src, dst):
            p.k[d] = p.k[s]
            if p.kv_dtype == "fp8":
                p.k_scale[d], p.v_scale[d] = p.k_scale[s], p.v_scale[s]

    def first_head(p, src, dst):
        for s, d in zip(src, dst):
            p.k[d, 0], p.v[d, 0] = p.k[s, 0], p.v[s, 0]
            if p.kv_dtype == "fp8":
                p.k_scale[d], p.v_scale[d] = p.k_scale[s], p.v_scale[s]

    def swapped(p, src, dst):
        oracle.pool.copy_blocks(p, dst, src)

    assert not _copy_pins_hold("fp8", no_scales)
    for kv in ("bf16", "fp8"):
        assert not _copy_pins_hold(kv, only_k)
        assert not _copy_pins_hold(kv, first_head)
        assert not _copy_pins_hold(kv, swapped)
