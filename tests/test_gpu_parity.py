"""GPU parity: the HIP library against the float64 oracle, on the same seeded
inputs, through the C ABI.  Bit-exact for the pool write and the block-table
gather; within the stated tolerance for attention (max |error| <= 1e-5 for
fp32, 2e-2 for bf16, 6e-2 for an fp8 pool), for outputs and logsumexps.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from oracle.pool import gather_kv
import workloads
from tests import harness as H

pytestmark = pytest.mark.gpu

pa = pytest.importorskip("online_softmax_paged_amd")


def _log(msg):
    print(msg, flush=True)


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _check_call(wl, call, pool, opool, num_splits=0, rows=None):
    dc = H.DeviceCall(wl, call)
    o, lse = dc.run(pool, num_splits=num_splits)
    torch.cuda.synchronize()
    if rows is None:
        ro, rl = H.oracle_call(opool, wl, call)
        eo, el = H.max_err(o, lse, ro, rl)
    else:
        ro, rl = H.oracle_rows(opool, wl, call, rows)
        t = torch.tensor([r[0] for r in rows])
        h = torch.tensor([r[1] for r in rows])
        eo, el = H.max_err(o.cpu()[t, h], lse.cpu()[t, h], ro, rl)
    tol = H.tolerance(wl)
    _log(f"  {wl.name} {call.kind}: max|dO|={eo:.3e} max|dLSE|={el:.3e} tol={tol}")
    assert eo <= tol and el <= tol, (eo, el, tol)
    return o, lse


# ------------------------------------------------------------ pool write / gather
@pytest.mark.parametrize("kv_dtype,src", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16"),
                                          ("fp8", "f32")])
def test_write_kv_bit_exact(kv_dtype, src):
    wl = workloads.small("decode", kv_dtype=kv_dtype, q_dtype="f32" if kv_dtype == "f32" else "bf16",
                         num_q_heads=8, num_kv_heads=4, head_dim=128,
                         ctx_lens=(1, 15, 16, 17, 250, 513), src_dtype=src, seed=31)
    _log(f"write_kv {kv_dtype} <- {src}")
    pool = H.device_pool(wl)
    opool = H.oracle_pool(wl)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(pool.k), opool.k)
    assert np.array_equal(_bits(pool.v), opool.v)
    if kv_dtype == "fp8":
        assert np.array_equal(_bits(pool.k_scale), opool.k_scale.view(np.uint32))
        assert np.array_equal(_bits(pool.v_scale), opool.v_scale.view(np.uint32))


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "fp8"])
def test_gather_kv_bit_exact(kv_dtype):
    wl = workloads.small("decode", kv_dtype=kv_dtype, q_dtype="f32" if kv_dtype == "f32" else "bf16",
                         num_q_heads=4, num_kv_heads=2, head_dim=64, ctx_lens=(3, 16, 40, 333),
                         seed=32)
    _log(f"gather_kv {kv_dtype}")
    pool = H.device_pool(wl)
    call = wl.calls[0]
    k, v = pa.gather_kv(pool, call.block_table.cuda(), call.ctx_lens.cuda(), int(call.ctx_lens.max()))
    kb, vb = _bits(k), _bits(v)
    opool = H.oracle_pool(wl)
    off = 0
    for b, c in enumerate(wl.ctx_lens):
        for t in range(c):
            p = int(call.block_table[b, t // 16])
            assert np.array_equal(kb[off + t], opool.k[p, :, t % 16, :])
            assert np.array_equal(vb[off + t], opool.v[p, :, :, t % 16])
        off += c


# ------------------------------------------------------------ append path
def _append_rounds(kv_dtype, src, D, seed):
    """Three sequences; sequence 1 forks sequence 0's pages (its last page
    partly filled and then shared); rounds of appends planned by the host
    allocator, copied (copy on write) and appended on the device and in the
    oracle.  Yields after every round."""
    g = torch.Generator().manual_seed(seed)
    NB, Hkv, W = 48, 2, 10
    pool = pa.KVPool(NB, Hkv, D, kv_dtype)
    opool = oracle.OraclePool(NB, Hkv, D, kv_dtype)
    alloc = pa.BlockAllocator(NB)
    bt = torch.full((3, W), -1, dtype=torch.int32)
    cl = torch.zeros(3, dtype=torch.int32)
    sdt = {"f32": torch.float32, "bf16": torch.bfloat16}[src]
    scales = iter([1.0, 2.0, 0.5, 3.0, 1.0])
    for r in ([37, 0, 5], "fork", [1, 1, 0], [0, 12, 16], [20, 3, 1], [1, 1, 1]):
        if r == "fork":
            bt[1], cl[1] = bt[0], cl[0]
            for p in bt[0, :(int(cl[0]) + 15) // 16].tolist():
                alloc.incref(p)
            continue
        slots, csrc, cdst = alloc.plan_append(bt, cl, r)
        sc = next(scales)
        k = (torch.randn(len(slots), Hkv, D, generator=g) * sc).to(sdt)
        v = (torch.randn(len(slots), Hkv, D, generator=g) * sc).to(sdt)
        if len(csrc):
            pa.copy_blocks(pool, csrc.cuda(), cdst.cuda())
            oracle.copy_blocks(opool, csrc.tolist(), cdst.tolist())
        pa.append_kv(pool, k.cuda(), v.cuda(), slots.cuda())
        oracle.append_kv(opool, k, v, slots)
        yield pool, opool, bt, cl, len(csrc)


@pytest.mark.parametrize("kv_dtype,src", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16"),
                                          ("fp8", "f32")])
def test_append_rounds_bit_exact(kv_dtype, src):
    _log(f"append_kv rounds {kv_dtype} <- {src}")
    copies = 0
    for pool, opool, bt, cl, nc in _append_rounds(kv_dtype, src, 64, seed=71):
        torch.cuda.synchronize()
        copies += nc
        assert np.array_equal(_bits(pool.k), opool.k)
        assert np.array_equal(_bits(pool.v), opool.v)
        if kv_dtype == "fp8":
            assert np.array_equal(_bits(pool.k_scale), opool.k_scale.view(np.uint32))
            assert np.array_equal(_bits(pool.v_scale), opool.v_scale.view(np.uint32))
    assert copies == 1                                     # the shared partial page


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "fp8"])
def test_decode_after_each_append_round(kv_dtype):
    _log(f"decode after appends {kv_dtype}")
    g = torch.Generator().manual_seed(72)
    Hq, D = 4, 128
    qd = torch.float32 if kv_dtype == "f32" else torch.bfloat16
    scale = D ** -0.5
    for pool, opool, bt, cl, _ in _append_rounds(kv_dtype, "f32" if kv_dtype == "f32" else "bf16",
                                                 D, seed=73):
        q = torch.randn(3, Hq, D, generator=g).to(qd)
        o, lse = pa.decode(pool, q.cuda(), cl.cuda(), bt.cuda(), scale, max_ctx_len=bt.shape[1] * 16)
        torch.cuda.synchronize()
        ro, rl = oracle.paged_attention(opool, q, torch.arange(4), cl, bt, Hq, scale, True)
        eo, el = H.max_err(o, lse, ro, rl)
        tol = H.TOL["fp8" if kv_dtype == "fp8" else ("f32" if kv_dtype == "f32" else "bf16")]
        _log(f"  ctx {cl.tolist()}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= tol and el <= tol, (cl.tolist(), eo, el)


# ------------------------------------------------------------ decode parity
DECODE_CASES = [
    ("f32", "f32", 64, 1, 1, (1, 15, 16, 17, 256)),
    ("f32", "f32", 128, 4, 2, (33, 200)),
    ("bf16", "bf16", 128, 8, 2, (1, 15, 16, 17, 100, 300, 1000)),
    ("bf16", "bf16", 128, 64, 8, (500, 2000)),
    ("bf16", "bf16", 64, 16, 16, (77, 300)),
    ("bf16", "bf16", 128, 32, 2, (129, 40)),
    ("bf16", "bf16", 64, 4, 2, (600,)),
    ("fp8", "bf16", 128, 8, 2, (1, 17, 300, 1000)),
    ("fp8", "bf16", 64, 16, 2, (50, 400)),
]


@pytest.mark.parametrize("kv,qd,D,Hq,Hkv,ctx", DECODE_CASES)
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_parity(kv, qd, D, Hq, Hkv, ctx, splits):
    _log(f"decode kv={kv} D={D} Hq={Hq} Hkv={Hkv} ctx={ctx} splits={splits}")
    wl = workloads.small("decode", kv_dtype=kv, q_dtype=qd, num_q_heads=Hq, num_kv_heads=Hkv,
                         head_dim=D, ctx_lens=ctx, seed=40 + D + Hq)
    _check_call(wl, wl.calls[0], H.device_pool(wl), H.oracle_pool(wl), num_splits=splits)


# ------------------------------------------------------------ prefill parity
PREFILL_CASES = [
    # kv, q, D, Hq, Hkv, ctx_lens, q_lens (None = whole sequence), causal
    ("f32", "f32", 64, 1, 1, (256, 17), None, True),
    ("f32", "f32", 128, 4, 2, (100, 40), (30, 40), True),
    ("bf16", "bf16", 128, 8, 2, (300, 1, 17, 64, 129), None, True),
    ("bf16", "bf16", 128, 8, 2, (700, 300), (45, 300), True),
    ("bf16", "bf16", 128, 8, 2, (200, 90), (77, 90), False),
    ("bf16", "bf16", 64, 16, 16, (250, 33), None, True),
    ("bf16", "bf16", 128, 64, 8, (300,), None, True),
    ("bf16", "bf16", 128, 32, 2, (97, 40), (50, 40), True),
    ("bf16", "bf16", 64, 4, 2, (333,), None, True),
    ("fp8", "bf16", 128, 8, 2, (400, 60), (256, 60), True),
    ("fp8", "bf16", 64, 16, 2, (150,), None, True),
]


@pytest.mark.parametrize("kv,qd,D,Hq,Hkv,ctx,ql,causal", PREFILL_CASES)
def test_prefill_parity(kv, qd, D, Hq, Hkv, ctx, ql, causal):
    _log(f"prefill kv={kv} D={D} Hq={Hq} Hkv={Hkv} ctx={ctx} q={ql} causal={causal}")
    wl = workloads.small("prefill", kv_dtype=kv, q_dtype=qd, num_q_heads=Hq, num_kv_heads=Hkv,
                         head_dim=D, ctx_lens=ctx, q_lens=ql, seed=50 + D + Hq)
    wl.calls[0].causal = causal
    _check_call(wl, wl.calls[0], H.device_pool(wl), H.oracle_pool(wl))


# ------------------------------------------------------------ the five named workloads
@functools.lru_cache(maxsize=1)
def _named(k):
    wl = workloads.NAMED[k]()
    return wl, H.oracle_pool(wl)


PREFILL_SPLIT_CASES = [
    # kv, D, Hq, Hkv, ctx_lens, q_lens, splits
    ("bf16", 128, 8, 2, (700, 300), (45, 300), 2),
    ("bf16", 128, 8, 2, (700, 300), (45, 300), 3),
    ("bf16", 64, 4, 2, (333,), None, 3),
    ("bf16", 128, 8, 2, (100, 37), None, 5),        # more splits than key tiles: empty ranges
    ("fp8", 128, 8, 2, (400, 60), (256, 60), 2),
    ("fp8", 128, 16, 2, (1000, 520), (256, 1), 4),
]


@pytest.mark.parametrize("kv,D,Hq,Hkv,ctx,ql,splits", PREFILL_SPLIT_CASES)
def test_prefill_key_splits(kv, D, Hq, Hkv, ctx, ql, splits):
    _log(f"prefill splits={splits} kv={kv} D={D} Hq={Hq} Hkv={Hkv} ctx={ctx} q={ql}")
    wl = workloads.small("prefill", kv_dtype=kv, q_dtype="bf16", num_q_heads=Hq, num_kv_heads=Hkv,
                         head_dim=D, ctx_lens=ctx, q_lens=ql, seed=80 + splits)
    _check_call(wl, wl.calls[0], H.device_pool(wl), H.oracle_pool(wl), num_splits=splits)


def test_mixed_batch_in_one_prefill_call():
    """Chunked prefills and q_len = 1 decode rows of one batch in a single
    call (with and without key splits) match the oracle and the decode path."""
    _log("mixed prefill + decode rows in one call")
    wl = workloads.small("prefill", kv_dtype="fp8", q_dtype="bf16", num_q_heads=8, num_kv_heads=2,
                         head_dim=128, ctx_lens=(600, 300, 900, 45), q_lens=(128, 1, 1, 45), seed=85)
    pool, opool = H.device_pool(wl), H.oracle_pool(wl)
    for splits in (1, 3, 0):
        o, lse = _check_call(wl, wl.calls[0], pool, opool, num_splits=splits)
    # the decode rows equal pa_decode on the same sequences
    call = wl.calls[0]
    sel = torch.tensor([1, 2])
    q_dec = call.q[call.cu_q_lens[1:3].long()].cuda()
    od, ld = pa.decode(pool, q_dec, call.ctx_lens[sel].cuda(), call.block_table[sel].cuda(),
                       wl.scale, max_ctx_len=900, num_splits=1)
    rows = call.cu_q_lens[1:3].long().cuda()
    assert (o[rows].float() - od.float()).abs().max() <= 2 * H.TOL["fp8"]
    assert (lse[rows] - ld).abs().max() <= 1e-3


BALANCED_CASES = [
    # kv, D, Hq, Hkv, ctx_lens
    ("bf16", 128, 32, 8, (1, 15, 16, 17, 250, 513, 2048, 40, 900, 33)),   # mixed, ragged
    ("bf16", 128, 8, 2, tuple(range(1, 700, 7))),                          # 100 sequences (> 64)
    ("bf16", 64, 16, 1, (3000, 17, 45, 2)),
    ("fp8", 128, 32, 8, (128, 2048, 1000, 129, 16, 700, 1536, 1)),
    ("fp8", 64, 8, 8, (64, 65, 300)),
    ("bf16", 128, 16, 16, (4096,)),                                        # one long sequence
]


@pytest.mark.parametrize("kv,D,Hq,Hkv,ctx", BALANCED_CASES)
def test_balanced_decode_parity(kv, D, Hq, Hkv, ctx):
    """Balanced decode (each KV head's pages of all sequences cut into equal
    per-wave chunks that may span sequences) against the oracle; and equal to
    the split decode within rounding."""
    _log(f"balanced decode kv={kv} D={D} Hq={Hq} Hkv={Hkv} ctx={ctx[:12]}")
    wl = workloads.small("decode", kv_dtype=kv, q_dtype="bf16", num_q_heads=Hq, num_kv_heads=Hkv,
                         head_dim=D, ctx_lens=ctx, seed=70 + D + Hkv)
    pool, opool = H.device_pool(wl), H.oracle_pool(wl)
    o, lse = _check_call(wl, wl.calls[0], pool, opool, num_splits=pa.DECODE_BALANCED)
    o2, l2 = H.DeviceCall(wl, wl.calls[0]).run(pool, num_splits=1)
    assert (o.float() - o2.float()).abs().max().item() <= H.tolerance(wl)
    assert (lse - l2).abs().max().item() <= 1e-3
    # bitwise repeatable
    o3, l3 = H.DeviceCall(wl, wl.calls[0]).run(pool, num_splits=pa.DECODE_BALANCED)
    assert torch.equal(o, o3) and torch.equal(lse, l3)


def test_decode_auto_choice_on_uneven_batch():
    """With the batch's total length known, a batch whose longest sequence is
    far above the mean is routed to the balanced kernel and still matches."""
    _log("decode auto choice, uneven batch")
    ctx = (3000,) + (40,) * 20 + (17, 1)
    wl = workloads.small("decode", kv_dtype="bf16", q_dtype="bf16", num_q_heads=16,
                         num_kv_heads=4, head_dim=128, ctx_lens=ctx, seed=77)
    assert pa.decode_choose_splits(len(ctx), 4, 3000, sum(ctx)) == pa.DECODE_BALANCED
    pool, opool = H.device_pool(wl), H.oracle_pool(wl)
    call = wl.calls[0]
    dc = H.DeviceCall(wl, call)
    o, lse = pa.decode(pool, dc.q, dc.ctx_lens, dc.block_table, wl.scale, max_ctx_len=3000,
                       total_ctx_len=sum(ctx))
    torch.cuda.synchronize()
    ro, rl = H.oracle_call(opool, wl, call)
    eo, el = H.max_err(o, lse, ro, rl)
    _log(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= H.TOL["bf16"] and el <= H.TOL["bf16"]
    o2, l2 = pa.decode(pool, dc.q, dc.ctx_lens, dc.block_table, wl.scale,
                       num_splits=pa.DECODE_BALANCED)
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_balanced_decode_named_full():
    """The 32-sequence mixed-length and 8 x 32768 decode workloads, balanced."""
    for k in (2, 4):
        _log(f"balanced decode, named workload {k}")
        wl, opool = _named(k)
        pool = H.device_pool(wl)
        call = [c for c in wl.calls if c.kind == "decode"][0]
        _check_call(wl, call, pool, opool, num_splits=pa.DECODE_BALANCED)


# ------------------------------------------------------------ fp8 products
FP8MMA_CASES = [
    # D, Hq, Hkv, ctx_lens, q_lens (None = whole sequences), causal
    (128, 8, 2, (600, 300, 45, 129), None, True),
    (128, 8, 2, (600, 300, 900), (128, 1, 77), True),    # chunks and a decode row
    (128, 8, 2, (300, 70), (100, 70), False),
    (64, 4, 4, (257, 33), None, True),                   # G = 1
    (128, 16, 2, (150, 90), (150, 17), True),            # G = 8
    (128, 8, 2, (20, 5, 70, 64), None, True),            # rows that see 1 .. 70 keys
    # block tables past 64 and 128 pages: the page-id lane vectors' later
    # chunks, and with 3 splits a split whose first tile lies in chunk 1
    (128, 8, 2, (2600, 2100), (64, 1), True),
    (64, 4, 2, (2200,), (40,), False),
]


def _fp8_products_check(opool, wl, call, o, lse, ro, rl):
    """Every row of the fp8-product path, and every logsumexp, within the
    fp8-KV bound.  Also the bound E4M3's rounding of the weights implies per
    element: each weight w_i reaches P.V as an E4M3 code of w_i f_i (f_i = 112
    times its V page scale over the largest); a single code carries a relative
    error |e_i| <= 2^-4 (normal codes, |w_i e_i| <= 2^-10 / f_i below them),
    and the kernel divides by the codes' own sum, so per feature d
        |O'_d - O_d| <= (2^-4 + n 2^-10 / f_min) / (1 - 2^-4) * max_i |v_id - O_d|
    over the row's n visible keys, plus 1e-2 for the rest (Q's remainder after
    its two parts, bf16 output rounding, fp32 sums).  Rows that see fewer than
    64 keys get P in two E4M3 parts, far inside it.  Returns the max errors of
    all rows and of the logsumexps."""
    go = o.detach().to(torch.float64).cpu().numpy()
    eo_all, el = H.max_err(o, lse, ro, rl)
    cu = call.cu_q_lens.tolist()
    G = wl.num_q_heads // wl.num_kv_heads
    for b in range(len(cu) - 1):
        c = int(call.ctx_lens[b])
        n = cu[b + 1] - cu[b]
        if n == 0 or c == 0:
            continue
        bt = call.block_table[b].numpy()
        vs = np.array([opool.v_scale[bt[p]] for p in range((c + 15) // 16)])
        f_min = 112.0 * vs.min() / vs.max()
        pos = c - n + np.arange(n)
        nk = np.minimum(pos + 1, c) if call.causal else np.full(n, c)
        for g in range(wl.num_kv_heads):
            _, V = gather_kv(opool, bt, c, g)
            vmax, vmin = np.maximum.accumulate(V, 0), np.minimum.accumulate(V, 0)
            for h in range(g * G, (g + 1) * G):
                O = ro[cu[b]:cu[b + 1], h]
                spread = np.maximum(vmax[nk - 1] - O, O - vmin[nk - 1])
                coef = (2.0 ** -4 + nk[:, None] * 2.0 ** -10 / f_min) / (1 - 2.0 ** -4)
                err = np.abs(go[cu[b]:cu[b + 1], h] - O)
                assert (err <= coef * spread + 1e-2).all(), (b, h, float((err - coef * spread).max()))
    return eo_all, el


@pytest.mark.parametrize("D,Hq,Hkv,ctx,ql,causal", FP8MMA_CASES)
@pytest.mark.parametrize("splits", [1, 3])
def test_prefill_fp8_products_parity(D, Hq, Hkv, ctx, ql, causal, splits):
    """Q (two E4M3 parts) and P (E4M3; two parts where rows see few keys) on
    the fp8 matrix cores, every row against the oracle at the fp8-KV bound
    and under the bound derived from E4M3's rounding; the error of the
    bf16-product path on the same inputs is logged beside it."""
    _log(f"fp8 products D={D} Hq={Hq} Hkv={Hkv} ctx={ctx} q={ql} causal={causal} splits={splits}")
    wl = workloads.small("prefill", kv_dtype="fp8", q_dtype="bf16", num_q_heads=Hq,
                         num_kv_heads=Hkv, head_dim=D, ctx_lens=ctx, q_lens=ql, seed=140 + D + Hq,
                         causal=causal)
    pool, opool = H.device_pool(wl), H.oracle_pool(wl)
    call = wl.calls[0]
    ro, rl = H.oracle_call(opool, wl, call)
    o, lse = H.DeviceCall(wl, call).run(pool, num_splits=splits, fp8_products=True)
    o2, l2 = H.DeviceCall(wl, call).run(pool, num_splits=splits)
    torch.cuda.synchronize()
    eo2, el2 = H.max_err(o2, l2, ro, rl)
    eo, el = _fp8_products_check(opool, wl, call, o, lse, ro, rl)
    _log(f"  fp8 products max|dO|={eo:.3e} max|dLSE|={el:.3e}; bf16 products {eo2:.3e} {el2:.3e}")
    assert eo <= H.TOL["fp8"] and el <= H.TOL["fp8"]


def test_prefill_fp8_products_mixed_step_full_size():
    """The 16-sequence mixed step's chunked prefill (8 x 256 over 1536 fp8
    keys, every row seeing 1281 keys or more) with fp8 products, every row
    against the oracle at the fp8-KV bound."""
    _log("fp8 products: mixed fp8 step, prefill call")
    wl, opool = _named(5)
    pool = H.device_pool(wl)
    call = [c for c in wl.calls if c.kind == "prefill"][0]
    dc = H.DeviceCall(wl, call)
    o, lse = dc.run(pool, fp8_products=True)
    torch.cuda.synchronize()
    ro, rl = H.oracle_call(opool, wl, call)
    eo, el = H.max_err(o, lse, ro, rl)
    _log(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= H.TOL["fp8"] and el <= H.TOL["fp8"]
    o2, l2 = dc.run(pool, fp8_products=True)
    assert torch.equal(o, o2) and torch.equal(lse, l2)


# ------------------------------------------------------------ shared prefix
def _run_shared(wl, call, pool, prefix, **kw):
    dc = H.DeviceCall(wl, call)
    return pa.prefill_shared_prefix(pool, dc.q, dc.cu_q_lens, dc.ctx_lens, dc.block_table,
                                    wl.scale, prefix, causal=call.causal,
                                    max_q_len=dc.max_q_len, max_ctx_len=dc.max_ctx_len,
                                    validate=True, **kw)


SHARED_CASES = [
    # kv, D, Hq, Hkv, prefix, ctx_lens, q_lens, causal
    ("bf16", 128, 8, 2, 64, (200, 130, 300, 65), (64, 1, 100, 1), True),
    ("bf16", 128, 8, 2, 48, (200, 130, 300, 49), (64, 1, 100, 1), True),   # prefix ends mid-tile
    ("bf16", 64, 16, 2, 96, (400, 97, 250), (1, 1, 150), False),
    ("fp8", 128, 8, 2, 64, (200, 130, 300, 65), (64, 1, 100, 1), True),
    ("fp8", 128, 8, 1, 48, (90, 333, 61), (17, 200, 1), True),
    ("fp8", 64, 4, 4, 128, (129, 140, 700, 300), (1, 12, 1, 172), False),
    ("bf16", 128, 8, 2, 64, (200, 130, 300, 65), (1, 1, 1, 1), True),       # decode rows only
    ("fp8", 128, 16, 2, 32, (90, 33, 61, 140, 47), (1, 1, 1, 1, 1), True),
]

# (mode, prefix, suffix, plain splits); 0 = the plan's
SHARED_PLANS = [(pa.SHARED_PACKED, 0, 0, 0), (pa.SHARED_PACKED, 1, 1, 1),
                (pa.SHARED_PACKED, 3, 2, 2), (pa.SHARED_PLAIN, 0, 0, 0),
                (pa.SHARED_PLAIN, 0, 0, 3), (pa.SHARED_AUTO, 0, 0, 0)]


@pytest.mark.parametrize("kv,D,Hq,Hkv,prefix,ctx,ql,causal", SHARED_CASES)
@pytest.mark.parametrize("plan", SHARED_PLANS)
def test_shared_prefix_parity(kv, D, Hq, Hkv, prefix, ctx, ql, causal, plan):
    """Queries of sequences that share their first pages.  Packed: the q_len = 1
    rows attend the prefix once, packed together, and their own keys apart,
    merged, while rows with q_len > 1 take the ordinary pass; plain: the
    ordinary pass for all.  The result matches the oracle (which knows nothing
    of the sharing) and pa_prefill."""
    _log(f"shared prefix kv={kv} D={D} Hq={Hq} Hkv={Hkv} prefix={prefix} ctx={ctx} "
         f"q={ql} causal={causal} plan={plan}")
    wl = workloads.small("prefill", kv_dtype=kv, q_dtype="bf16", num_q_heads=Hq,
                         num_kv_heads=Hkv, head_dim=D, ctx_lens=ctx, q_lens=ql, seed=90 + D,
                         shared_prefix=prefix, causal=causal)
    pool, opool = H.device_pool(wl), H.oracle_pool(wl)
    call = wl.calls[0]
    o, lse = _run_shared(wl, call, pool, prefix, mode=plan[0], prefix_splits=plan[1],
                         suffix_splits=plan[2], plain_splits=plan[3])
    torch.cuda.synchronize()
    ro, rl = H.oracle_call(opool, wl, call)
    eo, el = H.max_err(o, lse, ro, rl)
    tol = H.tolerance(wl)
    _log(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e} tol={tol}")
    assert eo <= tol and el <= tol
    o2, l2 = H.DeviceCall(wl, call).run(pool, num_splits=1)
    assert (o.float() - o2.float()).abs().max().item() <= tol
    assert (lse - l2).abs().max().item() <= 1e-3


@pytest.mark.parametrize("mode", [pa.SHARED_AUTO, pa.SHARED_PACKED])
def test_shared_prefix_mixed_step_full_size(mode):
    """The 16-sequence fp8 mixed step (8 chunks of 256 and 8 decode rows over a
    shared 1024-token prefix) as one shared-prefix call, in the benchmark's
    configuration (the library's choice) and packed, against the oracle on
    every row."""
    _log(f"shared prefix: mixed fp8 16x1536 as one call, mode {mode}")
    wl, opool = _named(5)
    pool = H.device_pool(wl)
    call = workloads.one_call(wl)
    o, lse = _run_shared(wl, call, pool, wl.shared_prefix, mode=mode)
    torch.cuda.synchronize()
    ro, rl = H.oracle_call(opool, wl, call)
    eo, el = H.max_err(o, lse, ro, rl)
    _log(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= H.TOL["fp8"] and el <= H.TOL["fp8"]
    # repeat: bitwise the same
    o2, l2 = _run_shared(wl, call, pool, wl.shared_prefix, mode=mode)
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_shared_prefix_decode_only_splits_the_prefix():
    """Decode rows only (one token per sequence) over a long shared prefix: the
    packed prefix pass has one query tile per KV head, so its keys are split."""
    _log("shared prefix: decode rows over a 4096-token prefix")
    wl = workloads.small("prefill", kv_dtype="bf16", q_dtype="bf16", num_q_heads=32,
                         num_kv_heads=8, head_dim=128, ctx_lens=(4200, 4097, 4400, 4111),
                         q_lens=(1, 1, 1, 1), seed=97, shared_prefix=4096)
    pool, opool = H.device_pool(wl), H.oracle_pool(wl)
    call = wl.calls[0]
    plan = pa.shared_prefix_plan(pool, 4, 32, 1, 4400, 4096, 4, mode=pa.SHARED_PACKED)
    sp, ss = plan["prefix_splits"], plan["suffix_splits"]
    assert sp > 1
    o, lse = _run_shared(wl, call, pool, 4096, mode=pa.SHARED_PACKED)
    torch.cuda.synchronize()
    ro, rl = H.oracle_call(opool, wl, call)
    eo, el = H.max_err(o, lse, ro, rl)
    _log(f"  splits={sp},{ss} max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= H.TOL["bf16"] and el <= H.TOL["bf16"]


def test_shared_prefix_auto_packs_decode_rows_of_a_mixed_batch():
    """16 decode rows and one 64-token chunk over a 4096-token bf16 prefix: the
    library packs the decode rows (their prefix reads beyond the first are
    252 MB) and runs the chunk through the ordinary pass; every row matches the
    oracle and the plain arrangement."""
    _log("shared prefix: auto plan on 16 decode rows + 1 chunk")
    ctx = tuple(4096 + 20 + 7 * i for i in range(16)) + (4096 + 64,)
    wl = workloads.small("prefill", kv_dtype="bf16", q_dtype="bf16", num_q_heads=32,
                         num_kv_heads=8, head_dim=128, ctx_lens=ctx, q_lens=(1,) * 16 + (64,),
                         seed=98, shared_prefix=4096)
    pool, opool = H.device_pool(wl), H.oracle_pool(wl)
    call = wl.calls[0]
    plan = pa.shared_prefix_plan(pool, 17, 32, 64, max(ctx), 4096, 80)
    assert plan["mode"] == pa.SHARED_PACKED
    o, lse = _run_shared(wl, call, pool, 4096)
    torch.cuda.synchronize()
    ro, rl = H.oracle_call(opool, wl, call)
    eo, el = H.max_err(o, lse, ro, rl)
    _log(f"  plan={plan} max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= H.TOL["bf16"] and el <= H.TOL["bf16"]
    o2, l2 = _run_shared(wl, call, pool, 4096, mode=pa.SHARED_PLAIN)
    assert (o.float() - o2.float()).abs().max().item() <= H.TOL["bf16"]
    assert (lse - l2).abs().max().item() <= 1e-3


@pytest.mark.parametrize("k", [1, 2, 4, 5])
def test_named_workload_full(k):
    _log(f"named workload {k}")
    wl, opool = _named(k)
    pool = H.device_pool(wl)
    for call in wl.calls:
        _check_call(wl, call, pool, opool)


def test_named_prefill_4x4096_every_row():
    """Full-size causal prefill (4 x 4096 tokens, 32 query / 8 KV heads, d 128)
    in the benchmark's launch configuration, every (token, head) row against
    the oracle.  o starts as NaN and lse as +inf, so a query tile the kernel
    never wrote fails, and one written with another tile's rows fails on its
    values."""
    _log("named workload 3 (every row)")
    wl, opool = _named(3)
    pool = H.device_pool(wl)
    call = wl.calls[0]
    dc = H.DeviceCall(wl, call)
    T, Hq, _ = dc.q.shape
    o = torch.full_like(dc.q, float("nan"))
    lse = torch.full((T, Hq), float("inf"), dtype=torch.float32, device=dc.q.device)
    S = pa.prefill_num_splits(len(call.q_lens), wl.num_kv_heads, Hq, dc.max_q_len, dc.max_ctx_len)
    dc.run(pool, num_splits=S, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), "unwritten rows"
    ro, rl = H.oracle_call(opool, wl, call)
    eo, el = H.max_err(o, lse, ro, rl)
    _log(f"  every row: max|dO|={eo:.3e} max|dLSE|={el:.3e} tol={H.TOL['bf16']}")
    assert eo <= H.TOL["bf16"] and el <= H.TOL["bf16"], (eo, el)


@pytest.mark.parametrize("kv,ctx0,splits,fp8p", [
    ("bf16", 0, 1, False), ("bf16", 0, 3, False), ("bf16", 5, 1, False),
    ("fp8", 5, 2, False), ("fp8", 5, 2, True), ("fp8", 0, 1, True), ("fp8", 0, 3, True)])
def test_rows_that_see_no_key_are_empty(kv, ctx0, splits, fp8p):
    """Lengths outside the contract (a sequence with ctx 0, or more queries
    than cached tokens) leave rows with no visible key: every such row, also
    with key splits, comes out as O = 0 and LSE = -inf, and the other rows as
    the oracle has them.  o and lse start as NaN and +inf."""
    _log(f"empty rows {kv} ctx0={ctx0} splits={splits} fp8_products={fp8p}")
    wl = workloads.small("prefill", kv_dtype=kv, num_q_heads=8, num_kv_heads=2, head_dim=128,
                         ctx_lens=(40, 300), q_lens=(8, 100), seed=71)
    call = wl.calls[0]
    call.ctx_lens = call.ctx_lens.clone()
    call.ctx_lens[0] = ctx0          # sequence 0: 8 queries over ctx0 keys
    pool, opool = H.device_pool(wl), H.oracle_pool(wl)
    dc = H.DeviceCall(wl, call)
    T, Hq, _ = dc.q.shape
    o = torch.full_like(dc.q, float("nan"))
    lse = torch.full((T, Hq), float("inf"), dtype=torch.float32, device=dc.q.device)
    dc.run(pool, num_splits=splits, out=o, lse=lse, fp8_products=fp8p)
    torch.cuda.synchronize()
    empty = 8 - ctx0                 # sequence 0's rows before position 0
    assert bool((o[:empty] == 0).all()) and bool((lse[:empty] == -float("inf")).all())
    ro, rl = H.oracle_call(opool, wl, call)
    eo, el = H.max_err(o, lse, ro, rl)
    tol = H.tolerance(wl)
    _log(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e} tol={tol}")
    assert eo <= tol and el <= tol


# ------------------------------------------------------------ invariants
def _run_both(wl, pool):
    return [H.DeviceCall(wl, c).run(pool) for c in wl.calls]


def test_block_relabelling_is_bit_identical():
    """Moving every page to another physical id (and remapping the tables)
    leaves outputs bit-identical: the math does not depend on where pages live."""
    _log("relabel")
    for kind in ("decode", "prefill"):
        wl = workloads.small(kind, num_q_heads=8, num_kv_heads=2, ctx_lens=(300, 45, 129), seed=60)
        r1 = _run_both(wl, H.device_pool(wl))
        perm = torch.randperm(wl.num_blocks, generator=torch.Generator().manual_seed(5)).to(torch.int32)
        wl.slot_mapping = perm[(wl.slot_mapping // 16).long()] * 16 + wl.slot_mapping % 16
        for c in wl.calls:
            bt = c.block_table.clone()
            bt[bt >= 0] = perm[bt[bt >= 0].long()]
            c.block_table = bt
        r2 = _run_both(wl, H.device_pool(wl))
        for (o1, l1), (o2, l2) in zip(r1, r2):
            assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_shared_prefix_equals_private_copies():
    """Sequences reading one shared physical prefix give bit-identical results
    to the same sequences with private copies of those bytes."""
    _log("shared prefix")
    mk = lambda shared: workloads.build(
        "p", kv_dtype="fp8", q_dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128,
        ctx_lens=[200, 200, 200], shared_prefix=shared,
        calls=[workloads.Call("decode", [0, 1, 2], [1, 1, 1])], seed=61)
    wl_s = mk(64)
    pool_s = H.device_pool(wl_s)
    # private copies: duplicate the shared pages into fresh physical blocks
    wl_p = mk(64)
    extra = 3 * 4
    pool_p = pa.KVPool(wl_s.num_blocks + extra, 2, 128, "fp8")
    pool_p.k[: wl_s.num_blocks] = pool_s.k
    pool_p.v[: wl_s.num_blocks] = pool_s.v
    pool_p.k_scale[: wl_s.num_blocks] = pool_s.k_scale
    pool_p.v_scale[: wl_s.num_blocks] = pool_s.v_scale
    bt = wl_p.calls[0].block_table.clone()
    nid = wl_s.num_blocks
    for b in range(3):
        for j in range(4):
            src = int(bt[b, j])
            pool_p.k[nid] = pool_s.k[src]
            pool_p.v[nid] = pool_s.v[src]
            pool_p.k_scale[nid] = pool_s.k_scale[src]
            pool_p.v_scale[nid] = pool_s.v_scale[src]
            bt[b, j] = nid
            nid += 1
    assert len(set(bt[:, :4].flatten().tolist())) == 12
    wl_p.calls[0].block_table = bt
    o1, l1 = H.DeviceCall(wl_s, wl_s.calls[0]).run(pool_s)
    o2, l2 = H.DeviceCall(wl_p, wl_p.calls[0]).run(pool_p)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_repeat_runs_are_bitwise_equal_and_splits_agree():
    _log("determinism / splits")
    wl = workloads.small("decode", num_q_heads=16, num_kv_heads=2, ctx_lens=(2000, 900, 31), seed=62)
    pool = H.device_pool(wl)
    dc = H.DeviceCall(wl, wl.calls[0])
    for s in (1, 2, 5, 16):
        a = dc.run(pool, num_splits=s)
        b = dc.run(pool, num_splits=s)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    ro, rl = H.oracle_call(H.oracle_pool(wl), wl, wl.calls[0])
    for s in (1, 2, 3, 7, 16, 64):
        eo, el = H.max_err(*dc.run(pool, num_splits=s), ro, rl)
        assert eo <= 2e-2 and el <= 1e-4, (s, eo, el)
    wl2 = workloads.small("prefill", num_q_heads=8, num_kv_heads=2, ctx_lens=(500, 70), seed=63)
    pool2 = H.device_pool(wl2)
    dc2 = H.DeviceCall(wl2, wl2.calls[0])
    a, b = dc2.run(pool2), dc2.run(pool2)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_reused_workspace_gives_the_same_results():
    """One workspace serves consecutive calls of different batches (and
    dtypes), bit-identical to a fresh workspace each time."""
    _log("decode workspace reuse")
    cases = [workloads.small("decode", num_q_heads=16, num_kv_heads=2, ctx_lens=(2000, 900, 31), seed=64),
             workloads.small("decode", num_q_heads=8, num_kv_heads=2, ctx_lens=(300, 45), seed=65),
             workloads.small("decode", kv_dtype="fp8", num_q_heads=8, num_kv_heads=2,
                             ctx_lens=(1000, 17, 400), seed=66)]
    S = 6
    need = max(pa.decode_workspace_bytes(len(wl.ctx_lens), wl.num_q_heads, wl.head_dim, S) for wl in cases)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")   # arbitrary contents
    for rep in range(2):
        for wl in cases:
            pool = H.device_pool(wl)
            dc = H.DeviceCall(wl, wl.calls[0])
            fresh = dc.run(pool, num_splits=S)
            reused = dc.run(pool, num_splits=S, workspace=ws)
            assert torch.equal(fresh[0], reused[0]) and torch.equal(fresh[1], reused[1]), (rep, wl.name)


def test_table_entries_past_the_end_are_never_read():
    """Entries after a sequence's last page: -1 (default) or a wild id NB+7."""
    _log("table poison")
    for kind in ("decode", "prefill"):
        wl = workloads.small(kind, num_q_heads=8, num_kv_heads=2, ctx_lens=(300, 20, 170), seed=64)
        pool = H.device_pool(wl)
        r1 = _run_both(wl, pool)
        for c in wl.calls:
            c.block_table[c.block_table < 0] = wl.num_blocks + 7
        r2 = _run_both(wl, pool)
        for (o1, l1), (o2, l2) in zip(r1, r2):
            assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_matches_last_prefill_row():
    """Decode of the last position's query equals prefill's last row (both
    against the oracle, and against each other within the bf16 tolerance)."""
    _log("decode vs prefill last row")
    wl = workloads.small("prefill", num_q_heads=8, num_kv_heads=2, ctx_lens=(333, 64), seed=65)
    pool = H.device_pool(wl)
    call = wl.calls[0]
    o_p, l_p = H.DeviceCall(wl, call).run(pool)
    last = call.cu_q_lens[1:] - 1
    dq = call.q[last.long()].contiguous().cuda()
    o_d, l_d = pa.decode(pool, dq, call.ctx_lens.cuda(), call.block_table.cuda(), wl.scale)
    assert (o_d.float() - o_p[last.long().cuda()].float()).abs().max().item() <= 2e-2
    assert (l_d - l_p[last.long().cuda()]).abs().max().item() <= 1e-4


def test_causal_first_row_is_v0_exactly():
    _log("first row")
    wl = workloads.small("prefill", num_q_heads=4, num_kv_heads=2, ctx_lens=(64,), seed=66)
    pool = H.device_pool(wl)
    o, lse = H.DeviceCall(wl, wl.calls[0]).run(pool)
    v0 = wl.v_src[0]                       # token 0, [Hkv, D]
    for h in range(4):
        assert torch.equal(o[0, h].cpu(), v0[h // 2])
        ref = wl.scale * float(wl.calls[0].q[0, h].double() @ wl.k_src[0, h // 2].double())
        assert abs(lse[0, h].item() - ref) <= 1e-4


def test_constant_v_gives_the_constant():
    _log("constant V")
    wl = workloads.small("prefill", num_q_heads=8, num_kv_heads=2, ctx_lens=(300, 33), seed=67)
    c = torch.linspace(-3, 3, 128).to(torch.bfloat16)
    wl.v_src = c.reshape(1, 1, 128).expand_as(wl.v_src).contiguous()
    pool = H.device_pool(wl)
    o, _ = H.DeviceCall(wl, wl.calls[0]).run(pool)
    assert (o.float().cpu() - c.float()).abs().max().item() <= 2e-2


def test_empty_batch_and_validation():
    wl = workloads.small("decode", num_q_heads=8, num_kv_heads=2, ctx_lens=(40,), seed=68)
    pool = H.device_pool(wl)
    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    e = torch.empty((0,), dtype=torch.int32, device="cuda")
    o, lse = pa.decode(pool, q, e, torch.zeros((0, 3), dtype=torch.int32, device="cuda"), 0.1,
                       max_ctx_len=40)
    assert o.numel() == 0
    bad = wl.calls[0].block_table.clone().cuda()
    bad[0, 0] = wl.num_blocks
    with pytest.raises(ValueError):
        pa.decode(pool, wl.calls[0].q.cuda(), wl.calls[0].ctx_lens.cuda(), bad, 0.1, validate=True)
