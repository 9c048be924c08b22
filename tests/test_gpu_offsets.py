"""Pages past 4 GiB: every kernel's byte offsets into the pools are 64-bit.

The same small workloads are written once into the first pages of a pool and
once into pages whose (page, KV head) chunks start beyond 2^32 bytes of a pool
of more than 4 GiB; slot mappings and block tables are relabelled by the same
page shift.  Where a page sits physically must not change any result (the
relabelling invariance the oracle is pinned to), so the two runs agree bit
for bit, in the same launch configurations; the low-page run is held to the
oracle as in the other parity tests.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import paged_attention_backward
from tests import harness as H

pytestmark = pytest.mark.gpu

pa = pytest.importorskip("online_softmax_paged_amd")


def _log(msg):
    print(msg, flush=True)


def _high_pool(wl):
    """A pool whose first written page starts past 2^32 bytes, and the shift."""
    es = {"f32": 4, "bf16": 2, "fp8": 1}[wl.kv_dtype]
    page_bytes = wl.num_kv_heads * 16 * wl.head_dim * es
    base = (1 << 32) // page_bytes + 1
    pool = pa.KVPool(base + wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
    slots = torch.where(wl.slot_mapping >= 0, wl.slot_mapping + base * 16, wl.slot_mapping)
    pa.write_kv(pool, wl.k_src.cuda(), wl.v_src.cuda(), slots.cuda())
    assert base * page_bytes > (1 << 32)
    return pool, base


def _calls(wl, call, base):
    lo = H.DeviceCall(wl, call)
    hi = H.DeviceCall(wl, call)
    bt = call.block_table.clone()
    hi.block_table = torch.where(bt >= 0, bt + base, bt).cuda()
    return lo, hi


def _same(a, b, what):
    for x, y in zip(a, b):
        assert torch.equal(x, y), what


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefill_and_decode_on_pages_past_4gib(kv):
    _log(f"pages past 4 GiB, {kv} pool: prefill, decode")
    pre = workloads.small("prefill", kv_dtype=kv, q_dtype="bf16", num_q_heads=8, num_kv_heads=2,
                          head_dim=128, ctx_lens=(300, 77, 129), q_lens=(300, 30, 1), seed=211)
    dec = workloads.small("decode", kv_dtype=kv, q_dtype="bf16", num_q_heads=8, num_kv_heads=2,
                          head_dim=128, ctx_lens=(1500, 33, 260, 700), seed=212)
    tol = H.tolerance(pre)
    for wl in (pre, dec):
        lo_pool = H.device_pool(wl)
        hi_pool, base = _high_pool(wl)
        call = wl.calls[0]
        lo, hi = _calls(wl, call, base)
        ro, rl = H.oracle_call(H.oracle_pool(wl), wl, call)
        runs = [dict(num_splits=0), dict(num_splits=3)]
        if call.kind == "decode":
            runs.append(dict(num_splits=pa.DECODE_BALANCED))
        elif kv == "fp8":
            runs += [dict(num_splits=1, fp8_products=True), dict(num_splits=3, fp8_products=True)]
        for kw in runs:
            a = lo.run(lo_pool, **kw)
            b = hi.run(hi_pool, **kw)
            torch.cuda.synchronize()
            _same(a, b, f"{call.kind} {kw}")
            if not kw.get("fp8_products"):
                eo, el = H.max_err(a[0], a[1], ro, rl)
                _log(f"  {call.kind} {kw}: bitwise equal; oracle max|dO|={eo:.2e} max|dLSE|={el:.2e}")
                assert eo <= tol and el <= tol
            else:
                _log(f"  {call.kind} {kw}: bitwise equal")
        del hi_pool
        torch.cuda.empty_cache()


def test_backward_on_pages_past_4gib():
    _log("pages past 4 GiB, bf16 pool: backward")
    wl = workloads.small("prefill", kv_dtype="bf16", q_dtype="bf16", num_q_heads=8,
                         num_kv_heads=2, head_dim=128, ctx_lens=(200, 45), q_lens=(200, 20),
                         seed=213)
    call = wl.calls[0]
    lo_pool = H.device_pool(wl)
    hi_pool, base = _high_pool(wl)
    lo, hi = _calls(wl, call, base)
    do = workloads.upstream_grad(call, wl.head_dim, wl.num_q_heads, 214).cuda()
    grads = []
    for dc, pool in ((lo, lo_pool), (hi, hi_pool)):
        o, lse = dc.run(pool, num_splits=1)
        grads.append(pa.prefill_backward(pool, dc.q, o, lse, do, dc.cu_q_lens, dc.ctx_lens,
                                         dc.block_table, wl.scale, causal=True,
                                         max_q_len=dc.max_q_len, max_ctx_len=dc.max_ctx_len,
                                         validate=True))
    torch.cuda.synchronize()
    (dq0, dk0, dv0), (dq1, dk1, dv1) = grads
    assert torch.equal(dq0, dq1)
    # the high pool's gradients sit at the shifted pages; all others stay zero
    assert torch.equal(dk1[base:], dk0) and torch.equal(dv1[base:], dv0)
    assert not dk1[:base].any() and not dv1[:base].any()
    ref_q, ref_k, ref_v = paged_attention_backward(H.oracle_pool(wl), call.q, do.cpu(),
                                                   call.cu_q_lens, call.ctx_lens, call.block_table,
                                                   wl.num_q_heads, wl.scale, True)
    for got, ref in ((dq0, ref_q), (dk0, ref_k), (dv0, ref_v)):
        g = got.cpu().to(torch.float64).numpy()
        assert np.abs(g - ref).max() <= 2e-2 * max(1.0, float(np.abs(ref).max()))
    _log("  backward: bitwise equal, low pages within the backward bar")
