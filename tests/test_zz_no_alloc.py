"""GPU test of pa_decode_noalloc, the decode entry point that allocates
nothing (its split partials live in the library's fixed per-device array):
through the C ABI its results equal pa_decode's bit for bit (same kernels,
same split count) and the oracle's within the dtype bound, on calls in a row
whose second input is smaller, and it refuses a split count whose partials
would not fit the array."""
import pytest
import torch

import workloads
from tests import harness as H

pytestmark = pytest.mark.gpu

pa = pytest.importorskip("online_softmax_paged_amd")


def _log(msg):
    print(msg, flush=True)


def _compare(wl, num_splits):
    call = [c for c in wl.calls if c.kind == "decode"][0]
    pool, opool = H.device_pool(wl), H.oracle_pool(wl)
    dc = H.DeviceCall(wl, call)
    B, Hq, _ = dc.q.shape
    S = num_splits or pa.decode_num_splits(B, wl.num_kv_heads, dc.max_ctx_len)
    o_ref, l_ref = pa.decode(pool, dc.q, dc.ctx_lens, dc.block_table, wl.scale,
                             max_ctx_len=dc.max_ctx_len, num_splits=S)
    o = torch.full_like(dc.q, float("nan"))
    lse = torch.full((B, Hq), float("inf"), dtype=torch.float32, device=dc.q.device)
    pa.decode_noalloc(pool, dc.q, dc.ctx_lens, dc.block_table, wl.scale, dc.max_ctx_len,
                      o, lse, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32))
    ro, rl = H.oracle_call(opool, wl, call)
    eo, el = H.max_err(o, lse, ro, rl)
    _log(f"  {wl.name} splits={S}: bit-identical to pa_decode; max|dO|={eo:.3e} "
         f"max|dLSE|={el:.3e} tol={H.tolerance(wl)}")
    assert eo <= H.tolerance(wl) and el <= H.tolerance(wl)


def test_decode_noalloc_equals_decode_on_calls_in_a_row():
    big = workloads.small("decode", kv_dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                          ctx_lens=(2000, 900, 1500, 333, 1234, 77), seed=81)
    small = workloads.small("decode", kv_dtype="fp8", num_q_heads=8, num_kv_heads=2,
                            head_dim=128, ctx_lens=(400, 37), seed=82)
    _log("decode_noalloc: larger batch, automatic split count")
    _compare(big, 0)
    _log("decode_noalloc: smaller batch after it")
    _compare(small, 0)
    _log("decode_noalloc: smaller batch, 3 splits and balanced")
    _compare(small, 3)
    _compare(small, pa.DECODE_BALANCED)


def test_decode_noalloc_refuses_partials_past_the_array():
    wl = workloads.small("decode", kv_dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                         ctx_lens=(4096,) * 8, seed=83)
    call = wl.calls[0]
    pool = H.device_pool(wl)
    dc = H.DeviceCall(wl, call)
    S = 256
    assert pa.decode_workspace_bytes(8, 32, 128, S) > pa.SCRATCH_BYTES
    o = torch.zeros_like(dc.q)
    lse = torch.zeros((8, 32), dtype=torch.float32, device=dc.q.device)
    with pytest.raises(pa.PAError) as e:
        pa.decode_noalloc(pool, dc.q, dc.ctx_lens, dc.block_table, wl.scale, dc.max_ctx_len,
                          o, lse, num_splits=S)
    assert e.value.status == pa.PA_ERR_WORKSPACE
