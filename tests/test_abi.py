"""Host-side tests of the C ABI (no GPU needed; nothing here launches a kernel).

The library must load and export every function include/pa.h declares; the
block allocator is pure host code; argument checks must return an error
status before anything is enqueued.
"""
import ctypes
import os
import re

import pytest

import online_softmax_paged_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 15
    lib = ctypes.CDLL(pa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in pa.h but not exported"
    assert sorted(pa.EXPORTED) == names


def test_status_strings_and_version():
    assert pa.abi_version() == 8
    assert pa.status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert pa.status_string(s) and pa.status_string(s) != "unknown status"
    assert pa.status_string(7) == "unknown status"


def test_allocator_alloc_free_refcount():
    a = pa.BlockAllocator(4)
    assert a.num_free() == 4
    ids = [a.alloc() for _ in range(4)]
    assert ids == [0, 1, 2, 3]
    assert a.alloc() == -1                       # exhausted
    a.incref(2)
    a.incref(2)
    assert a.refcount(2) == 3
    a.decref(2)
    a.decref(2)
    assert a.refcount(2) == 1 and a.num_free() == 0
    a.decref(2)
    assert a.refcount(2) == 0 and a.num_free() == 1
    with pytest.raises(pa.PAError) as e:
        a.decref(2)                              # double free
    assert e.value.status == pa.PA_ERR_INVALID_ARG
    with pytest.raises(pa.PAError):
        a.incref(2)                              # sharing a free block
    with pytest.raises(pa.PAError):
        a.decref(17)
    assert a.refcount(-1) == -1 and a.refcount(4) == -1
    assert a.alloc() == 2                        # lowest free id first


def test_allocator_shared_prefix_lifecycle():
    """16 sequences share 4 prefix blocks (one reference each) and own 2 each;
    ending every sequence returns every block."""
    a = pa.BlockAllocator(64)
    prefix = [a.alloc() for _ in range(4)]
    for _ in range(15):
        for p in prefix:
            a.incref(p)
    own = [[a.alloc(), a.alloc()] for _ in range(16)]
    assert all(a.refcount(p) == 16 for p in prefix)
    assert a.num_free() == 64 - 4 - 32
    for s in range(16):
        for p in prefix + own[s]:
            a.decref(p)
    assert a.num_free() == 64
    with pytest.raises(ValueError):
        pa.BlockAllocator(0)


class _FakePool:
    """A pool descriptor pointing at fake (never dereferenced) addresses."""

    def __init__(self, **kw):
        f = dict(k=0x1000, v=0x2000, k_scale=0x3000, v_scale=0x4000, num_blocks=8,
                 num_kv_heads=2, head_dim=128, block_size=16, kv_dtype=pa.PA_BF16)
        f.update(kw)
        self._c = pa._Pool(f["k"], f["v"], f["k_scale"], f["v_scale"], f["num_blocks"],
                           f["num_kv_heads"], f["head_dim"], f["block_size"], f["kv_dtype"])
        self.c = ctypes.byref(self._c)


def _prefill(pool, **kw):
    a = dict(q=0x5000, q_dtype=pa.PA_BF16, o=0x6000, lse=0x7000, cu=0x8000, ctx=0x9000,
             bt=0xa000, stride=4, B=2, Hq=8, max_q=64, max_ctx=64, scale=0.1, causal=1,
             splits=1, ws=0, ws_bytes=0)
    a.update(kw)
    return pa._prefill(pool.c, a["q"], a["q_dtype"], a["o"], a["lse"], a["cu"], a["ctx"], a["bt"],
                       a["stride"], a["B"], a["Hq"], a["max_q"], a["max_ctx"], a["scale"],
                       a["causal"], a["splits"], a["ws"], a["ws_bytes"], None)


def _decode(pool, **kw):
    a = dict(q=0x5000, q_dtype=pa.PA_BF16, o=0x6000, lse=0x7000, ctx=0x9000, bt=0xa000,
             stride=4, B=2, Hq=8, max_ctx=64, scale=0.1, splits=2, ws=0, ws_bytes=0)
    a.update(kw)
    return pa._decode(pool.c, a["q"], a["q_dtype"], a["o"], a["lse"], a["ctx"], a["bt"],
                      a["stride"], a["B"], a["Hq"], a["max_ctx"], a["scale"], a["splits"],
                      a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("pool_kw,call_kw,want", [
    (dict(block_size=32), {}, pa.PA_ERR_UNSUPPORTED),
    (dict(head_dim=96), {}, pa.PA_ERR_UNSUPPORTED),
    (dict(k=0), {}, pa.PA_ERR_INVALID_ARG),
    (dict(k=0x1008), {}, pa.PA_ERR_INVALID_ARG),             # misaligned pool
    (dict(kv_dtype=pa.PA_FP8_E4M3, k_scale=0), {}, pa.PA_ERR_INVALID_ARG),
    ({}, dict(q_dtype=pa.PA_F32), pa.PA_ERR_UNSUPPORTED),    # f32 q with bf16 pool
    ({}, dict(Hq=6), pa.PA_ERR_UNSUPPORTED),                 # group of 3
    ({}, dict(Hq=7), pa.PA_ERR_INVALID_ARG),                 # not a multiple of Hkv
    ({}, dict(q=0x5004), pa.PA_ERR_INVALID_ARG),             # misaligned q
    ({}, dict(stride=3), pa.PA_ERR_INVALID_ARG),             # table narrower than max ctx
    ({}, dict(max_q=65), pa.PA_ERR_INVALID_ARG),             # max_q_len > max_ctx_len
    ({}, dict(cu=0), pa.PA_ERR_INVALID_ARG),
    ({}, dict(scale=float("nan")), pa.PA_ERR_INVALID_ARG),
    ({}, dict(B=-1), pa.PA_ERR_INVALID_ARG),
])
def test_prefill_rejects_bad_arguments(pool_kw, call_kw, want):
    assert _prefill(_FakePool(**pool_kw), **call_kw) == want


def test_empty_batch_is_a_no_op():
    assert _prefill(_FakePool(), B=0) == pa.PA_OK
    assert _decode(_FakePool(), B=0) == pa.PA_OK


def test_decode_workspace_checks():
    need = pa.decode_workspace_bytes(2, 8, 128, 2)
    assert need >= 2 * 8 * 2 * (128 + 1) * 4
    assert pa.decode_workspace_bytes(2, 8, 128, 1) == 0
    assert _decode(_FakePool(), ws=0) == pa.PA_ERR_WORKSPACE
    assert _decode(_FakePool(), ws=0x10000, ws_bytes=need - 1) == pa.PA_ERR_WORKSPACE
    assert _decode(_FakePool(), ws=0x10008, ws_bytes=need) == pa.PA_ERR_INVALID_ARG
    assert _decode(_FakePool(), splits=-2) == pa.PA_ERR_INVALID_ARG
    # balanced decode: its own workspace, none given
    assert _decode(_FakePool(), splits=pa.DECODE_BALANCED, ws=0) == pa.PA_ERR_WORKSPACE
    nb = pa.decode_balanced_workspace_bytes(2, 8, 2, 128, 64)
    assert nb >= 8 * (4 * 1 + 2) * (128 + 1) * 4   # 64 tokens x 2 seqs -> one workgroup per head
    assert _decode(_FakePool(), splits=pa.DECODE_BALANCED, ws=0x10000,
                   ws_bytes=nb - 1) == pa.PA_ERR_WORKSPACE
    assert _decode(_FakePool(kv_dtype=pa.PA_F32), q_dtype=pa.PA_F32, splits=pa.DECODE_BALANCED,
                   ws=0x10000, ws_bytes=nb) == pa.PA_ERR_UNSUPPORTED


def test_prefill_split_checks_and_heuristic():
    need = pa.prefill_workspace_bytes(2, 64, 8, 128, 3)
    assert need >= 3 * 2 * 64 * 8 * (128 + 1) * 4
    assert pa.prefill_workspace_bytes(2, 64, 8, 128, 1) == 0
    assert _prefill(_FakePool(), splits=3, ws=0) == pa.PA_ERR_WORKSPACE
    assert _prefill(_FakePool(), splits=3, ws=0x10000, ws_bytes=need - 1) == pa.PA_ERR_WORKSPACE
    assert _prefill(_FakePool(), splits=3, ws=0x10008, ws_bytes=need) == pa.PA_ERR_INVALID_ARG
    assert _prefill(_FakePool(), splits=17) == pa.PA_ERR_INVALID_ARG
    # many query tiles: no split; few query tiles over long contexts: split
    assert pa.prefill_num_splits(4, 8, 32, 4096, 4096) == 1
    assert pa.prefill_num_splits(8, 8, 32, 256, 1536) == 1
    assert pa.prefill_num_splits(1, 8, 32, 256, 8192) == 8
    assert pa.prefill_num_splits(1, 1, 1, 10, 100) == 1


def _shared(pool, plan=(1, 1, 1, 1), **kw):
    """pa_prefill_shared_prefix through the C ABI; plan = (mode, prefix, suffix,
    plain splits) or None for the library's choice."""
    a = dict(q=0x5000, q_dtype=pa.PA_BF16, o=0x6000, lse=0x7000, cu=0x8000, ctx=0x9000,
             bt=0xa000, stride=8, B=2, Hq=8, max_q=32, max_ctx=128, scale=0.1, causal=1,
             prefix=64, T=40, ws=0, ws_bytes=0)
    a.update(kw)
    cp = None if plan is None else ctypes.byref(pa._SharedPlan(*plan, 0))
    return pa._prefill_sp(pool.c, a["q"], a["q_dtype"], a["o"], a["lse"], a["cu"], a["ctx"],
                          a["bt"], a["stride"], a["B"], a["Hq"], a["max_q"], a["max_ctx"],
                          a["scale"], a["causal"], a["prefix"], a["T"], cp, a["ws"],
                          a["ws_bytes"], None)


def _plan(**kw):
    return dict(zip(("mode", "prefix_splits", "suffix_splits", "plain_splits"),
                    kw.get("t", (pa.SHARED_PACKED, 1, 1, 1))))


def test_shared_prefix_checks():
    p = _FakePool()
    # packed, mixed batch: gathered decode rows + partials of both packed passes
    need = pa.shared_prefix_workspace_bytes(p, 2, 8, 32, _plan())
    assert need >= 2 * 8 * 128 * 2 + 2 * 2 * 8 * (128 + 1) * 4
    need3 = pa.shared_prefix_workspace_bytes(p, 2, 8, 32, _plan(t=(pa.SHARED_PACKED, 1, 1, 3)))
    assert need3 >= need + 3 * 2 * 32 * 8 * (128 + 1) * 4   # partials of the q_len > 1 rows
    # packed, decode rows only: no gather
    assert pa.shared_prefix_workspace_bytes(p, 2, 8, 1, _plan()) >= 2 * 2 * 8 * 129 * 4
    # plain: pa_decode's / pa_prefill's workspace
    assert pa.shared_prefix_workspace_bytes(p, 2, 8, 1, _plan(t=(pa.SHARED_PLAIN, 0, 0, 1))) == 0
    assert (pa.shared_prefix_workspace_bytes(p, 2, 8, 32, _plan(t=(pa.SHARED_PLAIN, 0, 0, 3)))
            == pa.prefill_workspace_bytes(2, 32, 8, 128, 3))
    for bad in ((3, 1, 1, 1), (pa.SHARED_AUTO, 1, 1, 1), (pa.SHARED_PACKED, 17, 1, 1),
                (pa.SHARED_PACKED, 1, 65, 1), (pa.SHARED_PACKED, 1, 0, 1),
                (pa.SHARED_PACKED, 1, 1, 17), (pa.SHARED_PLAIN, 0, 0, 17)):
        assert pa.shared_prefix_workspace_bytes(p, 2, 8, 32, _plan(t=bad)) == 0, bad
        assert _shared(p, plan=bad, ws=0x10000, ws_bytes=1 << 30) == pa.PA_ERR_INVALID_ARG, bad
    assert _shared(_FakePool(kv_dtype=pa.PA_F32), q_dtype=pa.PA_F32) == pa.PA_ERR_UNSUPPORTED
    assert _shared(p) == pa.PA_ERR_WORKSPACE                       # packed needs a workspace
    assert _shared(p, ws=0x10000, ws_bytes=need - 1) == pa.PA_ERR_WORKSPACE
    assert _shared(p, ws=0x10008, ws_bytes=need) == pa.PA_ERR_INVALID_ARG   # misaligned
    assert _shared(p, plan=(pa.SHARED_PLAIN, 0, 0, 3)) == pa.PA_ERR_WORKSPACE
    for bad in (dict(prefix=0), dict(prefix=24), dict(prefix=112),  # not whole pages; no room
                dict(T=0), dict(T=65), dict(cu=0), dict(max_q=0)):
        assert _shared(p, **bad) == pa.PA_ERR_INVALID_ARG, bad
        assert _shared(p, plan=None, **bad) == pa.PA_ERR_INVALID_ARG, bad
    assert _shared(p, B=0) == pa.PA_OK
    # one query per sequence: the decode pass takes row b as sequence b
    assert _shared(p, max_q=1, T=1) == pa.PA_ERR_INVALID_ARG
    assert _shared(p, max_q=1, T=2) == pa.PA_ERR_WORKSPACE        # rows == sequences: accepted
    with pytest.raises(pa.PAError):
        pa.shared_prefix_plan(p, 1, 8, 1, 64, 64, 1)             # no room past the prefix
    with pytest.raises(pa.PAError):
        pa.shared_prefix_plan(p, 2, 8, 32, 128, 64, 40, mode=7)


def test_shared_prefix_plan_choice():
    """Packing is chosen only where the prefix reads it saves outweigh its
    extra passes; a forced mode is kept."""
    bf16 = _FakePool(num_kv_heads=8, num_blocks=1 << 16)
    fp8 = _FakePool(num_kv_heads=8, num_blocks=1 << 16, kv_dtype=pa.PA_FP8_E4M3)
    # 64 decode rows over a 4096-token bf16 prefix: 1 GiB of prefix reads saved
    pl = pa.shared_prefix_plan(bf16, 64, 32, 1, 4608, 4096, 64)
    assert pl["mode"] == pa.SHARED_PACKED and pl["workspace_bytes"] > 0
    # 16 decode rows over a 1024-token fp8 prefix: 31 MB, not worth the passes
    assert pa.shared_prefix_plan(fp8, 16, 32, 1, 1536, 1024, 16)["mode"] == pa.SHARED_PLAIN
    # the mixed fp8 step (8 chunks of 256 and 8 decode rows): at most 8 rows
    # can be decode rows, so plain
    pl = pa.shared_prefix_plan(fp8, 16, 32, 256, 1536, 1024, 2056)
    assert pl["mode"] == pa.SHARED_PLAIN and pl["plain_splits"] == 1
    # 64 decode rows and one 256-token chunk over a 4096-token prefix: packed
    pl = pa.shared_prefix_plan(bf16, 65, 32, 256, 4608, 4096, 320)
    assert pl["mode"] == pa.SHARED_PACKED
    # forced modes are kept
    assert pa.shared_prefix_plan(fp8, 16, 32, 256, 1536, 1024, 2056,
                                 mode=pa.SHARED_PACKED)["mode"] == pa.SHARED_PACKED
    assert pa.shared_prefix_plan(bf16, 64, 32, 1, 4608, 4096, 64,
                                 mode=pa.SHARED_PLAIN)["mode"] == pa.SHARED_PLAIN
    # the packed prefix pass has few query tiles, so its keys split
    pl = pa.shared_prefix_plan(bf16, 8, 32, 1, 32768, 32768 - 64, 8, mode=pa.SHARED_PACKED)
    assert pl["prefix_splits"] > 1 and pl["suffix_splits"] == 1


def _backward(pool, **kw):
    a = dict(q=0x5000, o=0x6000, lse=0x7000, dout=0x8000, q_dtype=pa.PA_BF16, dq=0x9000,
             dk=0xa000, dv=0xb000, cu=0xc000, ctx=0xd000, bt=0xe000, stride=4, B=2, Hq=8,
             max_q=64, max_ctx=64, scale=0.1, causal=1, ws=0, ws_bytes=0)
    a.update(kw)
    return pa._bwd(pool.c, a["q"], a["o"], a["lse"], a["dout"], a["q_dtype"], a["dq"], a["dk"],
                   a["dv"], a["cu"], a["ctx"], a["bt"], a["stride"], a["B"], a["Hq"], a["max_q"],
                   a["max_ctx"], a["scale"], a["causal"], a["ws"], a["ws_bytes"], None)


def test_backward_checks():
    p = _FakePool()
    need = pa._bwd_ws(p.c, 2, 8, 64)
    # Q^T and dO^T: 2 KV heads x 128 features x 2 sequences x 256 rows, bf16
    assert need >= 2 * (2 * 128 * 2 * 256 * 2)
    assert pa._bwd_ws(p.c, 0, 8, 64) == 0
    assert _backward(_FakePool(kv_dtype=pa.PA_F32), q_dtype=pa.PA_F32) == pa.PA_ERR_UNSUPPORTED
    assert _backward(_FakePool(kv_dtype=pa.PA_FP8_E4M3)) == pa.PA_ERR_UNSUPPORTED
    assert _backward(p) == pa.PA_ERR_WORKSPACE
    assert _backward(p, ws=0x100000, ws_bytes=need - 1) == pa.PA_ERR_WORKSPACE
    for bad in (dict(lse=0), dict(dout=0), dict(dq=0), dict(dk=0), dict(dv=0), dict(cu=0),
                dict(dq=0x9004), dict(dk=0xa008), dict(max_q=0), dict(max_q=65)):
        assert _backward(p, ws=0x100000, ws_bytes=need, **bad) == pa.PA_ERR_INVALID_ARG, bad
    assert _backward(p, ws=0x100008, ws_bytes=need) == pa.PA_ERR_INVALID_ARG
    assert _backward(p, B=0) == pa.PA_OK


def test_prefill_fp8_checks():
    def call(pool, **kw):
        a = dict(q=0x5000, q_dtype=pa.PA_BF16, o=0x6000, lse=0x7000, cu=0x8000, ctx=0x9000,
                 bt=0xa000, stride=4, B=2, Hq=8, max_q=64, max_ctx=64, scale=0.1, causal=1,
                 splits=1, ws=0, ws_bytes=0)
        a.update(kw)
        return pa._prefill_fp8(pool.c, a["q"], a["q_dtype"], a["o"], a["lse"], a["cu"], a["ctx"],
                               a["bt"], a["stride"], a["B"], a["Hq"], a["max_q"], a["max_ctx"],
                               a["scale"], a["causal"], a["splits"], a["ws"], a["ws_bytes"], None)
    assert call(_FakePool()) == pa.PA_ERR_UNSUPPORTED                       # bf16 pool
    assert call(_FakePool(kv_dtype=pa.PA_F32), q_dtype=pa.PA_F32) == pa.PA_ERR_UNSUPPORTED
    f = _FakePool(kv_dtype=pa.PA_FP8_E4M3)
    assert call(f, q_dtype=pa.PA_F32) == pa.PA_ERR_UNSUPPORTED
    assert call(f, splits=3) == pa.PA_ERR_WORKSPACE
    assert call(f, max_q=0) == pa.PA_ERR_INVALID_ARG
    assert call(f, B=0) == pa.PA_OK


def test_probe_checks():
    """Measurement probes reject bad arguments before any launch."""
    rd = lambda buf, n, out, blocks: pa._probe_read(buf, n, out, blocks, None)
    assert rd(0, 1 << 20, 0x2000, 64) == pa.PA_ERR_INVALID_ARG       # null buffer
    assert rd(0x1000, 1 << 20, 0, 64) == pa.PA_ERR_INVALID_ARG       # null output
    assert rd(0x1000, 1000, 0x2000, 64) == pa.PA_ERR_INVALID_ARG     # not a multiple of 16
    assert rd(0x1000, 0, 0x2000, 64) == pa.PA_ERR_INVALID_ARG
    assert rd(0x1000, 1 << 20, 0x2000, 0) == pa.PA_ERR_INVALID_ARG
    assert rd(0x1000, 1 << 20, 0x2000, 65536) == pa.PA_ERR_INVALID_ARG
    mf = lambda dt, out, blocks, iters: pa._probe_mfma(dt, out, blocks, iters, None)
    assert mf(pa.PA_F32, 0x2000, 64, 10) == pa.PA_ERR_UNSUPPORTED
    assert mf(pa.PA_BF16, 0, 64, 10) == pa.PA_ERR_INVALID_ARG
    assert mf(pa.PA_BF16, 0x2000, 64, 0) == pa.PA_ERR_INVALID_ARG
    assert mf(pa.PA_FP8_E4M3, 0x2000, 0, 10) == pa.PA_ERR_INVALID_ARG
    assert pa.PROBE_MFMA_FLOP == {"bf16": 32768, "fp8": 131072}


def test_decode_split_heuristic():
    # long context, few sequences: many splits; short contexts: few
    assert pa.decode_num_splits(8, 8, 32768) == 8
    assert pa.decode_num_splits(1, 1, 100) == 1
    # a workgroup per compute unit already: no split
    assert pa.decode_num_splits(32, 8, 2048) == 1
    assert pa.decode_num_splits(16, 8, 2048) == 4
    assert pa.decode_num_splits(0, 8, 100) == 1
    # uneven batches go to the balanced kernel, even ones keep the split choice
    assert pa.decode_choose_splits(32, 8, 32768, 32768 + 31 * 256) == pa.DECODE_BALANCED
    assert pa.decode_choose_splits(64, 8, 8192, 4 * 8192 + 60 * 128) == pa.DECODE_BALANCED
    assert pa.decode_choose_splits(32, 8, 2048, 32 * 1088) == 1
    assert pa.decode_choose_splits(8, 8, 32768, 8 * 32768) == 8
    assert pa.decode_choose_splits(8, 8, 32768, 0) == 8          # total unknown
    assert pa.decode_choose_splits(1, 8, 5000, 10) == pa.decode_num_splits(1, 8, 5000)


def test_write_kv_checks():
    p = _FakePool()
    assert pa._write(p.c, 0x1000, 0x2000, pa.PA_F32, 0x3000, 4, None, 0, None) == pa.PA_ERR_UNSUPPORTED
    assert pa._write(p.c, 0x1000, 0x2000, pa.PA_BF16, 0x3000, -1, None, 0, None) == pa.PA_ERR_INVALID_ARG
    assert pa._write(p.c, 0x1000, 0x2000, pa.PA_BF16, 0x3000, 0, None, 0, None) == pa.PA_OK
    f = _FakePool(kv_dtype=pa.PA_FP8_E4M3)
    assert pa._write_ws(f.c) == 3 * 4 * 8
    assert pa._write(f.c, 0x1000, 0x2000, pa.PA_BF16, 0x3000, 4, None, 0, None) == pa.PA_ERR_WORKSPACE


def test_decode_noalloc_checks():
    """Refusals come from host checks before the device array is looked up
    (no GPU needed)."""
    def call(**kw):
        a = dict(q=0x5000, q_dtype=pa.PA_BF16, o=0x6000, lse=0x7000, ctx=0x9000, bt=0xa000,
                 stride=2048, B=64, Hq=64, max_ctx=32768, scale=0.1, splits=256)
        a.update(kw)
        return pa._decode_noalloc(_FakePool(num_kv_heads=8).c, a["q"], a["q_dtype"], a["o"],
                                  a["lse"], a["ctx"], a["bt"], a["stride"], a["B"], a["Hq"],
                                  a["max_ctx"], a["scale"], a["splits"], None)
    assert pa.decode_workspace_bytes(64, 64, 128, 256) > pa.SCRATCH_BYTES
    assert call() == pa.PA_ERR_WORKSPACE                  # partials past the fixed array
    assert call(splits=257) == pa.PA_ERR_INVALID_ARG
    assert call(splits=-2) == pa.PA_ERR_INVALID_ARG
    assert call(q=0) == pa.PA_ERR_INVALID_ARG
    assert call(stride=3) == pa.PA_ERR_INVALID_ARG
    assert call(B=0) == pa.PA_OK
