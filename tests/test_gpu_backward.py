"""GPU parity of the backward (dQ, dK, dV) against the float64 backward
oracle, through the C ABI.  The forward's o and lse come from the library's
own pa_prefill; the oracle recomputes everything from the same seeded Q, K,
V and dO.

Bar: max |g - g_ref| <= 2e-2 * max(1, max |g_ref|) for each of dQ, dK and dV
(bf16 inputs; P and dS are rounded to bf16 before their MFMAs and O is the
forward's bf16 output, each a relative 2^-9 per element -- the same rounding
budget as the forward's 2e-2 bar, applied to the gradients' own scale).
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import paged_attention_backward
from tests import harness as H

pytestmark = pytest.mark.gpu

pa = pytest.importorskip("online_softmax_paged_amd")

REL = 2e-2


def _log(msg):
    print(msg, flush=True)


def _run_backward(wl, call, seed, causal=True, **kw):
    pool = H.device_pool(wl)
    dc = H.DeviceCall(wl, call)
    o, lse = pa.prefill(pool, dc.q, dc.cu_q_lens, dc.ctx_lens, dc.block_table, wl.scale,
                        causal=causal, max_q_len=dc.max_q_len, max_ctx_len=dc.max_ctx_len,
                        num_splits=1)
    do = workloads.upstream_grad(call, wl.head_dim, wl.num_q_heads, seed)
    dq, dk, dv = pa.prefill_backward(pool, dc.q, o, lse, do.cuda(), dc.cu_q_lens, dc.ctx_lens,
                                     dc.block_table, wl.scale, causal=causal,
                                     max_q_len=dc.max_q_len, max_ctx_len=dc.max_ctx_len,
                                     validate=True, **kw)
    torch.cuda.synchronize()
    return do, dq, dk, dv


def _check(wl, call, do, dq, dk, dv, causal=True):
    ref_q, ref_k, ref_v = paged_attention_backward(H.oracle_pool(wl), call.q, do, call.cu_q_lens,
                                                   call.ctx_lens, call.block_table,
                                                   wl.num_q_heads, wl.scale, causal)
    errs = {}
    for name, got, ref in (("dQ", dq, ref_q), ("dK", dk, ref_k), ("dV", dv, ref_v)):
        g = got.detach().cpu().to(torch.float64).numpy()
        assert np.isfinite(g).all(), f"{name}: non-finite"
        err = float(np.abs(g - ref).max())
        bound = REL * max(1.0, float(np.abs(ref).max()))
        errs[name] = (err, bound)
        assert err <= bound, (name, err, bound)
    _log("  " + " ".join(f"{k}: {e:.2e} (bar {b:.2e})" for k, (e, b) in errs.items()))


BACKWARD_CASES = [
    # D, Hq, Hkv, ctx_lens, q_lens (None = whole sequences), causal
    (128, 8, 2, (100, 37, 300), None, True),
    (128, 8, 2, (300, 129, 70, 16), (64, 1, 70, 5), True),     # chunks, a decode row, ragged tails
    (128, 8, 2, (200, 45), (60, 45), False),
    (64, 4, 4, (257, 33), None, True),                          # G = 1
    (128, 16, 2, (150, 90), (150, 17), True),                   # G = 8
    (64, 16, 1, (70,), None, True),                             # G = 16
]


@pytest.mark.parametrize("D,Hq,Hkv,ctx,ql,causal", BACKWARD_CASES)
def test_backward_parity(D, Hq, Hkv, ctx, ql, causal):
    _log(f"backward D={D} Hq={Hq} Hkv={Hkv} ctx={ctx} q={ql} causal={causal}")
    wl = workloads.small("prefill", kv_dtype="bf16", q_dtype="bf16", num_q_heads=Hq,
                         num_kv_heads=Hkv, head_dim=D, ctx_lens=ctx, q_lens=ql, seed=110 + D + Hq,
                         causal=causal)
    call = wl.calls[0]
    do, dq, dk, dv = _run_backward(wl, call, seed=7, causal=causal)
    _check(wl, call, do, dq, dk, dv, causal)


def test_backward_is_deterministic_and_reuses_its_workspace():
    wl = workloads.small("prefill", kv_dtype="bf16", q_dtype="bf16", num_q_heads=8,
                         num_kv_heads=2, head_dim=128, ctx_lens=(333, 80), q_lens=(100, 80),
                         seed=121)
    call = wl.calls[0]
    ws = torch.full((1 << 26,), 0x7F, dtype=torch.uint8, device="cuda")
    _, a_q, a_k, a_v = _run_backward(wl, call, seed=3, workspace=ws)
    _, b_q, b_k, b_v = _run_backward(wl, call, seed=3, workspace=ws)
    assert torch.equal(a_q, b_q) and torch.equal(a_k, b_k) and torch.equal(a_v, b_v)


def test_backward_prefill_1x2048_sampled_against_oracle():
    """One 2048-token causal sequence, 32 q / 8 KV heads, d=128: every
    gradient against the oracle (a few seconds of float64 on the CPU)."""
    _log("backward 1 x 2048")
    wl = workloads.build("bwd_2048", kv_dtype="bf16", q_dtype="bf16", num_q_heads=32,
                         num_kv_heads=8, head_dim=128, ctx_lens=[2048],
                         calls=[workloads.Call("prefill", [0], [2048])], seed=131)
    call = wl.calls[0]
    do, dq, dk, dv = _run_backward(wl, call, seed=5)
    _check(wl, call, do, dq, dk, dv)


def test_backward_bench_shape_sampled_pairs_against_oracle():
    """The benchmark's backward, 4 x 4096 causal, 32 q / 8 KV heads, d=128, in
    the launch bench.py times (forward unsplit, dO from its seed).  Every
    gradient is finite; three (sequence, KV head) pairs -- first, middle and
    last -- are checked whole against the dense float64 backward of
    oracle/backward.py: dQ of their 4 x 4096 query rows and dK, dV of all
    their 256 pages (every workgroup of those pairs, both kernels)."""
    from oracle import gather_kv
    from oracle.backward import attention_backward_dense
    _log("backward 4 x 4096 (bench shape), sampled pairs")
    wl = workloads.causal_prefill_bf16()
    call = wl.calls[0]
    pool = H.device_pool(wl)
    dc = H.DeviceCall(wl, call)
    o, lse = pa.prefill(pool, dc.q, dc.cu_q_lens, dc.ctx_lens, dc.block_table, wl.scale,
                        max_q_len=dc.max_q_len, max_ctx_len=dc.max_ctx_len, num_splits=1)
    T, Hq, D = dc.q.shape
    do = workloads.upstream_grad(call, D, Hq, seed=2024)
    dq = torch.empty((T, Hq, D), dtype=torch.float32, device="cuda")
    dk = torch.zeros(pool.k.shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros(pool.v.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(pa.backward_workspace_bytes(pool, len(call.q_lens), Hq, dc.max_q_len),
                     dtype=torch.uint8, device="cuda")
    pa.prefill_backward(pool, dc.q, o, lse, do.cuda(), dc.cu_q_lens, dc.ctx_lens, dc.block_table,
                        wl.scale, max_q_len=dc.max_q_len, max_ctx_len=dc.max_ctx_len, dq=dq,
                        dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    dq, dk, dv = (x.cpu().to(torch.float64).numpy() for x in (dq, dk, dv))
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    opool = H.oracle_pool(wl)
    G = Hq // wl.num_kv_heads
    qf, dof = call.q.to(torch.float64).numpy(), do.to(torch.float64).numpy()
    cu, bt = call.cu_q_lens.tolist(), call.block_table.numpy()
    for b, g in ((0, 0), (2, 3), (3, 7)):
        c = int(call.ctx_lens[b])
        q0, q1 = cu[b], cu[b + 1]
        pos = c - (q1 - q0) + np.arange(q1 - q0)
        K, V = gather_kv(opool, bt[b], c, g)
        dk_ref, dv_ref = np.zeros((c, D)), np.zeros((c, D))
        dq_err = dq_max = 0.0
        for h in range(g * G, (g + 1) * G):
            rq, rk, rv = attention_backward_dense(qf[q0:q1, h], K, V, dof[q0:q1, h], wl.scale,
                                                  pos, True)
            dq_err = max(dq_err, float(np.abs(dq[q0:q1, h] - rq).max()))
            dq_max = max(dq_max, float(np.abs(rq).max()))
            dk_ref += rk
            dv_ref += rv
        pages = bt[b][np.arange(c) // 16]
        slots = np.arange(c) % 16
        dk_got = dk[pages, g, slots, :]
        dv_got = dv[pages, g, :, slots]
        dk_err = float(np.abs(dk_got - dk_ref).max())
        dv_err = float(np.abs(dv_got - dv_ref).max())
        bars = [REL * max(1.0, m) for m in (dq_max, float(np.abs(dk_ref).max()),
                                             float(np.abs(dv_ref).max()))]
        _log(f"  pair ({b},{g}): dQ {dq_err:.2e} (bar {bars[0]:.2e}) dK {dk_err:.2e} "
             f"(bar {bars[1]:.2e}) dV {dv_err:.2e} (bar {bars[2]:.2e})")
        assert dq_err <= bars[0] and dk_err <= bars[1] and dv_err <= bars[2]


def _random_cases(n, seed):
    import random
    rng = random.Random(seed)
    out = []
    for i in range(n):
        D = rng.choice([64, 128])
        Hkv = rng.choice([1, 2, 4])
        G = rng.choice([1, 2, 4, 8])
        B = rng.randint(1, 4)
        ctx = [rng.choice([rng.randint(1, 40), rng.randint(1, 400), 16 * rng.randint(1, 20),
                           32 * rng.randint(1, 12) + 1]) for _ in range(B)]
        ql = [rng.choice([1, c, rng.randint(1, c)]) for c in ctx]
        out.append((i, D, Hkv * G, Hkv, tuple(ctx), tuple(ql), rng.random() < 0.8))
    return out


@pytest.mark.parametrize("i,D,Hq,Hkv,ctx,ql,causal", _random_cases(8, 17),
                         ids=lambda v: None)
def test_backward_random_shapes(i, D, Hq, Hkv, ctx, ql, causal):
    """A seeded random sweep of small shapes (head dims, group sizes, ragged
    lengths, chunks of 1 token to the whole context, causal or not)."""
    _log(f"backward random {i}: D={D} Hq={Hq} Hkv={Hkv} ctx={ctx} q={ql} causal={causal}")
    wl = workloads.small("prefill", kv_dtype="bf16", q_dtype="bf16", num_q_heads=Hq,
                         num_kv_heads=Hkv, head_dim=D, ctx_lens=ctx, q_lens=ql, seed=400 + i,
                         causal=causal)
    call = wl.calls[0]
    do, dq, dk, dv = _run_backward(wl, call, seed=11 + i, causal=causal)
    _check(wl, call, do, dq, dk, dv, causal)
