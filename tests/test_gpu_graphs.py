"""The library's calls inside a captured HIP graph.

Every entry point enqueues kernels only (no allocation, no memset, no host
synchronisation), so a serving loop can capture a step once and replay it.
A step of split-KV decode (with its merge), chunked prefill with key splits
(with its merge) and the fp8-product prefill is captured on preallocated
buffers; it is replayed several times, with other work and synchronisations
between the replays, each replay compared bit for bit with the same calls run
eagerly, also after the queries are refreshed in place.
"""
import pytest
import torch

import workloads
from tests import harness as H

pytestmark = pytest.mark.gpu

pa = pytest.importorskip("online_softmax_paged_amd")


def _log(msg):
    print(msg, flush=True)


class _Call:
    """One call's device inputs and preallocated outputs and workspace."""

    def __init__(self, wl, call, pool, num_splits, fp8_products=False):
        self.dc = H.DeviceCall(wl, call)
        self.pool, self.wl, self.S, self.f8 = pool, wl, num_splits, fp8_products
        B, Hq, D = len(call.q_lens), wl.num_q_heads, wl.head_dim
        self.o = torch.empty_like(self.dc.q)
        self.lse = torch.empty(self.dc.q.shape[:2], dtype=torch.float32, device="cuda")
        if self.dc.kind == "prefill":
            n = pa.prefill_workspace_bytes(B, self.dc.max_q_len, Hq, D, num_splits)
        else:
            n = pa.decode_workspace_bytes(B, Hq, D, num_splits)
        self.ws = torch.empty(max(1, n), dtype=torch.uint8, device="cuda")

    def run(self):
        dc = self.dc
        if dc.kind == "prefill":
            pa.prefill(self.pool, dc.q, dc.cu_q_lens, dc.ctx_lens, dc.block_table, dc.scale,
                       causal=dc.causal, max_q_len=dc.max_q_len, max_ctx_len=dc.max_ctx_len,
                       out=self.o, lse=self.lse, num_splits=self.S, workspace=self.ws,
                       fp8_products=self.f8)
        else:
            pa.decode(self.pool, dc.q, dc.ctx_lens, dc.block_table, dc.scale,
                      max_ctx_len=dc.max_ctx_len, num_splits=self.S, workspace=self.ws,
                      out=self.o, lse=self.lse)

    def result(self):
        return self.o.clone(), self.lse.clone()


def test_captured_step_replays_match_eager_runs():
    dec_wl = workloads.small("decode", kv_dtype="bf16", q_dtype="bf16", num_q_heads=8,
                             num_kv_heads=2, head_dim=128, ctx_lens=(900, 40, 333, 1200),
                             seed=301)
    pre_wl = workloads.small("prefill", kv_dtype="bf16", q_dtype="bf16", num_q_heads=8,
                             num_kv_heads=2, head_dim=128, ctx_lens=(700, 260),
                             q_lens=(64, 100), seed=302)
    f8_wl = workloads.small("prefill", kv_dtype="fp8", q_dtype="bf16", num_q_heads=8,
                            num_kv_heads=2, head_dim=128, ctx_lens=(500, 300),
                            q_lens=(40, 60), seed=303)
    calls = [_Call(dec_wl, dec_wl.calls[0], H.device_pool(dec_wl), 3),
             _Call(pre_wl, pre_wl.calls[0], H.device_pool(pre_wl), 3),
             _Call(f8_wl, f8_wl.calls[0], H.device_pool(f8_wl), 2, fp8_products=True)]

    def step():
        for c in calls:
            c.run()

    # eager reference (and the warmup the capture wants, on a side stream)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [c.result() for c in calls]
    # the eager results are the right ones
    for c, (o, lse) in zip(calls, eager):
        ro, rl = H.oracle_call(H.oracle_pool(c.wl), c.wl, c.wl.calls[0])
        eo, el = H.max_err(o, lse, ro, rl)
        bar = H.TOL["fp8"] if c.f8 else H.tolerance(c.wl)
        assert eo <= bar and el <= bar, (c.dc.kind, eo, el)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for c in calls:  # clobber the outputs, so a replay that writes nothing fails
            c.o.fill_(float("nan"))
            c.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, c in enumerate(calls):
            o, lse = c.result()
            assert torch.equal(o, eager[i][0]) and torch.equal(lse, eager[i][1]), (rep, i)
        # unrelated eager work between replays
        x = torch.randn(1 << 20, device="cuda")
        (x * x).sum().item()
    _log("  3 replays bitwise equal to the eager step")

    # new queries, written in place: the replay reads them
    gen = torch.Generator(device="cpu").manual_seed(304)
    for c in calls:
        c.dc.q.copy_(torch.randn(c.dc.q.shape, generator=gen).to(c.dc.q.dtype))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    replayed = [c.result() for c in calls]
    step()
    torch.cuda.synchronize()
    for i, c in enumerate(calls):
        o, lse = c.result()
        assert torch.equal(o, replayed[i][0]) and torch.equal(lse, replayed[i][1]), i
        assert not torch.equal(o, eager[i][0]), i
    _log("  replay after an in-place query update equals the eager step on the new queries")
