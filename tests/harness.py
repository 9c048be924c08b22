"""Shared plumbing of the GPU parity tests, the smoke check and the benchmark:
move a seeded workload to the device, run it through the library, and build
the oracle's answer from the same seeded inputs (never from device results).
"""
from __future__ import annotations

import numpy as np
import torch

import online_softmax_paged_amd as pa
import workloads
from oracle import OraclePool, write_kv as oracle_write_kv, paged_attention, paged_attention_rows

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}


def tolerance(wl) -> float:
    return TOL[wl.kv_dtype] if wl.kv_dtype == "fp8" else TOL[wl.q_dtype]


def oracle_pool(wl) -> OraclePool:
    p = OraclePool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
    oracle_write_kv(p, wl.k_src, wl.v_src, wl.slot_mapping)
    return p


def device_pool(wl, device="cuda") -> pa.KVPool:
    pool = pa.KVPool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.kv_dtype, device=device)
    pa.write_kv(pool, wl.k_src.to(device), wl.v_src.to(device), wl.slot_mapping.to(device))
    return pool


class DeviceCall:
    """A call's inputs resident on the device."""

    def __init__(self, wl, call, device="cuda"):
        self.kind = call.kind
        self.q = call.q.to(device)
        self.cu_q_lens = call.cu_q_lens.to(device)
        self.ctx_lens = call.ctx_lens.to(device)
        self.block_table = call.block_table.to(device)
        self.max_q_len = max(call.q_lens)
        self.max_ctx_len = int(call.ctx_lens.max())
        self.scale = wl.scale
        self.causal = call.causal

    def run(self, pool, num_splits=0, **kw):
        if self.kind == "prefill":
            return pa.prefill(pool, self.q, self.cu_q_lens, self.ctx_lens, self.block_table,
                              self.scale, causal=self.causal, max_q_len=self.max_q_len,
                              max_ctx_len=self.max_ctx_len, num_splits=num_splits, **kw)
        return pa.decode(pool, self.q, self.ctx_lens, self.block_table, self.scale,
                         max_ctx_len=self.max_ctx_len, num_splits=num_splits, **kw)


def oracle_call(opool, wl, call):
    return paged_attention(opool, call.q, call.cu_q_lens, call.ctx_lens, call.block_table,
                           wl.num_q_heads, wl.scale, call.causal)


def oracle_rows(opool, wl, call, rows):
    return paged_attention_rows(opool, call.q, call.cu_q_lens, call.ctx_lens, call.block_table,
                                wl.num_q_heads, wl.scale, rows, call.causal)


def max_err(gpu_o, gpu_lse, ref_o, ref_lse):
    """Max |difference| of outputs and of logsumexps (rows with -inf must match)."""
    go = gpu_o.detach().to(torch.float64).cpu().numpy()
    gl = gpu_lse.detach().to(torch.float64).cpu().numpy()
    assert np.isfinite(go).all(), "non-finite output"
    eo = float(np.abs(go - ref_o).max()) if go.size else 0.0
    fin = np.isfinite(ref_lse)
    assert (np.isfinite(gl) == fin).all(), "lse -inf pattern differs"
    el = float(np.abs(gl[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    return eo, el


def sample_rows(call, num_q_heads, n, seed=0):
    """(token, head) rows to check one by one: every sequence's first and last
    query token on the first and last head, plus n seeded random rows."""
    g = torch.Generator().manual_seed(seed)
    cu = call.cu_q_lens.tolist()
    rows = set()
    for b in range(len(cu) - 1):
        for t in (cu[b], cu[b + 1] - 1, (cu[b] + cu[b + 1]) // 2):
            for h in (0, num_q_heads - 1):
                rows.add((t, h))
    T = cu[-1]
    ts = torch.randint(0, T, (n,), generator=g).tolist()
    hs = torch.randint(0, num_q_heads, (n,), generator=g).tolist()
    rows.update(zip(ts, hs))
    return sorted(rows)
