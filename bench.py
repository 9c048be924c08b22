"""Benchmark of the paged attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload headline|1..5|append] [--no-cpu-baseline]
    python bench.py --pmc-summary FETCH.csv WRITE.csv --copy-calib-mb N   (host only)

One step runs every call of the selected workloads once, inputs already
resident in HBM (the pool write is setup and is not timed).  The default
"headline" step is the 4 x 4096 causal prefill (bf16, 32 q / 8 KV heads,
d=128) followed by the 8 x 32768 long-context decode (bf16, 64 q / 8 KV heads,
d=128, split-KV + logsumexp merge).  Prints one JSON line:
  value     prefill TFLOP/s (4*d FLOPs per visible query-key pair per q head)
  decode    KV GB/s of the decode calls (K+V bytes read, logical)
  roofline  of the prefill kernel (MFMA bound), roofline_decode of the decode
  cpu_baseline  the float64 oracle timed on a bounded sample on the host.
Per-kernel times come from HIP events recorded on the stream the kernels run on,
created without the system-scope fence (a default event's record writes back
the L2, which adds microseconds around the launch it brackets).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
METRIC = "prefill TFLOP/s (% MFMA peak) + decode KV GB/s (% HBM peak), 1 MI355X"


def prefill_flops(call, head_dim, num_q_heads) -> float:
    """4*d FLOPs (QK^T and PV) for every visible (query, key) pair, per q head."""
    total = 0
    for b, q in enumerate(call.q_lens):
        c = int(call.ctx_lens[b])
        if call.causal:
            # query i sits at c - q + i and sees c - q + i + 1 keys
            total += q * (c - q) + q * (q + 1) // 2
        else:
            total += q * c
    return 4.0 * head_dim * num_q_heads * total


def decode_kv_bytes(call, wl) -> float:
    elem = {"f32": 4, "bf16": 2, "fp8": 1}[wl.kv_dtype]
    toks = int(call.ctx_lens.sum())
    return float(toks) * wl.num_kv_heads * wl.head_dim * 2 * elem


def _src_hash(name: str) -> str:
    p = os.path.join(ROOT, "online_softmax_paged_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def traffic_for(kernel_file: str, workload: str):
    """HBM bytes per launch from committed counter runs, if they were taken on
    the current source of the kernel; otherwise None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    data = json.load(open(path))
    rec = data.get(f"{kernel_file}:{workload}")
    if not rec or rec.get("source_sha") != _src_hash(kernel_file):
        return None
    return rec.get("bytes_per_launch")


def _pmc_per_dispatch(path: str):
    """{kernel name: [counter value of each dispatch]} from one rocprofv3
    counter_collection.csv holding a single counter."""
    import collections
    import csv

    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in csv.DictReader(open(path)):
        per[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def pmc_summary(fetch_csv: str, write_csv: str, copy_mb: int, names: dict):
    """Turn a FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch) into HBM
    bytes per launch of each library kernel.  Each counter is scaled by the
    ratio of the known size of a plain device-to-device copy of copy_mb MiB to
    what the same counter read for it; the result is stored, with a hash of the
    kernel source, in profiles/hbm_traffic.json."""
    fetch, write = _pmc_per_dispatch(fetch_csv), _pmc_per_dispatch(write_csv)

    def copy_kib(d):
        # the calibration copy is by far the largest blit dispatch of the run
        cands = [max(v) for k, v in d.items() if "copyBuffer" in k]
        return max(cands) if cands else None

    known_kib = float(copy_mb) * 1024
    cf, cw = copy_kib(fetch), copy_kib(write)
    if not cf or not cw:
        raise SystemExit("no copy kernel found in the counter files")
    f_fetch, f_write = known_kib / cf, known_kib / cw
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    files = {"prefill_dma_kernel": "prefill.hip", "prefill_kernel": "prefill.hip",
             "prefill_f32_kernel": "prefill.hip", "decode_split_kernel": "decode.hip",
             "decode_f32_kernel": "decode.hip", "decode_merge_kernel": "decode.hip"}
    rows = []
    for name, fv in sorted(fetch.items()):
        short = name.replace("pa::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        base = short.split("<")[0]
        if base not in files or name not in write:
            continue
        n, fk = len(fv), sum(fv) / len(fv)
        wk = sum(write[name]) / len(write[name])
        by = (fk * f_fetch + wk * f_write) * 1024
        rows.append((short, n, fk * f_fetch * 1024, wk * f_write * 1024, by))
        workload = names["prefill" if base.startswith("prefill") else "decode"]
        # the merge pass is keyed apart from the main kernel of its call
        key = f"{files[base]}:{workload}" + (":merge" if base == "decode_merge_kernel" else "")
        data[key] = {"kernel": short, "bytes_per_launch": by, "fetch_bytes": fk * f_fetch * 1024,
                     "write_bytes": wk * f_write * 1024, "dispatches": n,
                     "source_sha": _src_hash(files[base])}
    data["_calibration"] = {"copy_mib": copy_mb, "fetch_factor": f_fetch, "write_factor": f_write}
    json.dump(data, open(path, "w"), indent=1, sort_keys=True)
    print(f"copy of {copy_mb} MiB: FETCH_SIZE x{f_fetch:.4f}, WRITE_SIZE x{f_write:.4f}")
    print("| kernel | dispatches | HBM read MB | HBM write MB | total MB |")
    print("|---|---|---|---|---|")
    for short, n, fb, wb, by in rows:
        print(f"| `{short}` | {n} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {by / 1e6:.1f} |")


def cpu_baseline(wls, budget_s: float):
    """Time the float64 oracle on a bounded sample of the same workloads."""
    import numpy as np
    import torch

    from oracle import OraclePool, write_kv, gather_kv, attention_two_pass

    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    out = {}
    for wl in wls:
        opool = OraclePool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
        write_kv(opool, wl.k_src, wl.v_src, wl.slot_mapping)
        G = wl.num_q_heads // wl.num_kv_heads
        for call in wl.calls:
            work, n_units, t_used = 0.0, 0, 0.0
            cu = call.cu_q_lens.tolist()
            units = [(b, h) for b in range(len(call.seqs)) for h in range(wl.num_q_heads)]
            t0 = time.perf_counter()
            for (b, h) in units:
                c = int(call.ctx_lens[b])
                K, V = gather_kv(opool, call.block_table[b], c, h // G)
                q = call.q[cu[b]:cu[b + 1], h] if call.kind == "prefill" else call.q[b:b + 1, h]
                nq = q.shape[0]
                pos = np.arange(c - nq, c)
                attention_two_pass(q, K, V, wl.scale, pos, call.causal)
                if call.kind == "prefill":
                    vis = nq * (c - nq) + nq * (nq + 1) // 2 if call.causal else nq * c
                    work += 4.0 * wl.head_dim * vis
                else:
                    work += c * wl.head_dim * 2 * {"f32": 4, "bf16": 2, "fp8": 1}[wl.kv_dtype] / G
                n_units += 1
                t_used = time.perf_counter() - t0
                if t_used > budget_s / max(1, sum(len(w.calls) for w in wls)):
                    break
            unit = "TFLOP/s" if call.kind == "prefill" else "GB/s"
            rate = work / t_used / (1e12 if call.kind == "prefill" else 1e9)
            out[call.kind] = {"value": rate, "unit": unit, "cores": cores, "kind": "oracle",
                              "sample": f"{n_units} of {len(units)} (sequence, q-head) rows of "
                                        f"{wl.name} {call.kind}, {t_used:.1f} s"}
    return out


def bench_append(args):
    """One decode step's KV append per batch: host planning (pa_plan_append),
    the slot upload (through pinned memory), copies of shared pages (none: every sequence owns its
    pages here) and pa_append_kv, on the batched decode batch (bf16 pool, 32
    sequences) and the mixed batch's shapes (fp8 pool, 16 sequences of 1536
    tokens, so every step re-quantises 16 partly filled pages).  Each step
    appends one token to every sequence."""
    import torch

    import online_softmax_paged_amd as pa
    import workloads

    dev = torch.device("cuda:0")
    out = {"metric": "KV append per decode step (plan + copies + append_kv), 1 MI355X",
           "unit": "us", "higher_is_better": False, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "vs_baseline": None, "scaling": "weak",
           "data": "synthetic (seeded N(0,1) K/V)", "parts": []}
    for wl in (workloads.batched_decode_bf16(), workloads.mixed_fp8()):
        B, Hkv, D = len(wl.ctx_lens), wl.num_kv_heads, wl.head_dim
        steps = args.warmup + args.steps
        W = (max(wl.ctx_lens) + steps + 15) // 16
        NB = sum((c + steps + 15) // 16 for c in wl.ctx_lens) + 8
        pool = pa.KVPool(NB, Hkv, D, wl.kv_dtype, device=dev)
        alloc = pa.BlockAllocator(NB)
        bt = torch.full((B, W), -1, dtype=torch.int32)
        cl = torch.zeros(B, dtype=torch.int32)
        slots, _, _ = alloc.plan_append(bt, cl, list(wl.ctx_lens))
        src_dt = torch.bfloat16
        n0 = int(slots.numel())
        g = torch.Generator().manual_seed(2024)
        pa.write_kv(pool, torch.randn(n0, Hkv, D, generator=g).to(src_dt).to(dev),
                    torch.randn(n0, Hkv, D, generator=g).to(src_dt).to(dev), slots.to(dev))
        kn = torch.randn(steps, B, Hkv, D, generator=g).to(src_dt).to(dev)
        vn = torch.randn(steps, B, Hkv, D, generator=g).to(src_dt).to(dev)
        ws = torch.empty(max(1, pa.write_kv_workspace_bytes(pool)), dtype=torch.uint8, device=dev)
        staged = torch.empty(B, dtype=torch.int32, pin_memory=True)   # slot upload staging
        slots_dev = torch.empty(B, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        host_s, dev_ms = 0.0, 0.0
        for i in range(steps):
            t0 = time.perf_counter()
            slots, csrc, cdst = alloc.plan_append(bt, cl, [1] * B)
            staged.copy_(slots)
            t1 = time.perf_counter()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if len(csrc):
                pa.copy_blocks(pool, csrc.to(dev), cdst.to(dev))
            slots_dev.copy_(staged, non_blocking=True)
            pa.append_kv(pool, kn[i], vn[i], slots_dev, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            if i >= args.warmup:
                host_s += t1 - t0
                dev_ms += e0.elapsed_time(e1)
        out["parts"].append({"workload": wl.name, "kv_dtype": wl.kv_dtype, "sequences": B,
                             "device_us": dev_ms * 1e3 / args.steps,
                             "plan_us": host_s * 1e6 / args.steps})
    out["value"] = sum(p["device_us"] + p["plan_us"] for p in out["parts"]) / len(out["parts"])
    out["ms_per_step"] = out["value"] / 1e3
    out["dtype"] = "bf16+bf16-src/fp8-kv"
    out["config"] = {"workload": " + ".join(p["workload"] for p in out["parts"]) + " (append)"}
    out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_backward(args):
    """Backward of the causal prefill 4 x 4096 (32 q / 8 KV heads, d=128,
    bf16): dQ, dK, dV from the forward's o and lse.  FLOPs are the usual five
    products per visible (query, key, head) -- Q K^T, dO V^T, P^T dO, dS^T Q,
    dS K -- 2.5 times the forward's; the kernels compute Q K^T and dO V^T
    twice (once for dK/dV, once for dQ), 7 products in all."""
    import torch
    import online_softmax_paged_amd as pa
    import workloads
    dev = torch.device("cuda:0")
    wl = workloads.causal_prefill_bf16()
    pool = pa.KVPool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.kv_dtype, device=dev)
    pa.write_kv(pool, wl.k_src.to(dev), wl.v_src.to(dev), wl.slot_mapping.to(dev))
    call = wl.calls[0]
    q = call.q.to(dev)
    cu, ctx, bt = call.cu_q_lens.to(dev), call.ctx_lens.to(dev), call.block_table.to(dev)
    mq, mc = max(call.q_lens), int(call.ctx_lens.max())
    B, (T, Hq, D) = len(call.q_lens), q.shape
    o, lse = pa.prefill(pool, q, cu, ctx, bt, wl.scale, max_q_len=mq, max_ctx_len=mc, num_splits=1)
    do = workloads.upstream_grad(call, D, Hq, seed=2024).to(dev)
    dq = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    dk = torch.zeros(pool.k.shape, dtype=torch.float32, device=dev)
    dv = torch.zeros(pool.v.shape, dtype=torch.float32, device=dev)
    ws = torch.empty(pa.backward_workspace_bytes(pool, B, Hq, mq), dtype=torch.uint8, device=dev)
    fn = lambda: pa.prefill_backward(pool, q, o, lse, do, cu, ctx, bt, wl.scale, max_q_len=mq,
                                     max_ctx_len=mc, dq=dq, dk=dk, dv=dv, workspace=ws)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    fl = 2.5 * prefill_flops(call, D, Hq)
    tf = fl / (ms * 1e-3) / 1e12
    result = {"metric": "prefill backward TFLOP/s (5 products per visible pair)", "value": tf,
              "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "bf16", "data": "synthetic (seeded N(0,1) Q/K/V/dO, shuffled pages)",
              "config": {"workload": wl.name + " backward"},
              "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": tf / PEAK_BF16_TFLOPS, "traffic": None},
              "parts": {"flops": fl, "products_computed": 7}}
    print(json.dumps(result), flush=True)


def bench_shared_prefix_decode(args):
    """64 decode rows over a shared 4096-token prefix (+512 own tokens each):
    pa_decode against pa_prefill_shared_prefix, each timed alone with the
    last-level cache evicted before every step.  The metric is the logical
    K/V bytes the step attends over (what pa_decode reads) per second."""
    import torch
    import online_softmax_paged_amd as pa
    import workloads
    dev = torch.device("cuda:0")
    wl = workloads.shared_prefix_decode_bf16()
    pool = pa.KVPool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.kv_dtype, device=dev)
    pa.write_kv(pool, wl.k_src.to(dev), wl.v_src.to(dev), wl.slot_mapping.to(dev))
    call = wl.calls[0]
    q = call.q.to(dev)
    ctx, bt = call.ctx_lens.to(dev), call.block_table.to(dev)
    cu = torch.arange(q.shape[0] + 1, dtype=torch.int32, device=dev)
    B, Hq, D = q.shape
    mc, P = int(call.ctx_lens.max()), wl.shared_prefix
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    S = pa.decode_choose_splits(B, wl.num_kv_heads, mc, int(call.ctx_lens.sum()))
    ws = torch.empty(max(1, pa.decode_workspace_bytes(B, Hq, D, S)), dtype=torch.uint8, device=dev)
    plan = pa.shared_prefix_plan(pool, B, Hq, 1, mc, P, B)
    ws2 = torch.empty(max(1, plan["workspace_bytes"]), dtype=torch.uint8, device=dev)
    fns = {
        "decode": lambda: pa.decode(pool, q, ctx, bt, wl.scale, max_ctx_len=mc, num_splits=S,
                                    workspace=ws, out=o, lse=lse),
        "shared_prefix": lambda: pa.prefill_shared_prefix(
            pool, q, cu, ctx, bt, wl.scale, P, max_q_len=1, max_ctx_len=mc, out=o, lse=lse,
            workspace=ws2),
    }
    scratch = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
    logical = decode_kv_bytes(call, wl)
    unique = 2.0 * wl.num_kv_heads * D * 2 * (P + B * (mc - P))
    times = {}
    for name, fn in fns.items():
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        tot = 0.0
        for _ in range(args.steps):
            scratch.sum(dtype=torch.int64)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
        times[name] = tot / args.steps
    ms = times["shared_prefix"]
    result = {"metric": "decode over a shared prefix: logical KV GB/s", "value": logical / (ms * 1e-3) / 1e9,
              "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "bf16", "data": "synthetic (seeded N(0,1) Q/K/V, shuffled pages)",
              "config": {"workload": wl.name, "cache_flush_mb": 512},
              "parts": {"decode_ms": times["decode"], "shared_prefix_ms": ms,
                        "speedup": times["decode"] / ms, "logical_kv_bytes": logical,
                        "unique_kv_bytes": unique, "decode_splits": S,
                        "shared_prefix_plan": {k: plan[k] for k in (
                            "mode", "prefix_splits", "suffix_splits", "plain_splits")},
                        "unique_gbps": unique / (ms * 1e-3) / 1e9}}
    print(json.dumps(result), flush=True)


def one_call_timings(pa, wl, pool, dev, args, scratch):
    """The workload's calls (chunks and decode rows) as ONE varlen call, timed
    two ways after the main loop: pa_prefill, and pa_prefill_shared_prefix
    (prefix attended once by all queries packed together).  Reported beside
    the step; the step itself keeps its separate calls."""
    import torch
    import workloads
    call = workloads.one_call(wl)
    q = call.q.to(dev)
    cu, ctx, bt = call.cu_q_lens.to(dev), call.ctx_lens.to(dev), call.block_table.to(dev)
    mq, mc = max(call.q_lens), int(call.ctx_lens.max())
    B, (T, Hq, D) = len(call.q_lens), q.shape
    o = torch.empty_like(q)
    lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    S = pa.prefill_num_splits(B, wl.num_kv_heads, Hq, mq, mc)
    ws = torch.empty(max(1, pa.prefill_workspace_bytes(B, mq, Hq, D, S)), dtype=torch.uint8,
                     device=dev)
    plans = {m: pa.shared_prefix_plan(pool, B, Hq, mq, mc, wl.shared_prefix, T, mode=m)
             for m in (pa.SHARED_AUTO, pa.SHARED_PACKED)}
    ws2 = torch.empty(max(1, max(p["workspace_bytes"] for p in plans.values())),
                      dtype=torch.uint8, device=dev)

    def shared(mode):
        return lambda: pa.prefill_shared_prefix(
            pool, q, cu, ctx, bt, wl.scale, wl.shared_prefix, causal=call.causal, max_q_len=mq,
            max_ctx_len=mc, out=o, lse=lse, mode=mode, workspace=ws2)
    fns = {
        "prefill": lambda: pa.prefill(pool, q, cu, ctx, bt, wl.scale, causal=call.causal,
                                      max_q_len=mq, max_ctx_len=mc, out=o, lse=lse,
                                      num_splits=S, workspace=ws),
        "shared_prefix": shared(pa.SHARED_AUTO),
        "shared_prefix_packed": shared(pa.SHARED_PACKED),
    }
    mode_name = {pa.SHARED_PACKED: "packed", pa.SHARED_PLAIN: "plain"}
    out = {"workload": wl.name, "flops": prefill_flops(call, wl.head_dim, wl.num_q_heads),
           "splits": {"prefill": S,
                      "shared_prefix": {mode_name[p["mode"]]: [p["prefix_splits"],
                                                               p["suffix_splits"],
                                                               p["plain_splits"]]
                                        for p in plans.values()}},
           "shared_prefix_mode": mode_name[plans[pa.SHARED_AUTO]["mode"]]}
    for name, fn in fns.items():
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        tot = 0.0
        for _ in range(args.steps):
            if scratch is not None:
                scratch.sum(dtype=torch.int64)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
        out[name + "_ms"] = tot / args.steps
    return out


def measured_ceilings(pa, dev) -> dict:
    """What this GPU sustains, measured in the same process with the library's
    probes (pa_probe_stream_read, pa_probe_mfma): the best of three grid sizes
    for a non-temporal streaming read of 1 GiB, and MFMA loops of 4
    independent chains per wave on register operands (bf16 and fp8)."""
    import torch

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    best = 0.0
    for blocks in (1024, 2048, 4096):
        out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
        sec = timed(lambda: pa.probe_stream_read(buf, blocks=blocks, out=out), 10)
        best = max(best, buf.numel() / sec / 1e9)
    del buf
    res = {"hbm_read_gbps": best}
    out = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
    for dt, iters in (("bf16", 2000), ("fp8", 1000)):
        flop = [0.0]

        def run():
            flop[0] = pa.probe_mfma(dt, blocks=2048, iters=iters, out=out)
        sec = timed(run, 3)
        res[f"mfma_{dt}_tflops"] = flop[0] / sec / 1e12
    res["method"] = ("library probes in this process: non-temporal streaming read of 1 GiB "
                     "(best of 1024/2048/4096 workgroups); 4 independent MFMA chains per wave "
                     "on register operands, 2048 workgroups")
    return res


def page_pattern_floor(pa, dev, nbytes: float, steps: int, scratch) -> dict:
    """The decode's read pattern with no arithmetic (pa_probe_page_stream) over
    about the same volume, spread evenly over 256, 512 or 1024 workgroups (the
    best of the three), timed like the decode (cache evicted first when the
    decode's is)."""
    import torch
    unit = 1024 * 8192
    nb = max(unit, int(nbytes) // unit * unit)
    buf = torch.ones(nb, dtype=torch.uint8, device=dev)
    out = torch.empty(1024 * 256, dtype=torch.int32, device=dev)
    best = None
    for blocks in (256, 512, 1024):
        pa.probe_page_stream(buf, blocks=blocks, out=out)
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(3, steps)):
            if scratch is not None:
                scratch.sum(dtype=torch.int64)
            e0, e1 = FenceFreeEvent(), FenceFreeEvent()
            e0.record()
            pa.probe_page_stream(buf, blocks=blocks, out=out)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = statistics.median(ts)
        if best is None or ms < best["ms"]:
            best = {"bytes": nb, "ms": ms, "gbps": nb / (ms * 1e-3) / 1e9, "workgroups": blocks}
    del buf
    return best


class FenceFreeEvent:
    """A HIP timing event created with hipEventDisableSystemFence, from the HIP
    runtime torch has loaded.  Its record carries no system-scope release, so
    it takes no L2 write-back: a default event's fence adds several
    microseconds around the launch it brackets and slows the launch after it.
    Elapsed times are read only after a device synchronisation."""

    _hip = None
    _FLAG = 0x20000000  # hipEventDisableSystemFence

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            path = next((l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l), None)
            if path is None:
                raise RuntimeError("HIP runtime not loaded (initialise torch.cuda first)")
            cls._hip = ctypes.CDLL(path)
        return cls._hip

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self.ev), ctypes.c_uint(self._FLAG))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")

    def record(self, stream=None):
        import torch
        s = (stream or torch.cuda.current_stream()).cuda_stream
        rc = self._lib().hipEventRecord(self.ev, self._ct.c_void_p(s))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_time(self, end):
        ms = self._ct.c_float()
        rc = self._lib().hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the prefill reaches its steady rate only after some 50-100 ms of sustained
    # load: timed after 5 warmup steps it runs ~8% slower than after 100
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--decode-splits", type=int, default=0,
                    help="KV splits for decode calls (0 = the library's choice, "
                         "-1 = balanced chunks across sequences)")
    ap.add_argument("--flush-mb", type=int, default=-1,
                    help="MB of scratch written between steps to evict the 256 MB last-level "
                         "cache (-1 = 512 when a decode call reads less than 512 MB of KV)")
    ap.add_argument("--bf16-products", action="store_true",
                    help="prefill calls on fp8 pools use pa_prefill (codes widened to bf16, "
                         "products on the bf16 matrix cores) instead of pa_prefill_fp8 (Q and "
                         "P in E4M3, both products on the fp8 matrix cores)")
    ap.add_argument("--torch-events", action="store_true",
                    help="time the launches with torch's default events, whose record carries a "
                         "system-scope fence (L2 write-back), instead of fence-free HIP events")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured ceilings (streaming read, MFMA loops) after the timed steps")
    ap.add_argument("--one-call", action="store_true",
                    help="also time a shared-prefix workload's calls joined into one call "
                         "(pa_prefill and pa_prefill_shared_prefix), outside the step")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="run one plain device-to-device copy of this many MiB after the "
                         "warmup (outside the timed region) to calibrate HBM byte counters")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: summarise two rocprofv3 --pmc runs of this script "
                         "(FETCH_SIZE, then WRITE_SIZE) into profiles/hbm_traffic.json")
    args = ap.parse_args()
    if args.pmc_summary:
        if not args.copy_calib_mb:
            raise SystemExit("--pmc-summary needs the --copy-calib-mb the runs used")
        import workloads
        if args.workload == "headline":
            names = {"prefill": workloads.NAMES[3], "decode": workloads.NAMES[4]}
        else:
            n = workloads.NAMES[int(args.workload)]
            names = {"prefill": n, "decode": n}
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.copy_calib_mb, names)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence and KV head, see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    import online_softmax_paged_amd as pa
    import workloads

    if args.workload == "append":
        bench_append(args)
        return
    if args.workload == "shared":
        bench_shared_prefix_decode(args)
        return
    if args.workload == "backward":
        bench_backward(args)
        return
    if args.workload == "headline":
        wls = [workloads.causal_prefill_bf16(), workloads.long_decode_bf16()]
    else:
        wls = [workloads.NAMED[int(args.workload)]()]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    launches = []   # (kind, wl, call, fn, fp8 products)
    pools = {}
    for wl in wls:
        pool = pa.KVPool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.kv_dtype, device=dev)
        pa.write_kv(pool, wl.k_src.to(dev), wl.v_src.to(dev), wl.slot_mapping.to(dev))
        pools[wl.name] = pool
        for call in wl.calls:
            q = call.q.to(dev)
            cu, ctx, bt = call.cu_q_lens.to(dev), call.ctx_lens.to(dev), call.block_table.to(dev)
            mq, mc = max(call.q_lens), int(call.ctx_lens.max())
            o = torch.empty_like(q)
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
            if call.kind == "prefill":
                B, Hq, D = len(call.q_lens), q.shape[1], q.shape[2]
                S = pa.prefill_num_splits(B, wl.num_kv_heads, Hq, mq, mc)
                ws = torch.empty(max(1, pa.prefill_workspace_bytes(B, mq, Hq, D, S)),
                                 dtype=torch.uint8, device=dev)
                f8 = wl.kv_dtype == "fp8" and not args.bf16_products
                fn = (lambda pool=pool, q=q, cu=cu, ctx=ctx, bt=bt, mq=mq, mc=mc, o=o, lse=lse, wl=wl,
                      c=call, S=S, ws=ws, f8=f8:
                      pa.prefill(pool, q, cu, ctx, bt, wl.scale, causal=c.causal, max_q_len=mq,
                                 max_ctx_len=mc, out=o, lse=lse, num_splits=S, workspace=ws,
                                 fp8_products=f8))
            else:
                f8 = False
                B, Hq, D = q.shape
                S = args.decode_splits or pa.decode_choose_splits(
                    B, wl.num_kv_heads, mc, int(call.ctx_lens.sum()))
                nws = (pa.decode_balanced_workspace_bytes(B, Hq, wl.num_kv_heads, D, mc)
                       if S == pa.DECODE_BALANCED else pa.decode_workspace_bytes(B, Hq, D, S))
                ws = torch.empty(max(1, nws), dtype=torch.uint8, device=dev)
                fn = (lambda pool=pool, q=q, ctx=ctx, bt=bt, mc=mc, o=o, lse=lse, wl=wl, ws=ws, S=S:
                      pa.decode(pool, q, ctx, bt, wl.scale, max_ctx_len=mc, num_splits=S,
                                workspace=ws, out=o, lse=lse))
            launches.append((call.kind, wl, call, fn, call.kind == "prefill" and f8))
    flush_mb = args.flush_mb
    if flush_mb < 0:
        small = any(k == "decode" and decode_kv_bytes(c, w) < 512e6 for k, w, c, _, _ in launches)
        flush_mb = 512 if small else 0
    scratch = torch.ones(flush_mb << 20, dtype=torch.uint8, device=dev) if flush_mb else None
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for _, _, _, fn, _ in launches:
            fn()
    torch.cuda.synchronize()
    if args.copy_calib_mb:
        src = torch.ones(args.copy_calib_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.torch_events:
        def mk():
            return torch.cuda.Event(enable_timing=True)
    else:
        mk = FenceFreeEvent
    evs = [[(mk(), mk()) for _ in launches] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if scratch is not None:
            # read (not write) the scratch: evicts the KV from the cache without
            # leaving dirty lines whose write-back would overlap the timed launches
            scratch.sum(dtype=torch.int64)
        for i, (_, _, _, fn, _) in enumerate(launches):
            evs[s][i][0].record()
            fn()
            evs[s][i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    step_ms = [[evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)]
               for i in range(len(launches))]
    per_launch_ms = [sum(x) / len(x) for x in step_ms]
    # with a flush between steps the step time is the sum of the launches'
    # event times; otherwise it is the wall clock of the K steps
    ms_per_step = sum(per_launch_ms) if scratch is not None else wall * 1e3 / args.steps
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "data": "synthetic (seeded N(0,1) Q/K/V, shuffled pages)",
              "timing": ("torch events (system-scope fence)" if args.torch_events
                         else "HIP events without system fence, one pair per launch")}
    parts = {}
    for (kind, wl, call, _, f8), ms, sms in zip(launches, per_launch_ms, step_ms):
        spread = {"ms_median": statistics.median(sms), "ms_min": min(sms)}
        if kind == "prefill":
            fl = prefill_flops(call, wl.head_dim, wl.num_q_heads)
            tf = fl / (ms * 1e-3) / 1e12
            parts.setdefault("prefill", []).append(
                {"workload": wl.name, "ms": ms, "tflops": tf, "frac_bf16_peak": tf / PEAK_BF16_TFLOPS,
                 "products": "fp8" if f8 else "bf16",
                 "frac_products_peak": tf / (PEAK_FP8_TFLOPS if f8 else PEAK_BF16_TFLOPS),
                 "flops": fl, "dtype": wl.kv_dtype, **spread})
        else:
            by = decode_kv_bytes(call, wl)
            gbps = by / (ms * 1e-3) / 1e9
            parts.setdefault("decode", []).append(
                {"workload": wl.name, "ms": ms, "gbps": gbps, "frac_hbm_peak": gbps / PEAK_HBM_GBPS,
                 "kv_bytes": by, "dtype": wl.kv_dtype, **spread})
    pre = parts.get("prefill", [])
    dec = parts.get("decode", [])
    if pre:
        fl = sum(p["flops"] for p in pre)
        ms = sum(p["ms"] for p in pre)
        result["value"] = fl / (ms * 1e-3) / 1e12
        result["unit"] = "TFLOP/s"
    else:
        by = sum(d["kv_bytes"] for d in dec)
        ms = sum(d["ms"] for d in dec)
        result["value"] = by / (ms * 1e-3) / 1e9
        result["unit"] = "GB/s"
    # the arithmetic type of the products: fp8 pools take E4M3 products unless
    # --bf16-products; their decode widens the codes and runs in fp32/bf16
    f8_pre = any(p["products"] == "fp8" for p in parts.get("prefill", []))
    result["dtype"] = "bf16" if all(w.kv_dtype == "bf16" for w in wls) else \
        ("fp8" if f8_pre else "+".join(sorted({("bf16-q/fp8-kv" if w.kv_dtype == "fp8" else w.kv_dtype)
                                               for w in wls})))
    result["config"] = {"workload": " + ".join(w.name for w in wls), "cache_flush_mb": flush_mb}
    if pre:
        p = pre[0]
        pk = PEAK_FP8_TFLOPS if p["products"] == "fp8" else PEAK_BF16_TFLOPS
        result["roofline"] = {"bound": "mfma", "achieved": p["tflops"], "peak": pk,
                              "unit": "TFLOP/s", "frac": p["tflops"] / pk,
                              "traffic": traffic_for("prefill.hip", p["workload"])}
    if dec:
        d = dec[0]
        key = "roofline_decode" if pre else "roofline"
        result[key] = {"bound": "hbm", "achieved": d["gbps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                       "frac": d["gbps"] / PEAK_HBM_GBPS,
                       "traffic": traffic_for("decode.hip", d["workload"])}
        result["decode"] = {"value": sum(x["kv_bytes"] for x in dec) / (sum(x["ms"] for x in dec) * 1e-3) / 1e9,
                            "unit": "GB/s", "frac_hbm_peak": None}
        result["decode"]["frac_hbm_peak"] = result["decode"]["value"] / PEAK_HBM_GBPS
    if not args.no_ceilings:
        ceil = measured_ceilings(pa, dev)
        result["ceilings"] = ceil
        for key in ("roofline", "roofline_decode"):
            r = result.get(key)
            if not r:
                continue
            if r["bound"] == "hbm":
                m = ceil["hbm_read_gbps"]
            else:
                m = ceil["mfma_fp8_tflops" if r["peak"] == PEAK_FP8_TFLOPS else "mfma_bf16_tflops"]
            r["measured_peak"] = m
            r["frac_measured"] = r["achieved"] / m
    if not args.no_ceilings:
        for d in dec:
            f = page_pattern_floor(pa, dev, d["kv_bytes"], args.steps, scratch)
            d["page_pattern_floor"] = f
            d["frac_of_page_pattern_floor"] = (f["ms"] * d["kv_bytes"] / f["bytes"]) / d["ms"]
    if args.one_call:
        for wl in wls:
            if wl.shared_prefix and len(wl.calls) > 1:
                parts["one_call"] = one_call_timings(pa, wl, pools[wl.name], dev, args, scratch)
    result["parts"] = parts
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wls, args.cpu_budget)
        first = cb.get("prefill") or cb.get("decode")
        result["cpu_baseline"] = dict(first)
        if first.get("value"):
            result["cpu_baseline"]["gpu_over_oracle"] = result["value"] / first["value"]
        if "prefill" in cb and "decode" in cb:
            result["cpu_baseline"]["decode"] = dict(cb["decode"])
            if cb["decode"].get("value") and "decode" in result:
                result["cpu_baseline"]["decode"]["gpu_over_oracle"] = \
                    result["decode"]["value"] / cb["decode"]["value"]
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
