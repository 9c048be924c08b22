"""Seeded random sweep of small shapes through every attention entry point,
against the oracle: batch sizes, head counts and group sizes, head dims 64 and
128, ragged context lengths (partial last pages, page- and tile-aligned ends),
chunk lengths from 1 to the whole context, causal and not, key splits, and
bf16 / fp8 / fp32 pools.  Each case prints its parameters before it runs."""
import random

import pytest
import torch

import workloads
from tests import harness as H
from tests.test_gpu_parity import _fp8_products_check

pytestmark = pytest.mark.gpu

pa = pytest.importorskip("online_softmax_paged_amd")


def _cases(n, seed):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        kv = rng.choice(["bf16", "bf16", "fp8", "fp8", "f32"])
        D = rng.choice([64, 128])
        Hkv = rng.choice([1, 2, 4])
        G = rng.choice([1, 2, 4, 8])
        if kv == "f32":
            D, G = 64, rng.choice([1, 2])
        B = rng.randint(1, 5)
        ctx = []
        for _ in range(B):
            c = rng.choice([rng.randint(1, 40), rng.randint(1, 700), 16 * rng.randint(1, 30),
                            32 * rng.randint(1, 20), 64 * rng.randint(1, 10) + 1])
            ctx.append(c)
        ql = [rng.choice([1, c, rng.randint(1, c)]) for c in ctx]
        causal = rng.random() < 0.8
        splits = rng.choice([0, 1, 2, 5])
        out.append(dict(i=i, kv=kv, D=D, Hq=Hkv * G, Hkv=Hkv, ctx=tuple(ctx), ql=tuple(ql),
                        causal=causal, splits=splits, seed=1000 + i))
    return out


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("case", _cases(24, 7), ids=lambda c: f"case{c['i']}")
def test_random_prefill(case):
    _log(f"random prefill {case}")
    wl = workloads.small("prefill", kv_dtype=case["kv"], q_dtype="f32" if case["kv"] == "f32" else "bf16",
                         num_q_heads=case["Hq"], num_kv_heads=case["Hkv"], head_dim=case["D"],
                         ctx_lens=case["ctx"], q_lens=case["ql"], seed=case["seed"],
                         causal=case["causal"])
    pool, opool = H.device_pool(wl), H.oracle_pool(wl)
    call = wl.calls[0]
    ro, rl = H.oracle_call(opool, wl, call)
    S = 0 if case["kv"] == "f32" else case["splits"]
    o, lse = H.DeviceCall(wl, call).run(pool, num_splits=S)
    torch.cuda.synchronize()
    eo, el = H.max_err(o, lse, ro, rl)
    tol = H.tolerance(wl)
    _log(f"  max|dO|={eo:.2e} max|dLSE|={el:.2e} tol={tol}")
    assert eo <= tol and el <= tol
    if case["kv"] == "fp8":
        o8, l8 = H.DeviceCall(wl, call).run(pool, num_splits=S, fp8_products=True)
        torch.cuda.synchronize()
        eo8, el8 = _fp8_products_check(opool, wl, call, o8, l8, ro, rl)
        _log(f"  fp8 products: {eo8:.2e}, lse {el8:.2e}")
        assert eo8 <= H.TOL["fp8"] and el8 <= H.TOL["fp8"]


@pytest.mark.parametrize("case", _cases(16, 11), ids=lambda c: f"case{c['i']}")
def test_random_decode(case):
    _log(f"random decode {case}")
    wl = workloads.small("decode", kv_dtype=case["kv"], q_dtype="f32" if case["kv"] == "f32" else "bf16",
                         num_q_heads=case["Hq"], num_kv_heads=case["Hkv"], head_dim=case["D"],
                         ctx_lens=case["ctx"], seed=case["seed"])
    pool, opool = H.device_pool(wl), H.oracle_pool(wl)
    call = wl.calls[0]
    ro, rl = H.oracle_call(opool, wl, call)
    tol = H.tolerance(wl)
    modes = [case["splits"]] + ([pa.DECODE_BALANCED] if case["kv"] != "f32" else [])
    for S in modes:
        o, lse = H.DeviceCall(wl, call).run(pool, num_splits=S)
        torch.cuda.synchronize()
        eo, el = H.max_err(o, lse, ro, rl)
        _log(f"  splits={S}: max|dO|={eo:.2e} max|dLSE|={el:.2e} tol={tol}")
        assert eo <= tol and el <= tol
