"""Seeded synthetic workloads for paged attention.

This module only draws inputs: sequence lengths, the physical page assignment
(a seeded relabelling of pages allocated in logical order, as the block-table
scheme of the PagedAttention page, section on its core principle, describes),
and Q/K/V values from N(0, 1).  It holds none of the attention arithmetic and
no quantisation: the kernels and the oracle each do that on their own.  Both
the product tests and the oracle read inputs from here.

Recipe (fixed for every workload):
  1. ``g = torch.Generator('cpu').manual_seed(seed)``.
  2. Random context lengths, when the workload asks for them, with
     ``torch.randint`` on ``g``.
  3. Pages are given logical ids in order (shared prefix first, then each
     sequence's own pages), then relabelled to physical ids with
     ``torch.randperm(num_blocks, generator=g)``.  The pool holds the pages in
     use plus ``spare_pages`` that nothing writes (tests fill them with NaN).
  4. Query tokens of every prefill call, then K, then V for every unique
     written token in logical order, then query tokens of every decode call,
     all as float32 ``torch.randn`` on ``g`` and cast (round to nearest even)
     to the workload's dtype.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BLOCK_SIZE = 16

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class Call:
    """One attention call over a subset of the sequences.

    kind: "prefill" (q_lens[i] queries that end at the sequence's last token,
    causal) or "decode" (one query at the last position).
    """
    kind: str
    seqs: list
    q_lens: list
    causal: bool = True
    # filled in by build():
    q: torch.Tensor | None = None          # [sum(q_lens), Hq, d] in q dtype
    cu_q_lens: torch.Tensor | None = None  # int32 [B+1]
    ctx_lens: torch.Tensor | None = None   # int32 [B]
    block_table: torch.Tensor | None = None  # int32 [B, W]


@dataclass
class Workload:
    name: str
    kv_dtype: str            # "f32" | "bf16" | "fp8"  (pool storage)
    src_dtype: str           # dtype of the K/V tokens handed to the write step
    q_dtype: str             # "f32" | "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    num_blocks: int
    ctx_lens: list           # per sequence
    block_tables: torch.Tensor  # int32 [num_seqs, W]; -1 past the last used page
    k_src: torch.Tensor      # [n_tok, Hkv, d] src dtype, unique written tokens
    v_src: torch.Tensor
    slot_mapping: torch.Tensor  # int32 [n_tok]: phys * 16 + offset
    calls: list = field(default_factory=list)
    seed: int = 0
    shared_prefix: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _pages(n_tokens: int) -> int:
    return (n_tokens + BLOCK_SIZE - 1) // BLOCK_SIZE


def build(name: str, *, kv_dtype: str, q_dtype: str, num_q_heads: int,
          num_kv_heads: int, head_dim: int, ctx_lens=None, ctx_len_range=None,
          num_seqs: int | None = None, calls: list, seed: int,
          shared_prefix: int = 0, spare_pages: int = 8, scale: float | None = None,
          src_dtype: str | None = None) -> Workload:
    """Draw one workload.  ``calls`` lists Call(kind, seqs, q_lens) templates."""
    assert shared_prefix % BLOCK_SIZE == 0
    g = torch.Generator("cpu").manual_seed(seed)
    if ctx_lens is None:
        lo, hi = ctx_len_range
        ctx_lens = torch.randint(lo, hi + 1, (num_seqs,), generator=g).tolist()
    ctx_lens = [int(c) for c in ctx_lens]
    B = len(ctx_lens)
    assert all(c > shared_prefix for c in ctx_lens) or shared_prefix == 0

    # -- logical page ids: shared prefix pages, then each sequence's own pages
    n_shared = shared_prefix // BLOCK_SIZE
    logical_tables = []
    next_id = n_shared
    for c in ctx_lens:
        own = _pages(c) - n_shared
        logical_tables.append(list(range(n_shared)) + list(range(next_id, next_id + own)))
        next_id += own
    used = next_id
    num_blocks = used + spare_pages
    perm = torch.randperm(num_blocks, generator=g)
    W = max(len(t) for t in logical_tables)
    bt = torch.full((B, W), -1, dtype=torch.int32)
    for b, t in enumerate(logical_tables):
        bt[b, : len(t)] = perm[torch.tensor(t, dtype=torch.long)].to(torch.int32)

    # -- unique written tokens in logical order, with their slots
    def slots_of(b, t0, t1):
        t = torch.arange(t0, t1, dtype=torch.long)
        return bt[b, t // BLOCK_SIZE].long() * BLOCK_SIZE + t % BLOCK_SIZE

    pieces = [slots_of(0, 0, shared_prefix)]
    for b, c in enumerate(ctx_lens):
        pieces.append(slots_of(b, shared_prefix, c))
    slot_mapping = torch.cat(pieces).to(torch.int32)
    n_tok = int(slot_mapping.numel())

    src_dtype = src_dtype or ("f32" if kv_dtype == "f32" else "bf16")
    sdt = _TORCH_DTYPES[src_dtype]
    qdt = _TORCH_DTYPES[q_dtype]
    Hq, Hkv, d = num_q_heads, num_kv_heads, head_dim

    def draw(shape, dt):
        return torch.randn(shape, dtype=torch.float32, generator=g).to(dt)

    out_calls = []
    for tmpl in calls:
        out_calls.append(Call(tmpl.kind, list(tmpl.seqs), list(tmpl.q_lens), tmpl.causal))
    for c in out_calls:
        if c.kind == "prefill":
            c.q = draw((sum(c.q_lens), Hq, d), qdt)
    k_src = draw((n_tok, Hkv, d), sdt)
    v_src = draw((n_tok, Hkv, d), sdt)
    for c in out_calls:
        if c.kind == "decode":
            assert all(x == 1 for x in c.q_lens)
            c.q = draw((len(c.seqs), Hq, d), qdt)
    for c in out_calls:
        c.ctx_lens = torch.tensor([ctx_lens[s] for s in c.seqs], dtype=torch.int32)
        cu = [0]
        for x in c.q_lens:
            cu.append(cu[-1] + x)
        c.cu_q_lens = torch.tensor(cu, dtype=torch.int32)
        c.block_table = bt[torch.tensor(c.seqs, dtype=torch.long)].contiguous()
        for x, s in zip(c.q_lens, c.seqs):
            assert 1 <= x <= ctx_lens[s]

    return Workload(
        name=name, kv_dtype=kv_dtype, src_dtype=src_dtype, q_dtype=q_dtype,
        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
        scale=scale if scale is not None else 1.0 / math.sqrt(d),
        num_blocks=num_blocks, ctx_lens=ctx_lens, block_tables=bt,
        k_src=k_src, v_src=v_src, slot_mapping=slot_mapping, calls=out_calls,
        seed=seed, shared_prefix=shared_prefix)


def upstream_grad(call: Call, head_dim: int, num_q_heads: int, seed: int,
                  dtype: str = "bf16") -> torch.Tensor:
    """A seeded upstream gradient dO for a call's queries: [T, Hq, d] drawn
    as float32 randn on its own generator and cast (nearest even) to dtype."""
    g = torch.Generator("cpu").manual_seed(seed)
    T = int(call.cu_q_lens[-1])
    return torch.randn((T, num_q_heads, head_dim), dtype=torch.float32,
                       generator=g).to(_TORCH_DTYPES[dtype])


def one_call(wl: Workload) -> Call:
    """The workload's calls joined into one varlen call: sequences and query
    tokens in call order (a decode query is a one-token chunk at the last
    position).  Only concatenation; nothing is drawn."""
    seqs, q_lens = [], []
    for c in wl.calls:
        seqs += c.seqs
        q_lens += c.q_lens
    assert len(set(c.causal for c in wl.calls)) == 1
    out = Call("prefill", seqs, q_lens, wl.calls[0].causal)
    out.q = torch.cat([c.q for c in wl.calls])
    out.ctx_lens = torch.tensor([wl.ctx_lens[s] for s in seqs], dtype=torch.int32)
    cu = [0]
    for x in q_lens:
        cu.append(cu[-1] + x)
    out.cu_q_lens = torch.tensor(cu, dtype=torch.int32)
    out.block_table = wl.block_tables[torch.tensor(seqs, dtype=torch.long)].contiguous()
    return out


# ---------------------------------------------------------------------------
# The five named workloads.  Seeds are 1000 + k for workload k.

NAMES = {
    1: "tiny_fp32_1x256_d64",
    2: "decode_bf16_32seq_len128-2048_gqa4_d128",
    3: "prefill_bf16_4x4096_gqa4_d128",
    4: "decode_bf16_8x32768_gqa8_d128",
    5: "mixed_fp8kv_16x1536_prefix1024_gqa4_d128",
}

def tiny_fp32() -> Workload:
    """1 sequence, 1 head, d=64, 256 tokens in 16 shuffled pages; causal
    prefill of all 256 positions, plus one fresh decode query at position 255."""
    return build(NAMES[1], kv_dtype="f32", q_dtype="f32",
                 num_q_heads=1, num_kv_heads=1, head_dim=64, ctx_lens=[256],
                 calls=[Call("prefill", [0], [256]), Call("decode", [0], [1])],
                 seed=1001, scale=1.0 / 8.0)


def batched_decode_bf16() -> Workload:
    """32 sequences, lengths U{128..2048}, 32 q heads / 8 KV heads, d=128."""
    return build(NAMES[2], kv_dtype="bf16",
                 q_dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                 ctx_len_range=(128, 2048), num_seqs=32,
                 calls=[Call("decode", list(range(32)), [1] * 32)], seed=1002)


def causal_prefill_bf16() -> Workload:
    """4 sequences x 4096 tokens, causal prefill, 32 q heads / 8 KV heads, d=128."""
    return build(NAMES[3], kv_dtype="bf16", q_dtype="bf16",
                 num_q_heads=32, num_kv_heads=8, head_dim=128, ctx_lens=[4096] * 4,
                 calls=[Call("prefill", [0, 1, 2, 3], [4096] * 4)], seed=1003)


def long_decode_bf16() -> Workload:
    """8 sequences x 32768 tokens, 64 q heads / 8 KV heads, d=128, one query each."""
    return build(NAMES[4], kv_dtype="bf16", q_dtype="bf16",
                 num_q_heads=64, num_kv_heads=8, head_dim=128, ctx_lens=[32768] * 8,
                 calls=[Call("decode", list(range(8)), [1] * 8)], seed=1004)


def mixed_fp8() -> Workload:
    """16 sequences sharing a 1024-token prefix plus 512 own tokens each; fp8
    KV pool with one scale per page; sequences 0-7 run a 256-token chunked
    prefill (their last 256 positions), sequences 8-15 decode one token."""
    return build(NAMES[5], kv_dtype="fp8",
                 q_dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                 ctx_lens=[1536] * 16, shared_prefix=1024,
                 calls=[Call("prefill", list(range(8)), [256] * 8),
                        Call("decode", list(range(8, 16)), [1] * 8)], seed=1005)


def shared_prefix_decode_bf16() -> Workload:
    """64 sequences that share a 4096-token prefix and hold 512 own tokens
    each (4608 in all), one decode query each; 32 q / 8 KV heads, d=128."""
    return build("shared_prefix_decode_bf16_64x4608_prefix4096_gqa4_d128", kv_dtype="bf16",
                 q_dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                 ctx_lens=[4608] * 64, shared_prefix=4096,
                 calls=[Call("decode", list(range(64)), [1] * 64)], seed=1006)


NAMED = {
    1: tiny_fp32,
    2: batched_decode_bf16,
    3: causal_prefill_bf16,
    4: long_decode_bf16,
    5: mixed_fp8,
}


def small(kind: str, *, kv_dtype="bf16", q_dtype="bf16", num_q_heads=8,
          num_kv_heads=2, head_dim=128, ctx_lens=(100, 37, 300), q_lens=None,
          seed=7, shared_prefix=0, spare_pages=8, src_dtype=None,
          causal=True) -> Workload:
    """A small workload of the same structure, for parity at oracle-friendly size."""
    ctx_lens = list(ctx_lens)
    B = len(ctx_lens)
    if kind == "decode":
        calls = [Call("decode", list(range(B)), [1] * B)]
    elif kind == "prefill":
        q_lens = list(q_lens) if q_lens is not None else list(ctx_lens)
        calls = [Call("prefill", list(range(B)), q_lens, causal)]
    else:
        raise ValueError(kind)
    return build(f"small_{kind}_{kv_dtype}", kv_dtype=kv_dtype, q_dtype=q_dtype,
                 num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, ctx_lens=ctx_lens, calls=calls, seed=seed,
                 shared_prefix=shared_prefix, spare_pages=spare_pages,
                 src_dtype=src_dtype)
