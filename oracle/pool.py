"""The oracle's own paged KV pool (test infrastructure only).

Layout, the documented one of the library boundary, one contiguous chunk per
(physical page, KV head):
  K: [num_blocks, num_kv_heads, 16, head_dim]   (token-major inside a page)
  V: [num_blocks, num_kv_heads, head_dim, 16]   (feature-major inside a page)
The pages (PagedAttention page, core principle section; the "core modules"
chapter, section 2.2) fix only that a physical block holds the K and V of 16
tokens and is found through the block table; the order inside a page is this
library's choice and the oracle follows it so that pool bytes can be compared.

Storage: float32 values, bfloat16 bit patterns (uint16), or fp8 E4M3 codes
(uint8) with one float32 scale per physical page for K and one for V, shared by
all KV heads.  Slots nobody wrote hold NaN (0x7FC00000, 0x7FC0, 0x7F).
"""
from __future__ import annotations

import numpy as np
import torch

from . import fp8_e4m3

BLOCK = 16
_NAN_BITS = {"f32": np.uint32(0x7FC00000), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}
_STORE = {"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8}


class OraclePool:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, kv_dtype: str):
        self.num_blocks, self.num_kv_heads, self.head_dim = num_blocks, num_kv_heads, head_dim
        self.kv_dtype = kv_dtype
        st = _STORE[kv_dtype]
        self.k = np.full((num_blocks, num_kv_heads, BLOCK, head_dim), _NAN_BITS[kv_dtype], dtype=st)
        self.v = np.full((num_blocks, num_kv_heads, head_dim, BLOCK), _NAN_BITS[kv_dtype], dtype=st)
        if kv_dtype == "fp8":
            self.k_scale = np.full(num_blocks, np.nan, dtype=np.float32)
            self.v_scale = np.full(num_blocks, np.nan, dtype=np.float32)
        else:
            self.k_scale = self.v_scale = None


def _bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a CPU tensor (float32 -> uint32, bfloat16 -> uint16)."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(t.dtype)


def _to_f32(t: torch.Tensor) -> np.ndarray:
    """Exact widening of f32 / bf16 source values to float32 (bf16 bits << 16)."""
    b = _bits(t)
    if b.dtype == np.uint16:
        return (b.astype(np.uint32) << 16).view(np.float32)
    return b.view(np.float32)


def _quantize_page(x: np.ndarray):
    """One page's worth of values (float32) -> (E4M3 codes, float32 scale).
    scale = amax / 448 rounded to float32 (1 when amax is 0); each code is the
    nearest-even E4M3 value to x / scale (float32 division), clamped to +-448."""
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    if amax == 0:
        s = np.float32(1.0)
    else:
        s = np.float32(amax / np.float32(fp8_e4m3.FP8_MAX))
    y = (x.astype(np.float32) / s).astype(np.float32)
    y = np.clip(y, np.float32(-fp8_e4m3.FP8_MAX), np.float32(fp8_e4m3.FP8_MAX))
    return fp8_e4m3.encode_rne(y), s


def write_kv(pool: OraclePool, k_src: torch.Tensor, v_src: torch.Tensor,
             slot_mapping: torch.Tensor) -> None:
    """Scatter token t's K/V ([Hkv, d] each) to slot_mapping[t] = page*16 + offset.

    For an fp8 pool, each page touched by this write gets one K and one V scale
    from the amax over every value this write puts in that page (all heads,
    all dims, all its tokens), and all its written tokens are quantised with it.
    """
    slots = slot_mapping.numpy().astype(np.int64)
    pages, offs = slots // BLOCK, slots % BLOCK
    assert ((pages >= 0) & (pages < pool.num_blocks)).all()
    if pool.kv_dtype in ("f32", "bf16"):
        want = torch.float32 if pool.kv_dtype == "f32" else torch.bfloat16
        assert k_src.dtype == want and v_src.dtype == want
        kb, vb = _bits(k_src), _bits(v_src)          # [n, Hkv, d]
        pool.k[pages, :, offs, :] = kb
        pool.v[pages, :, :, offs] = vb
        return
    kf, vf = _to_f32(k_src), _to_f32(v_src)
    order = np.argsort(pages, kind="stable")
    uniq, starts = np.unique(pages[order], return_index=True)
    bounds = list(starts) + [len(order)]
    for i, p in enumerate(uniq):
        toks = order[bounds[i]:bounds[i + 1]]
        for src, dst, scales, transpose in ((kf, pool.k, pool.k_scale, False),
                                            (vf, pool.v, pool.v_scale, True)):
            codes, s = _quantize_page(src[toks])        # [n_p, Hkv, d]
            scales[p] = s
            for j, t in enumerate(toks):
                if transpose:
                    dst[p, :, :, offs[t]] = codes[j]
                else:
                    dst[p, :, offs[t], :] = codes[j]


def _decode(bits: np.ndarray, kv_dtype: str, scale=None) -> np.ndarray:
    if kv_dtype == "f32":
        return bits.view(np.float32).astype(np.float64)
    if kv_dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return fp8_e4m3.decode(bits) * np.float64(scale)


def gather_kv(pool: OraclePool, block_table_row, ctx_len: int, kv_head: int):
    """K, V of one sequence and KV head as float64 [ctx_len, d], found page by
    page through the block table (logical page j -> physical page bt[j])."""
    d = pool.head_dim
    K = np.empty((ctx_len, d), dtype=np.float64)
    V = np.empty((ctx_len, d), dtype=np.float64)
    for j in range((ctx_len + BLOCK - 1) // BLOCK):
        p = int(block_table_row[j])
        assert 0 <= p < pool.num_blocks, f"block table entry {p} out of range"
        n = min(BLOCK, ctx_len - j * BLOCK)
        ks = pool.k_scale[p] if pool.kv_dtype == "fp8" else None
        vs = pool.v_scale[p] if pool.kv_dtype == "fp8" else None
        K[j * BLOCK: j * BLOCK + n] = _decode(pool.k[p, kv_head, :n, :], pool.kv_dtype, ks)
        V[j * BLOCK: j * BLOCK + n] = _decode(pool.v[p, kv_head, :, :n].T, pool.kv_dtype, vs)
    return K, V


def append_kv(pool: OraclePool, k_src: torch.Tensor, v_src: torch.Tensor,
              slot_mapping: torch.Tensor) -> None:
    """Append token t's K/V to slot_mapping[t], keeping the tokens a touched page
    already holds: those at offsets below the lowest offset written to it here.

    f32 / bf16 pools: the same copy as write_kv.  fp8 pools: per touched page,
    the existing tokens' values as stored (code times the old scale, in float32)
    and the new values share one new scale (amax over both, all heads, / 448)
    and are all encoded with it, nearest even after clamping to +-448.
    """
    if pool.kv_dtype in ("f32", "bf16"):
        write_kv(pool, k_src, v_src, slot_mapping)
        return
    slots = slot_mapping.numpy().astype(np.int64)
    pages, offs = slots // BLOCK, slots % BLOCK
    assert ((pages >= 0) & (pages < pool.num_blocks)).all()
    kf, vf = _to_f32(k_src), _to_f32(v_src)                      # [n, Hkv, d]
    table = fp8_e4m3.decode_table().astype(np.float32)
    for p in np.unique(pages):
        toks = np.nonzero(pages == p)[0]
        m = int(offs[toks].min())                                  # existing: offsets < m
        # K: page rows are tokens; V: page columns are tokens
        old_k = table[pool.k[p, :, :m, :]] * np.float32(pool.k_scale[p]) if m else None
        old_v = table[pool.v[p, :, :, :m]] * np.float32(pool.v_scale[p]) if m else None
        new_k = kf[toks]                                           # [n_p, Hkv, d]
        new_v = vf[toks]
        # one quantisation over [existing; new] values of the page
        k_all = new_k.reshape(-1) if old_k is None else np.concatenate(
            [old_k.astype(np.float32).reshape(-1), new_k.reshape(-1)])
        v_all = new_v.reshape(-1) if old_v is None else np.concatenate(
            [old_v.astype(np.float32).reshape(-1), new_v.reshape(-1)])
        k_codes, ks = _quantize_page(k_all)
        v_codes, vs = _quantize_page(v_all)
        pool.k_scale[p], pool.v_scale[p] = ks, vs
        nk_old = 0 if old_k is None else old_k.size
        nv_old = 0 if old_v is None else old_v.size
        if m:
            pool.k[p, :, :m, :] = k_codes[:nk_old].reshape(old_k.shape)
            pool.v[p, :, :, :m] = v_codes[:nv_old].reshape(old_v.shape)
        kn = k_codes[nk_old:].reshape(new_k.shape)
        vn = v_codes[nv_old:].reshape(new_v.shape)
        for j, t in enumerate(toks):
            pool.k[p, :, offs[t], :] = kn[j]
            pool.v[p, :, :, offs[t]] = vn[j]


def copy_blocks(pool: OraclePool, src, dst) -> None:
    """Block dst[i] becomes a copy of block src[i] (both pools, and fp8 scales)."""
    for s, d in zip(list(src), list(dst)):
        pool.k[d] = pool.k[s]
        pool.v[d] = pool.v[s]
        if pool.kv_dtype == "fp8":
            pool.k_scale[d] = pool.k_scale[s]
            pool.v_scale[d] = pool.v_scale[s]
