"""Paged attention forward for MI355X: Python binding of libpa.so.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of libpa.so; PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing, importing this package
raises.

The function names follow the C ABI in include/pa.h:
  write_kv, gather_kv, prefill, decode, decode_num_splits,
  decode_workspace_bytes, write_kv_workspace_bytes, BlockAllocator.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_OOM, PA_ERR_LAUNCH = \
    0, -1, -2, -3, -4, -5
PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
BLOCK_SIZE = 16

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python online_softmax_paged_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)


class _Pool(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int)]


_P, _I32, _F, _SZ, _VP = ctypes.POINTER(_Pool), ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype, f.argtypes = res, args
    return f


_status_string = _sig("pa_status_string", ctypes.c_char_p, [ctypes.c_int])
_abi_version = _sig("pa_abi_version", _I32, [])
_write_ws = _sig("pa_write_kv_workspace_bytes", _SZ, [_P])
_write = _sig("pa_write_kv", ctypes.c_int, [_P, _VP, _VP, ctypes.c_int, _VP, _I32, _VP, _SZ, _VP])
_gather = _sig("pa_gather_kv", ctypes.c_int, [_P, _VP, _I32, _VP, _VP, _I32, _I32, _VP, _VP, _VP])
_prefill = _sig("pa_prefill", ctypes.c_int,
                [_P, _VP, ctypes.c_int, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32,
                 _F, _I32, _I32, _VP, _SZ, _VP])
_prefill_fp8 = _sig("pa_prefill_fp8", ctypes.c_int,
                    [_P, _VP, ctypes.c_int, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32,
                     _F, _I32, _I32, _VP, _SZ, _VP])
_pre_splits = _sig("pa_prefill_num_splits", _I32, [_I32, _I32, _I32, _I32, _I32])
_pre_ws = _sig("pa_prefill_workspace_bytes", _SZ, [_I32, _I32, _I32, _I32, _I32])


class _SharedPlan(ctypes.Structure):
    """pa_shared_plan."""
    _fields_ = [("mode", ctypes.c_int32), ("prefix_splits", ctypes.c_int32),
                ("suffix_splits", ctypes.c_int32), ("plain_splits", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


_SPP = ctypes.POINTER(_SharedPlan)
_sp_plan = _sig("pa_shared_prefix_plan", ctypes.c_int,
                [_P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _SPP])
_sp_ws = _sig("pa_shared_prefix_workspace_bytes", _SZ, [_P, _I32, _I32, _I32, _SPP])
_prefill_sp = _sig("pa_prefill_shared_prefix", ctypes.c_int,
                   [_P, _VP, ctypes.c_int, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32,
                    _F, _I32, _I32, _I32, _SPP, _VP, _SZ, _VP])
_bwd_ws = _sig("pa_backward_workspace_bytes", _SZ, [_P, _I32, _I32, _I32])
_bwd = _sig("pa_prefill_backward", ctypes.c_int,
            [_P, _VP, _VP, _VP, _VP, ctypes.c_int, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32,
             _I32, _I32, _F, _I32, _VP, _SZ, _VP])
_num_splits = _sig("pa_decode_num_splits", _I32, [_I32, _I32, _I32])
_choose_splits = _sig("pa_decode_choose_splits", _I32, [_I32, _I32, _I32, ctypes.c_int64])
_dec_ws = _sig("pa_decode_workspace_bytes", _SZ, [_I32, _I32, _I32, _I32])
_dec_bal_ws = _sig("pa_decode_balanced_workspace_bytes", _SZ, [_I32, _I32, _I32, _I32, _I32])
_decode = _sig("pa_decode", ctypes.c_int,
               [_P, _VP, ctypes.c_int, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _F, _I32,
                _VP, _SZ, _VP])
_decode_noalloc = _sig("pa_decode_noalloc", ctypes.c_int,
                      [_P, _VP, ctypes.c_int, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _F,
                       _I32, _VP])
_alloc_create = _sig("pa_allocator_create", _VP, [_I32])
_alloc_destroy = _sig("pa_allocator_destroy", None, [_VP])
_alloc_block = _sig("pa_alloc_block", _I32, [_VP])
_incref = _sig("pa_block_incref", ctypes.c_int, [_VP, _I32])
_decref = _sig("pa_block_decref", ctypes.c_int, [_VP, _I32])
_refcount = _sig("pa_block_refcount", _I32, [_VP, _I32])
_num_free = _sig("pa_num_free_blocks", _I32, [_VP])
_append = _sig("pa_append_kv", ctypes.c_int, [_P, _VP, _VP, ctypes.c_int, _VP, _I32, _VP, _SZ, _VP])
_copy_blocks = _sig("pa_copy_blocks", ctypes.c_int, [_P, _VP, _VP, _I32, _VP])
_plan_append = _sig("pa_plan_append", ctypes.c_int,
                    [_VP, _VP, _I32, _VP, _VP, _I32, _VP, _VP, _VP, _I32, _VP])
_probe_read = _sig("pa_probe_stream_read", ctypes.c_int, [_VP, _SZ, _VP, _I32, _VP])
_probe_page = _sig("pa_probe_page_stream", ctypes.c_int, [_VP, _SZ, _VP, _I32, _VP])
_probe_mfma = _sig("pa_probe_mfma", ctypes.c_int, [ctypes.c_int, _VP, _I32, _I32, _VP])

EXPORTED = ["pa_status_string", "pa_abi_version", "pa_write_kv_workspace_bytes", "pa_write_kv",
            "pa_gather_kv", "pa_prefill", "pa_decode_num_splits", "pa_decode_workspace_bytes",
            "pa_decode", "pa_allocator_create", "pa_allocator_destroy", "pa_alloc_block",
            "pa_block_incref", "pa_block_decref", "pa_block_refcount", "pa_num_free_blocks",
            "pa_append_kv", "pa_copy_blocks", "pa_plan_append", "pa_prefill_num_splits",
            "pa_prefill_workspace_bytes", "pa_shared_prefix_plan",
            "pa_shared_prefix_workspace_bytes", "pa_prefill_shared_prefix",
            "pa_decode_balanced_workspace_bytes", "pa_decode_choose_splits",
            "pa_backward_workspace_bytes", "pa_prefill_backward", "pa_prefill_fp8",
            "pa_probe_stream_read", "pa_probe_page_stream", "pa_probe_mfma", "pa_decode_noalloc"]

SCRATCH_BYTES = 8 << 20   # PA_SCRATCH_BYTES

DECODE_BALANCED = -1


class PAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


def status_string(s: int) -> str:
    return _status_string(s).decode()


def abi_version() -> int:
    return int(_abi_version())


def _check(status: int, what: str):
    if status != PA_OK:
        raise PAError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_DT = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.uint8: PA_FP8_E4M3}
_NAMES = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}


class KVPool:
    """Device tensors of one KV block pool (layout in include/pa.h):
    k [NB, Hkv, 16, D], v [NB, Hkv, D, 16]; fp8 pools are uint8 codes plus
    float32 k_scale / v_scale [NB]."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, kv_dtype: str,
                 device="cuda", fill_nan: bool = True):
        dt = _NAMES[kv_dtype]
        self.num_blocks, self.num_kv_heads, self.head_dim = num_blocks, num_kv_heads, head_dim
        self.kv_dtype = kv_dtype
        nan = {"f32": float("nan"), "bf16": float("nan"), "fp8": 0x7F}[kv_dtype]
        shape_k = (num_blocks, num_kv_heads, BLOCK_SIZE, head_dim)
        shape_v = (num_blocks, num_kv_heads, head_dim, BLOCK_SIZE)
        if fill_nan:
            self.k = torch.full(shape_k, nan, dtype=dt, device=device)
            self.v = torch.full(shape_v, nan, dtype=dt, device=device)
        else:
            self.k = torch.empty(shape_k, dtype=dt, device=device)
            self.v = torch.empty(shape_v, dtype=dt, device=device)
        if kv_dtype == "fp8":
            self.k_scale = torch.full((num_blocks,), float("nan"), dtype=torch.float32, device=device)
            self.v_scale = torch.full((num_blocks,), float("nan"), dtype=torch.float32, device=device)
        else:
            self.k_scale = self.v_scale = None
        self._c = _Pool(self.k.data_ptr(), self.v.data_ptr(),
                        self.k_scale.data_ptr() if self.k_scale is not None else None,
                        self.v_scale.data_ptr() if self.v_scale is not None else None,
                        num_blocks, num_kv_heads, head_dim, BLOCK_SIZE, _DT[dt])

    @property
    def c(self):
        return ctypes.byref(self._c)

    def nbytes(self) -> int:
        n = self.k.numel() * self.k.element_size() * 2
        if self.k_scale is not None:
            n += 2 * self.k_scale.numel() * 4
        return n


def write_kv_workspace_bytes(pool: KVPool) -> int:
    return int(_write_ws(pool.c))


def write_kv(pool: KVPool, k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
             workspace: torch.Tensor | None = None, stream=None):
    """Scatter (and for fp8 pools, quantise per block) new tokens into the pool."""
    n = int(slot_mapping.numel())
    need = write_kv_workspace_bytes(pool)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=k_new.device)
    _check(_write(pool.c, _ptr(k_new), _ptr(v_new), _DT[k_new.dtype], _ptr(slot_mapping), n,
                  _ptr(workspace), 0 if workspace is None else workspace.numel(),
                  _stream(stream)), "pa_write_kv")


def append_kv(pool: KVPool, k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
              workspace: torch.Tensor | None = None, stream=None):
    """Append tokens to partly filled pages (fp8 pools re-quantise each touched page)."""
    n = int(slot_mapping.numel())
    need = write_kv_workspace_bytes(pool)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=k_new.device)
    _check(_append(pool.c, _ptr(k_new), _ptr(v_new), _DT[k_new.dtype], _ptr(slot_mapping), n,
                   _ptr(workspace), 0 if workspace is None else workspace.numel(),
                   _stream(stream)), "pa_append_kv")


def copy_blocks(pool: KVPool, src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Device copy of whole blocks: dst[i] <- src[i] (int32 device tensors)."""
    n = int(src.numel())
    if n != int(dst.numel()):
        raise ValueError("src and dst differ in length")
    _check(_copy_blocks(pool.c, _ptr(src), _ptr(dst), n, _stream(stream)), "pa_copy_blocks")


def gather_kv(pool: KVPool, block_table, ctx_lens, max_ctx_len: int, stream=None):
    """Copy each sequence's tokens out of the pool -> (k, v) [sum ctx, Hkv, D]."""
    B = int(ctx_lens.numel())
    cu = torch.zeros(B + 1, dtype=torch.int32, device=ctx_lens.device)
    cu[1:] = torch.cumsum(ctx_lens, 0)
    total = int(cu[-1].item())
    shape = (total, pool.num_kv_heads, pool.head_dim)
    k_out = torch.empty(shape, dtype=pool.k.dtype, device=pool.k.device)
    v_out = torch.empty(shape, dtype=pool.k.dtype, device=pool.k.device)
    _check(_gather(pool.c, _ptr(block_table), block_table.shape[1], _ptr(ctx_lens), _ptr(cu), B,
                   max_ctx_len, _ptr(k_out), _ptr(v_out), _stream(stream)), "pa_gather_kv")
    return k_out, v_out


def _validate(pool: KVPool, ctx_lens, block_table, q_lens=None):
    """Host-side check of the device-resident metadata contract (copies to CPU)."""
    ctx = ctx_lens.cpu().tolist()
    bt = block_table.cpu()
    for b, c in enumerate(ctx):
        if c < 1:
            raise ValueError(f"sequence {b}: ctx_len {c} < 1")
        n = (c + BLOCK_SIZE - 1) // BLOCK_SIZE
        if n > bt.shape[1]:
            raise ValueError(f"sequence {b}: block table too short")
        ids = bt[b, :n]
        if (ids < 0).any() or (ids >= pool.num_blocks).any():
            raise ValueError(f"sequence {b}: block id out of range")
        if q_lens is not None and not (1 <= q_lens[b] <= c):
            raise ValueError(f"sequence {b}: q_len {q_lens[b]} not in [1, {c}]")


def prefill_num_splits(num_seqs: int, num_kv_heads: int, num_q_heads: int, max_q_len: int,
                       max_ctx_len: int) -> int:
    return int(_pre_splits(num_seqs, num_kv_heads, num_q_heads, max_q_len, max_ctx_len))


def prefill_workspace_bytes(num_seqs: int, max_q_len: int, num_q_heads: int, head_dim: int,
                            num_splits: int) -> int:
    return int(_pre_ws(num_seqs, max_q_len, num_q_heads, head_dim, num_splits))


def prefill(pool: KVPool, q: torch.Tensor, cu_q_lens, ctx_lens, block_table, scale: float,
            causal: bool = True, max_q_len: int | None = None, max_ctx_len: int | None = None,
            out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
            num_splits: int = 0, workspace: torch.Tensor | None = None,
            validate: bool = False, stream=None, fp8_products: bool = False):
    """Attention of query chunks (the last q_len_b positions of each sequence).
    Returns (o, lse): o like q, lse float32 [T, Hq].  fp8_products (fp8 pools
    only): Q and P quantised to E4M3 and both products on the fp8 matrix
    cores (pa_prefill_fp8)."""
    B = int(ctx_lens.numel())
    if max_q_len is None or max_ctx_len is None or validate:
        cu = cu_q_lens.cpu()
        q_lens = (cu[1:] - cu[:-1]).tolist()
        if max_q_len is None:
            max_q_len = max(q_lens) if q_lens else 0
        if max_ctx_len is None:
            max_ctx_len = int(ctx_lens.max().item()) if B else 0
        if validate:
            _validate(pool, ctx_lens, block_table, q_lens)
    T, Hq, D = q.shape
    if num_splits == 0:
        num_splits = prefill_num_splits(B, pool.num_kv_heads, Hq, max_q_len, max_ctx_len)
    if pool.kv_dtype == "f32":
        num_splits = 1
    need = prefill_workspace_bytes(B, max_q_len, Hq, D, num_splits)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = out if out is not None else torch.empty_like(q)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    fn, name = (_prefill_fp8, "pa_prefill_fp8") if fp8_products else (_prefill, "pa_prefill")
    _check(fn(pool.c, _ptr(q), _DT[q.dtype], _ptr(o), _ptr(lse), _ptr(cu_q_lens),
              _ptr(ctx_lens), _ptr(block_table), block_table.shape[1], B, Hq, max_q_len,
              max_ctx_len, scale, 1 if causal else 0, num_splits,
              _ptr(workspace) if need else None, workspace.numel() if need else 0,
              _stream(stream)), name)
    return o, lse


SHARED_AUTO, SHARED_PACKED, SHARED_PLAIN = 0, 1, 2   # PA_SHARED_*


def shared_prefix_plan(pool: KVPool, num_seqs: int, num_q_heads: int, max_q_len: int,
                       max_ctx_len: int, prefix_len: int, num_q_tokens: int,
                       mode: int = SHARED_AUTO) -> dict:
    """pa_shared_prefix_plan: the arrangement prefill_shared_prefix takes (SHARED_PACKED
    or SHARED_PLAIN), its split counts and its workspace bytes."""
    p = _SharedPlan()
    _check(_sp_plan(pool.c, num_seqs, num_q_heads, max_q_len, max_ctx_len, prefix_len,
                    num_q_tokens, mode, ctypes.byref(p)), "pa_shared_prefix_plan")
    return {f: getattr(p, f) for f, _ in _SharedPlan._fields_}


def shared_prefix_workspace_bytes(pool: KVPool, num_seqs: int, num_q_heads: int, max_q_len: int,
                                  plan: dict) -> int:
    p = _SharedPlan(**{k: plan[k] for k in ("mode", "prefix_splits", "suffix_splits",
                                            "plain_splits")})
    return int(_sp_ws(pool.c, num_seqs, num_q_heads, max_q_len, ctypes.byref(p)))


def prefill_shared_prefix(pool: KVPool, q: torch.Tensor, cu_q_lens, ctx_lens, block_table,
                          scale: float, prefix_len: int, causal: bool = True,
                          max_q_len: int | None = None, max_ctx_len: int | None = None,
                          out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                          mode: int = SHARED_AUTO, prefix_splits: int = 0,
                          suffix_splits: int = 0, plain_splits: int = 0,
                          workspace: torch.Tensor | None = None, validate: bool = False,
                          stream=None):
    """prefill() for sequences that all start with the same prefix_len tokens in
    the same physical blocks.  SHARED_PACKED: the q_len = 1 rows attend the
    prefix once, packed together, and their own keys separately, the two
    merged; rows with q_len > 1 take prefill()'s pass.  SHARED_PLAIN: the
    whole batch as prefill() / decode().  SHARED_AUTO lets the library choose.
    Nonzero split counts replace the plan's.  Returns (o, lse) as prefill() does."""
    B = int(ctx_lens.numel())
    T, Hq, D = q.shape
    if max_q_len is None or max_ctx_len is None or validate:
        cu = cu_q_lens.cpu()
        q_lens = (cu[1:] - cu[:-1]).tolist()
        if max_q_len is None:
            max_q_len = max(q_lens) if q_lens else 0
        if max_ctx_len is None:
            max_ctx_len = int(ctx_lens.max().item()) if B else 0
        if validate:
            _validate(pool, ctx_lens, block_table, q_lens)
            if int(cu[-1]) != T:
                raise ValueError(f"cu_q_lens ends at {int(cu[-1])}, q has {T} rows")
            bt = block_table.cpu()
            n = prefix_len // 16
            if B and not bool((bt[:, :n] == bt[0:1, :n]).all()):
                raise ValueError("block tables do not share the prefix pages")
            cl = ctx_lens.cpu().tolist()
            for b in range(B):
                if cl[b] - q_lens[b] < prefix_len:
                    raise ValueError(f"sequence {b}: a query lies inside the prefix")
    if B == 0:
        return (out if out is not None else torch.empty_like(q),
                lse if lse is not None else torch.empty((T, Hq), dtype=torch.float32,
                                                        device=q.device))
    plan = shared_prefix_plan(pool, B, Hq, max_q_len, max_ctx_len, prefix_len, T, mode)
    plan["prefix_splits"] = prefix_splits or plan["prefix_splits"]
    plan["suffix_splits"] = suffix_splits or plan["suffix_splits"]
    plan["plain_splits"] = plain_splits or plan["plain_splits"]
    need = shared_prefix_workspace_bytes(pool, B, Hq, max_q_len, plan)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = out if out is not None else torch.empty_like(q)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    cplan = _SharedPlan(plan["mode"], plan["prefix_splits"], plan["suffix_splits"],
                        plan["plain_splits"], need)
    _check(_prefill_sp(pool.c, _ptr(q), _DT[q.dtype], _ptr(o), _ptr(lse), _ptr(cu_q_lens),
                       _ptr(ctx_lens), _ptr(block_table), block_table.shape[1], B, Hq, max_q_len,
                       max_ctx_len, scale, 1 if causal else 0, prefix_len, T,
                       ctypes.byref(cplan), _ptr(workspace) if need else None,
                       workspace.numel() if need else 0, _stream(stream)),
           "pa_prefill_shared_prefix")
    return o, lse


def backward_workspace_bytes(pool: KVPool, num_seqs: int, num_q_heads: int,
                             max_q_len: int) -> int:
    return int(_bwd_ws(pool.c, num_seqs, num_q_heads, max_q_len))


def prefill_backward(pool: KVPool, q: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                     dout: torch.Tensor, cu_q_lens, ctx_lens, block_table, scale: float,
                     causal: bool = True, max_q_len: int | None = None,
                     max_ctx_len: int | None = None, dq: torch.Tensor | None = None,
                     dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, validate: bool = False,
                     stream=None):
    """Gradients of prefill() for the upstream gradient dout, from its o and
    lse.  Returns (dq [T, Hq, d], dk shaped like pool.k, dv shaped like
    pool.v), all float32; dk and dv are zero on pages no sequence uses
    (allocated zeroed here when not given)."""
    B = int(ctx_lens.numel())
    T, Hq, D = q.shape
    if max_q_len is None or max_ctx_len is None or validate:
        cu = cu_q_lens.cpu()
        q_lens = (cu[1:] - cu[:-1]).tolist()
        if max_q_len is None:
            max_q_len = max(q_lens) if q_lens else 0
        if max_ctx_len is None:
            max_ctx_len = int(ctx_lens.max().item()) if B else 0
        if validate:
            _validate(pool, ctx_lens, block_table, q_lens)
            bt, cl = block_table.cpu(), ctx_lens.cpu().tolist()
            used = [int(x) for b in range(B) for x in bt[b, :(cl[b] + 15) // 16].tolist()]
            if len(used) != len(set(used)):
                raise ValueError("a physical page is used twice: its gradient would race")
    dq = dq if dq is not None else torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    dk = dk if dk is not None else torch.zeros(pool.k.shape, dtype=torch.float32, device=q.device)
    dv = dv if dv is not None else torch.zeros(pool.v.shape, dtype=torch.float32, device=q.device)
    if B == 0:
        return dq, dk, dv
    need = backward_workspace_bytes(pool, B, Hq, max_q_len)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(_bwd(pool.c, _ptr(q), _ptr(o), _ptr(lse), _ptr(dout), _DT[q.dtype], _ptr(dq), _ptr(dk),
                _ptr(dv), _ptr(cu_q_lens), _ptr(ctx_lens), _ptr(block_table), block_table.shape[1],
                B, Hq, max_q_len, max_ctx_len, scale, 1 if causal else 0, _ptr(workspace),
                workspace.numel(), _stream(stream)), "pa_prefill_backward")
    return dq, dk, dv


def decode_num_splits(num_seqs: int, num_kv_heads: int, max_ctx_len: int) -> int:
    return int(_num_splits(num_seqs, num_kv_heads, max_ctx_len))


def decode_choose_splits(num_seqs: int, num_kv_heads: int, max_ctx_len: int,
                         total_ctx_len: int) -> int:
    """Split count, or DECODE_BALANCED for batches of very uneven lengths."""
    return int(_choose_splits(num_seqs, num_kv_heads, max_ctx_len, total_ctx_len))


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, num_splits: int) -> int:
    return int(_dec_ws(num_seqs, num_q_heads, head_dim, num_splits))


def decode_balanced_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                    head_dim: int, max_ctx_len: int) -> int:
    return int(_dec_bal_ws(num_seqs, num_q_heads, num_kv_heads, head_dim, max_ctx_len))


def decode(pool: KVPool, q: torch.Tensor, ctx_lens, block_table, scale: float,
           max_ctx_len: int | None = None, num_splits: int = 0,
           workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
           lse: torch.Tensor | None = None, validate: bool = False, stream=None,
           total_ctx_len: int | None = None):
    """One query per sequence at its last position.  Returns (o, lse).
    With num_splits = 0 the library chooses; total_ctx_len (the sum of the
    lengths, if the caller knows it) lets it pick the balanced kernel for very
    uneven batches.  Lengths are read back from the device only when
    max_ctx_len is not given."""
    B, Hq, D = q.shape
    if max_ctx_len is None:
        cl = ctx_lens.cpu()
        max_ctx_len = int(cl.max().item())
        if total_ctx_len is None:
            total_ctx_len = int(cl.clamp(min=0).sum().item())
    if validate:
        _validate(pool, ctx_lens, block_table)
    if num_splits == 0:
        if pool.kv_dtype != "f32" and total_ctx_len:
            num_splits = decode_choose_splits(B, pool.num_kv_heads, max_ctx_len, total_ctx_len)
        else:
            num_splits = decode_num_splits(B, pool.num_kv_heads, max_ctx_len)
    if num_splits == DECODE_BALANCED:
        need = decode_balanced_workspace_bytes(B, Hq, pool.num_kv_heads, D, max_ctx_len)
    else:
        need = decode_workspace_bytes(B, Hq, D, num_splits)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = out if out is not None else torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(_decode(pool.c, _ptr(q), _DT[q.dtype], _ptr(o), _ptr(lse), _ptr(ctx_lens),
                   _ptr(block_table), block_table.shape[1], B, Hq, max_ctx_len, scale,
                   num_splits, _ptr(workspace), 0 if workspace is None else workspace.numel(),
                   _stream(stream)), "pa_decode")
    return o, lse


def decode_noalloc(pool: KVPool, q: torch.Tensor, ctx_lens, block_table, scale: float,
                   max_ctx_len: int, out: torch.Tensor, lse: torch.Tensor, num_splits: int = 0,
                   stream=None):
    """pa_decode_noalloc: pa_decode with the split partials in the library's
    fixed per-device array, for callers that cannot allocate.  Allocates
    nothing here either: out and lse are the caller's.  Calls that may overlap
    on one GPU race (they share the array)."""
    B, Hq, _ = q.shape
    _check(_decode_noalloc(pool.c, _ptr(q), _DT[q.dtype], _ptr(out), _ptr(lse), _ptr(ctx_lens),
                           _ptr(block_table), block_table.shape[1], B, Hq, max_ctx_len, scale,
                           num_splits, _stream(stream)), "pa_decode_noalloc")
    return out, lse


class BlockAllocator:
    """Host block allocator of the library (free list + reference counts)."""

    def __init__(self, num_blocks: int):
        self._h = _alloc_create(num_blocks)
        if not self._h:
            raise ValueError("pa_allocator_create failed")

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            _alloc_destroy(h)

    def alloc(self) -> int:
        return int(_alloc_block(self._h))

    def incref(self, block: int):
        _check(_incref(self._h, block), "pa_block_incref")

    def decref(self, block: int):
        _check(_decref(self._h, block), "pa_block_decref")

    def refcount(self, block: int) -> int:
        return int(_refcount(self._h, block))

    def num_free(self) -> int:
        return int(_num_free(self._h))

    def plan_append(self, block_table: torch.Tensor, ctx_lens: torch.Tensor, num_new):
        """Host planning of an append (pa_plan_append).  block_table [B, W] and
        ctx_lens [B] are contiguous int32 CPU tensors, updated in place.
        Returns (slot_mapping int32 CPU tensor, copy_src, copy_dst int32 CPU
        tensors of the blocks to copy before appending)."""
        for t in (block_table, ctx_lens):
            if t.device.type != "cpu" or t.dtype != torch.int32 or not t.is_contiguous():
                raise ValueError("block_table and ctx_lens must be contiguous int32 CPU tensors")
        B = int(ctx_lens.numel())
        nn = torch.as_tensor(num_new, dtype=torch.int32).contiguous()
        slots = torch.empty(max(1, int(nn.sum())), dtype=torch.int32)
        csrc = torch.empty(max(1, B), dtype=torch.int32)
        cdst = torch.empty(max(1, B), dtype=torch.int32)
        nc = ctypes.c_int32(0)
        _check(_plan_append(self._h, _ptr(block_table), block_table.shape[1], _ptr(ctx_lens),
                            _ptr(nn), B, _ptr(slots), _ptr(csrc), _ptr(cdst), B,
                            ctypes.byref(nc)), "pa_plan_append")
        k = int(nn.sum())
        return slots[:k], csrc[:nc.value], cdst[:nc.value]


# ------------------------------------------------------------ measurement probes
def probe_stream_read(buf: torch.Tensor, blocks: int = 2048, out: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """Read every byte of the contiguous device tensor buf once (pa_probe_stream_read);
    returns the per-thread XORs (int32 [blocks * 256])."""
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.int32, device=buf.device)
    _check(_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), blocks,
                       _stream(stream)), "pa_probe_stream_read")
    return out


def probe_page_stream(buf: torch.Tensor, blocks: int = 256, out: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """Read buf in the decode's page pattern, evenly over `blocks` workgroups
    (pa_probe_page_stream); returns the per-thread XORs."""
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.int32, device=buf.device)
    _check(_probe_page(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), blocks,
                       _stream(stream)), "pa_probe_page_stream")
    return out


PROBE_MFMA_FLOP = {"bf16": 32 * 32 * 16 * 2, "fp8": 32 * 32 * 64 * 2}


def probe_mfma(dtype: str = "bf16", blocks: int = 2048, iters: int = 2000,
               out: torch.Tensor | None = None, stream=None) -> float:
    """Run the MFMA loop (pa_probe_mfma); returns the FLOP it performs."""
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    dt = {"bf16": PA_BF16, "fp8": PA_FP8_E4M3}[dtype]
    _check(_probe_mfma(dt, _ptr(out), blocks, iters, _stream(stream)), "pa_probe_mfma")
    return float(blocks) * 16 * iters * PROBE_MFMA_FLOP[dtype]
