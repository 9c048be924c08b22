// C ABI of libpa: host-side argument checks, then dispatch to the launchers.
// Every check runs before anything is enqueued; no HIP call happens on a
// failed check.
#include <math.h>

#include <atomic>
#include <mutex>

#include "pa_internal.h"

using namespace pa;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pa_status check_pool(const pa_kv_pool* pool) {
  if (!pool || !pool->k || !pool->v) return PA_ERR_INVALID_ARG;
  if (pool->block_size != PA_BLOCK_SIZE) return PA_ERR_UNSUPPORTED;
  if (pool->num_blocks < 1 || pool->num_kv_heads < 1) return PA_ERR_INVALID_ARG;
  if (pool->head_dim != 64 && pool->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (pool->kv_dtype != PA_F32 && pool->kv_dtype != PA_BF16 && pool->kv_dtype != PA_FP8_E4M3)
    return PA_ERR_INVALID_ARG;
  if (pool->kv_dtype == PA_FP8_E4M3 && (!pool->k_scale || !pool->v_scale))
    return PA_ERR_INVALID_ARG;
  if (!aligned16(pool->k) || !aligned16(pool->v)) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

pa_status check_attn(const pa_kv_pool* pool, const void* q, pa_dtype q_dtype, const void* o,
                     const int32_t* ctx_lens, const int32_t* block_table, int32_t bt_stride,
                     int32_t num_seqs, int32_t num_q_heads, int32_t max_ctx_len, float scale) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  if (num_seqs < 0) return PA_ERR_INVALID_ARG;
  if (!q || !o || !ctx_lens || !block_table) return PA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o)) return PA_ERR_INVALID_ARG;
  if (q_dtype == PA_F32) {
    if (pool->kv_dtype != PA_F32) return PA_ERR_UNSUPPORTED;
  } else if (q_dtype == PA_BF16) {
    if (pool->kv_dtype != PA_BF16 && pool->kv_dtype != PA_FP8_E4M3) return PA_ERR_UNSUPPORTED;
  } else {
    return PA_ERR_UNSUPPORTED;
  }
  if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  int g = num_q_heads / pool->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return PA_ERR_UNSUPPORTED;
  if (max_ctx_len < 1) return PA_ERR_INVALID_ARG;
  if (bt_stride < (max_ctx_len + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE) return PA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

AttnArgs make_args(const pa_kv_pool* pool, const void* q, void* o, float* lse,
                   const int32_t* ctx_lens, const int32_t* block_table, int32_t bt_stride,
                   int32_t num_seqs, int32_t num_q_heads, int32_t max_ctx_len, float scale) {
  AttnArgs a{};
  a.k = pool->k;
  a.v = pool->v;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.num_blocks = pool->num_blocks;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.kv_dtype = pool->kv_dtype;
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.ctx_lens = ctx_lens;
  a.block_table = block_table;
  a.bt_stride = bt_stride;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.max_ctx_len = max_ctx_len;
  a.scale = scale;
  return a;
}

pa_status launched(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, group size or block size";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_OOM: return "no free block";
    case PA_ERR_LAUNCH: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t pa_abi_version(void) { return 8; }

size_t pa_write_kv_workspace_bytes(const pa_kv_pool* pool) {
  if (!pool || pool->kv_dtype != PA_FP8_E4M3 || pool->num_blocks < 1) return 0;
  return 3 * sizeof(uint32_t) * static_cast<size_t>(pool->num_blocks);
}

}  // extern "C"

namespace {

pa_status write_or_append(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                          pa_dtype src_dtype, const int32_t* slot_mapping, int32_t num_tokens,
                          void* workspace, size_t workspace_bytes, bool append, void* stream) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return PA_ERR_INVALID_ARG;
  if (pool->kv_dtype == PA_FP8_E4M3) {
    if (src_dtype != PA_F32 && src_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < pa_write_kv_workspace_bytes(pool)) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_INVALID_ARG;
  } else if (src_dtype != pool->kv_dtype) {
    return PA_ERR_UNSUPPORTED;
  }
  return launched(launch_write_kv(*pool, k_new, v_new, src_dtype, slot_mapping, num_tokens,
                                  static_cast<uint32_t*>(workspace), append,
                                  static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

pa_status pa_write_kv(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                      pa_dtype src_dtype, const int32_t* slot_mapping, int32_t num_tokens,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return write_or_append(pool, k_new, v_new, src_dtype, slot_mapping, num_tokens, workspace,
                         workspace_bytes, false, stream);
}

pa_status pa_append_kv(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                       pa_dtype src_dtype, const int32_t* slot_mapping, int32_t num_tokens,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return write_or_append(pool, k_new, v_new, src_dtype, slot_mapping, num_tokens, workspace,
                         workspace_bytes, true, stream);
}

pa_status pa_copy_blocks(const pa_kv_pool* pool, const int32_t* src_blocks,
                         const int32_t* dst_blocks, int32_t num_pairs, void* stream) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!src_blocks || !dst_blocks) return PA_ERR_INVALID_ARG;
  return launched(launch_copy_blocks(*pool, src_blocks, dst_blocks, num_pairs,
                                     static_cast<hipStream_t>(stream)));
}

pa_status pa_gather_kv(const pa_kv_pool* pool, const int32_t* block_table, int32_t bt_stride,
                       const int32_t* ctx_lens, const int32_t* cu_ctx, int32_t num_seqs,
                       int32_t max_ctx_len, void* k_out, void* v_out, void* stream) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  if (num_seqs < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!block_table || !ctx_lens || !cu_ctx || !k_out || !v_out) return PA_ERR_INVALID_ARG;
  if (max_ctx_len < 1 || bt_stride < (max_ctx_len + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE)
    return PA_ERR_INVALID_ARG;
  return launched(launch_gather_kv(*pool, block_table, bt_stride, ctx_lens, cu_ctx, num_seqs,
                                   max_ctx_len, k_out, v_out, static_cast<hipStream_t>(stream)));
}

int32_t pa_prefill_num_splits(int32_t num_seqs, int32_t num_kv_heads, int32_t num_q_heads,
                              int32_t max_q_len, int32_t max_ctx_len) {
  if (num_seqs < 1 || num_kv_heads < 1 || num_q_heads < num_kv_heads || max_q_len < 1 ||
      max_ctx_len < 1)
    return 1;
  // Query tiles hold 128 rows (positions x the group's heads).  Split the keys
  // only when the tiles alone give fewer than 512 workgroups (two per compute
  // unit), keeping at least 8 key tiles of 32 per split.  With enough tiles
  // the kernel is bound by each unit's throughput, not by the length of a
  // tile's key loop (8 x 256 queries over 1536 fp8 keys: 85 us unsplit, 85 us
  // with 2 splits plus 26 us of merge); with few it is not (1 x 256 queries
  // over 8192 bf16 keys: 214 us unsplit, 70 us with 4 splits, 60 us with 8).
  const int64_t G = num_q_heads / num_kv_heads;
  const int64_t tq = G >= 128 ? 1 : 128 / G;
  const int64_t tiles = (max_q_len + tq - 1) / tq;
  const int64_t wgs = static_cast<int64_t>(num_seqs) * num_kv_heads * tiles;
  int64_t s = (512 + wgs - 1) / wgs;
  const int64_t by_keys = (max_ctx_len + 32 * 8 - 1) / (32 * 8);
  if (s > by_keys) s = by_keys;
  if (s > 16) s = 16;
  return static_cast<int32_t>(s < 1 ? 1 : s);
}

size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads,
                                  int32_t head_dim, int32_t num_splits) {
  if (num_seqs < 1 || max_q_len < 1 || num_q_heads < 1 || head_dim < 1 || num_splits <= 1)
    return 0;
  const size_t rows = static_cast<size_t>(num_splits) * num_seqs * max_q_len * num_q_heads;
  const size_t o_bytes = (rows * head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
  return o_bytes + rows * sizeof(float);
}

static pa_status prefill_impl(const pa_kv_pool* pool, const void* q, pa_dtype q_dtype, void* o,
                              float* lse, const int32_t* cu_q_lens, const int32_t* ctx_lens,
                              const int32_t* block_table, int32_t bt_stride, int32_t num_seqs,
                              int32_t num_q_heads, int32_t max_q_len, int32_t max_ctx_len,
                              float scale, int32_t causal, int32_t num_splits, void* workspace,
                              size_t workspace_bytes, void* stream, bool fp8_mma) {
  if (num_seqs == 0 && pool) return check_pool(pool);
  pa_status s = check_attn(pool, q, q_dtype, o, ctx_lens, block_table, bt_stride, num_seqs,
                           num_q_heads, max_ctx_len, scale);
  if (s != PA_OK) return s;
  if (!cu_q_lens || max_q_len < 1 || max_q_len > max_ctx_len) return PA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > 16) return PA_ERR_INVALID_ARG;
  if (num_splits == 0)
    num_splits = pa_prefill_num_splits(num_seqs, pool->num_kv_heads, num_q_heads, max_q_len,
                                       max_ctx_len);
  if (pool->kv_dtype == PA_F32) num_splits = 1;  // the fp32 kernel does not split keys
  if (fp8_mma && pool->kv_dtype != PA_FP8_E4M3) return PA_ERR_UNSUPPORTED;
  AttnArgs a = make_args(pool, q, o, lse, ctx_lens, block_table, bt_stride, num_seqs,
                         num_q_heads, max_ctx_len, scale);
  a.fp8_mma = fp8_mma ? 1 : 0;
  a.cu_q_lens = cu_q_lens;
  a.max_q_len = max_q_len;
  a.causal = causal ? 1 : 0;
  a.num_splits = num_splits;
  if (num_splits > 1) {
    const size_t need = pa_prefill_workspace_bytes(num_seqs, max_q_len, num_q_heads,
                                                   pool->head_dim, num_splits);
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_INVALID_ARG;
    const size_t rows = static_cast<size_t>(num_splits) * num_seqs * max_q_len * num_q_heads;
    const size_t o_bytes = (rows * pool->head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
    a.ws_o = static_cast<float*>(workspace);
    a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
    a.part_rows = static_cast<int64_t>(num_seqs) * max_q_len;
  }
  return launched(launch_prefill(a, static_cast<hipStream_t>(stream)));
}

pa_status pa_prefill(const pa_kv_pool* pool, const void* q, pa_dtype q_dtype, void* o,
                     float* lse, const int32_t* cu_q_lens, const int32_t* ctx_lens,
                     const int32_t* block_table, int32_t bt_stride, int32_t num_seqs,
                     int32_t num_q_heads, int32_t max_q_len, int32_t max_ctx_len,
                     float scale, int32_t causal, int32_t num_splits, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return prefill_impl(pool, q, q_dtype, o, lse, cu_q_lens, ctx_lens, block_table, bt_stride,
                      num_seqs, num_q_heads, max_q_len, max_ctx_len, scale, causal, num_splits,
                      workspace, workspace_bytes, stream, false);
}

pa_status pa_prefill_fp8(const pa_kv_pool* pool, const void* q, pa_dtype q_dtype, void* o,
                         float* lse, const int32_t* cu_q_lens, const int32_t* ctx_lens,
                         const int32_t* block_table, int32_t bt_stride, int32_t num_seqs,
                         int32_t num_q_heads, int32_t max_q_len, int32_t max_ctx_len,
                         float scale, int32_t causal, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return prefill_impl(pool, q, q_dtype, o, lse, cu_q_lens, ctx_lens, block_table, bt_stride,
                      num_seqs, num_q_heads, max_q_len, max_ctx_len, scale, causal, num_splits,
                      workspace, workspace_bytes, stream, true);
}

// Rows with q_len = 1 that a batch can hold at most: every other sequence
// has 2 .. max_q_len queries.
static int64_t most_single_rows(int32_t num_seqs, int32_t max_q_len, int32_t num_q_tokens) {
  if (max_q_len == 1) return num_seqs;
  int64_t n = (static_cast<int64_t>(num_seqs) * max_q_len - num_q_tokens) / (max_q_len - 1);
  return n < 0 ? 0 : (n > num_seqs ? num_seqs : n);
}

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace of a shared-prefix plan, in order: gathered q_len = 1 rows (mixed
// batches), partial outputs and logsumexps of the packed passes, partials of
// the rows with q_len > 1 (mixed batches, plain_splits > 1).  Plain mode uses
// pa_decode's or pa_prefill's workspace.
struct SpLayout {
  size_t qd, o, lse, rest, total;
};
static SpLayout shared_layout(const pa_shared_plan& p, int32_t num_seqs, int32_t num_q_heads,
                              int32_t head_dim, int32_t max_q_len) {
  SpLayout L{};
  if (p.mode == PA_SHARED_PLAIN) {
    L.total = max_q_len == 1
                  ? pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, p.plain_splits)
                  : pa_prefill_workspace_bytes(num_seqs, max_q_len, num_q_heads, head_dim,
                                               p.plain_splits);
    return L;
  }
  const bool mixed = max_q_len > 1;
  const size_t rows = static_cast<size_t>(p.prefix_splits + p.suffix_splits) * num_seqs *
                      num_q_heads;
  size_t off = 0;
  L.qd = off;
  off += mixed ? align256(static_cast<size_t>(num_seqs) * num_q_heads * head_dim * 2) : 0;
  L.o = off;
  off += align256(rows * head_dim * sizeof(float));
  L.lse = off;
  off += align256(rows * sizeof(float));
  L.rest = off;
  if (mixed)
    off += pa_prefill_workspace_bytes(num_seqs, max_q_len, num_q_heads, head_dim, p.plain_splits);
  L.total = off;
  return L;
}

static pa_status check_shared_shape(const pa_kv_pool* pool, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t max_q_len, int32_t max_ctx_len,
                                    int32_t prefix_len, int32_t num_q_tokens) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  if (pool->kv_dtype == PA_F32) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 1 || num_q_heads < pool->num_kv_heads || num_q_heads % pool->num_kv_heads != 0)
    return PA_ERR_INVALID_ARG;
  if (max_q_len < 1 || max_q_len > max_ctx_len) return PA_ERR_INVALID_ARG;
  if (prefix_len < PA_BLOCK_SIZE || prefix_len % PA_BLOCK_SIZE != 0 ||
      prefix_len + max_q_len > max_ctx_len)
    return PA_ERR_INVALID_ARG;
  if (num_q_tokens < 1 ||
      static_cast<int64_t>(num_q_tokens) > static_cast<int64_t>(num_seqs) * max_q_len)
    return PA_ERR_INVALID_ARG;
  // With one query per sequence, row b is sequence b's query.
  if (max_q_len == 1 && num_q_tokens != num_seqs) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

pa_status pa_shared_prefix_plan(const pa_kv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                int32_t max_q_len, int32_t max_ctx_len, int32_t prefix_len,
                                int32_t num_q_tokens, int32_t mode, pa_shared_plan* plan) {
  if (!plan) return PA_ERR_INVALID_ARG;
  pa_status s = check_shared_shape(pool, num_seqs, num_q_heads, max_q_len, max_ctx_len,
                                   prefix_len, num_q_tokens);
  if (s != PA_OK) return s;
  if (mode != PA_SHARED_AUTO && mode != PA_SHARED_PACKED && mode != PA_SHARED_PLAIN)
    return PA_ERR_INVALID_ARG;
  const int32_t Hkv = pool->num_kv_heads;
  if (mode == PA_SHARED_AUTO) {
    // Packing saves the prefix reads of all but one of the q_len = 1 rows and
    // costs three more launches (prefix pass, merge, and for a mixed batch
    // the gather) plus partial traffic, about 10-15 us.  Rows with q_len > 1
    // gain nothing: their tiles meet every prefix key either way.  So pack
    // only when the prefix bytes the q_len = 1 rows would read beyond the
    // first are well above that cost (128 MiB, about 20 us at 6.5 TB/s).
    // 64 rows x 4096-token bf16 prefix (1 GiB saved): 55.2 us packed against
    // 128.9 us; 16 rows x 1024 fp8 (31 MB): 36.3 against 26.2 us.
    const int64_t n1 = most_single_rows(num_seqs, max_q_len, num_q_tokens);
    const double es = pool->kv_dtype == PA_FP8_E4M3 ? 1.0 : 2.0;
    const double saved = static_cast<double>(n1 - 1) * prefix_len * Hkv * pool->head_dim * 2.0 * es;
    mode = (n1 >= 2 && saved >= 128.0 * (1 << 20)) ? PA_SHARED_PACKED : PA_SHARED_PLAIN;
  }
  plan->mode = mode;
  if (mode == PA_SHARED_PLAIN) {
    plan->prefix_splits = plan->suffix_splits = 0;
    plan->plain_splits =
        max_q_len == 1
            ? pa_decode_num_splits(num_seqs, Hkv, max_ctx_len)
            : pa_prefill_num_splits(num_seqs, Hkv, num_q_heads, max_q_len, max_ctx_len);
  } else {
    plan->prefix_splits = pa_prefill_num_splits(1, Hkv, num_q_heads, num_seqs, prefix_len);
    plan->suffix_splits = pa_decode_num_splits(num_seqs, Hkv, max_ctx_len - prefix_len);
    plan->plain_splits =
        max_q_len == 1
            ? 1
            : pa_prefill_num_splits(num_seqs, Hkv, num_q_heads, max_q_len, max_ctx_len);
  }
  plan->workspace_bytes =
      shared_layout(*plan, num_seqs, num_q_heads, pool->head_dim, max_q_len).total;
  return PA_OK;
}

static bool plan_ok(const pa_shared_plan& p, int32_t max_q_len) {
  if (p.mode == PA_SHARED_PLAIN)
    return p.plain_splits >= 1 && p.plain_splits <= (max_q_len == 1 ? 64 : 16);
  if (p.mode != PA_SHARED_PACKED) return false;
  return p.prefix_splits >= 1 && p.prefix_splits <= 16 && p.suffix_splits >= 1 &&
         p.suffix_splits <= 64 && p.plain_splits >= 1 && p.plain_splits <= 16;
}

size_t pa_shared_prefix_workspace_bytes(const pa_kv_pool* pool, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_q_len,
                                        const pa_shared_plan* plan) {
  if (!plan || check_pool(pool) != PA_OK || num_seqs < 1 || num_q_heads < 1 || max_q_len < 1 ||
      !plan_ok(*plan, max_q_len))
    return 0;
  return shared_layout(*plan, num_seqs, num_q_heads, pool->head_dim, max_q_len).total;
}

pa_status pa_prefill_shared_prefix(const pa_kv_pool* pool, const void* q, pa_dtype q_dtype,
                                   void* o, float* lse, const int32_t* cu_q_lens,
                                   const int32_t* ctx_lens, const int32_t* block_table,
                                   int32_t bt_stride, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_q_len, int32_t max_ctx_len, float scale,
                                   int32_t causal, int32_t prefix_len, int32_t num_q_tokens,
                                   const pa_shared_plan* plan, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (num_seqs == 0 && pool) return check_pool(pool);
  pa_status s = check_attn(pool, q, q_dtype, o, ctx_lens, block_table, bt_stride, num_seqs,
                           num_q_heads, max_ctx_len, scale);
  if (s != PA_OK) return s;
  if (!cu_q_lens) return PA_ERR_INVALID_ARG;
  s = check_shared_shape(pool, num_seqs, num_q_heads, max_q_len, max_ctx_len, prefix_len,
                         num_q_tokens);
  if (s != PA_OK) return s;
  pa_shared_plan p;
  if (plan) {
    p = *plan;
    if (!plan_ok(p, max_q_len)) return PA_ERR_INVALID_ARG;
  } else {
    s = pa_shared_prefix_plan(pool, num_seqs, num_q_heads, max_q_len, max_ctx_len, prefix_len,
                              num_q_tokens, PA_SHARED_AUTO, &p);
    if (s != PA_OK) return s;
  }
  if (p.mode == PA_SHARED_PLAIN) {
    if (max_q_len == 1)
      return pa_decode(pool, q, q_dtype, o, lse, ctx_lens, block_table, bt_stride, num_seqs,
                       num_q_heads, max_ctx_len, scale, p.plain_splits, workspace,
                       workspace_bytes, stream);
    return prefill_impl(pool, q, q_dtype, o, lse, cu_q_lens, ctx_lens, block_table, bt_stride,
                        num_seqs, num_q_heads, max_q_len, max_ctx_len, scale, causal,
                        p.plain_splits, workspace, workspace_bytes, stream, false);
  }
  const SpLayout L = shared_layout(p, num_seqs, num_q_heads, pool->head_dim, max_q_len);
  if (!workspace || workspace_bytes < L.total) return PA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PA_ERR_INVALID_ARG;
  AttnArgs a = make_args(pool, q, o, lse, ctx_lens, block_table, bt_stride, num_seqs,
                         num_q_heads, max_ctx_len, scale);
  a.cu_q_lens = cu_q_lens;
  a.max_q_len = max_q_len;
  a.causal = causal ? 1 : 0;
  char* w = static_cast<char*>(workspace);
  SharedLaunch sl{};
  sl.prefix_len = prefix_len;
  sl.s_prefix = p.prefix_splits;
  sl.s_suffix = p.suffix_splits;
  sl.s_plain = max_q_len > 1 ? p.plain_splits : 1;
  sl.qd = max_q_len > 1 ? w + L.qd : nullptr;
  sl.ws_o = reinterpret_cast<float*>(w + L.o);
  sl.ws_lse = reinterpret_cast<float*>(w + L.lse);
  if (max_q_len > 1 && sl.s_plain > 1) {
    const size_t rows = static_cast<size_t>(sl.s_plain) * num_seqs * max_q_len * num_q_heads;
    sl.ws_o2 = reinterpret_cast<float*>(w + L.rest);
    sl.ws_lse2 = reinterpret_cast<float*>(w + L.rest + align256(rows * pool->head_dim * 4));
  }
  return launched(launch_prefill_shared_prefix(a, sl, static_cast<hipStream_t>(stream)));
}

size_t pa_backward_workspace_bytes(const pa_kv_pool* pool, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_q_len) {
  if (check_pool(pool) != PA_OK || num_seqs < 1 || max_q_len < 1 ||
      num_q_heads < pool->num_kv_heads || num_q_heads % pool->num_kv_heads != 0)
    return 0;
  return backward_layout(num_seqs, max_q_len, num_q_heads, pool->num_kv_heads, pool->head_dim,
                         pool->num_blocks)
      .total;
}

pa_status pa_prefill_backward(const pa_kv_pool* pool, const void* q, const void* o,
                              const float* lse, const void* dout, pa_dtype q_dtype, float* dq,
                              float* dk, float* dv, const int32_t* cu_q_lens,
                              const int32_t* ctx_lens, const int32_t* block_table,
                              int32_t bt_stride, int32_t num_seqs, int32_t num_q_heads,
                              int32_t max_q_len, int32_t max_ctx_len, float scale,
                              int32_t causal, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (num_seqs == 0 && pool) return check_pool(pool);
  pa_status s = check_attn(pool, q, q_dtype, o, ctx_lens, block_table, bt_stride, num_seqs,
                           num_q_heads, max_ctx_len, scale);
  if (s != PA_OK) return s;
  if (pool->kv_dtype != PA_BF16 || q_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (!lse || !dout || !dq || !dk || !dv || !cu_q_lens) return PA_ERR_INVALID_ARG;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return PA_ERR_INVALID_ARG;
  if (max_q_len < 1 || max_q_len > max_ctx_len) return PA_ERR_INVALID_ARG;
  const BwdLayout L = backward_layout(num_seqs, max_q_len, num_q_heads, pool->num_kv_heads,
                                      pool->head_dim, pool->num_blocks);
  // a sequence's transposed rows are addressed with 32-bit offsets
  if (static_cast<int64_t>(L.lpad) * pool->head_dim * 2 >= (int64_t{1} << 31))
    return PA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < L.total) return PA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PA_ERR_INVALID_ARG;
  BwdArgs a{};
  a.k = static_cast<const uint16_t*>(pool->k);
  a.v = static_cast<const uint16_t*>(pool->v);
  a.num_blocks = pool->num_blocks;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.q = static_cast<const uint16_t*>(q);
  a.o = static_cast<const uint16_t*>(o);
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.cu_q_lens = cu_q_lens;
  a.ctx_lens = ctx_lens;
  a.block_table = block_table;
  a.bt_stride = bt_stride;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.max_q_len = max_q_len;
  a.max_ctx_len = max_ctx_len;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  a.lpad = L.lpad;
  char* w = static_cast<char*>(workspace);
  a.qt = reinterpret_cast<uint16_t*>(w + L.off[0]);
  a.dot = reinterpret_cast<uint16_t*>(w + L.off[1]);
  a.delta = reinterpret_cast<float*>(w + L.off[2]);
  a.lse2 = reinterpret_cast<float*>(w + L.off[3]);
  a.kfm = reinterpret_cast<uint16_t*>(w + L.off[4]);
  a.vtm = reinterpret_cast<uint16_t*>(w + L.off[5]);
  return launched(launch_backward(a, static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_num_splits(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx_len) {
  if (num_seqs < 1 || num_kv_heads < 1 || max_ctx_len < 1) return 1;
  // With one workgroup per compute unit or more, splitting only adds partial
  // traffic and a merge (32 x 128..2048 tokens: 36.4 us unsplit, 42.5 us
  // with 2 splits; 32 x 2048: 50.6 / 56.0 us; 256 x 256: 62.4 / 82.6 us).
  // Below that, aim for about 512 workgroups (two per compute unit, all
  // resident) while keeping at least 8 pages (2 per wave) in every split
  // (8 x 32768 tokens: 8 splits 171 us, 16 splits 187 us, 32 splits 205 us).
  const int64_t base = static_cast<int64_t>(num_seqs) * num_kv_heads;
  if (base >= 256) return 1;
  const int32_t pages = (max_ctx_len + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE;
  int64_t s = (512 + base - 1) / base;
  int64_t max_by_pages = pages / 8;
  if (s > max_by_pages) s = max_by_pages;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return static_cast<int32_t>(s);
}

int32_t pa_decode_choose_splits(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx_len,
                                int64_t total_ctx_len) {
  if (num_seqs < 1 || num_kv_heads < 1 || max_ctx_len < 1) return 1;
  // A batch whose longest sequence is well above the mean leaves most
  // compute units idle in the split kernel (one workgroup per sequence and
  // split); the balanced kernel gives every wave the same number of pages.
  // 1 x 32768 + 31 x 256 tokens: 251.5 us with the split heuristic, 78.9 us
  // with the best split count, 52.5 us balanced; 4 x 8192 + 60 x 128: 128.4,
  // 61.0 and 44.5 us.  For even lengths the split kernel is faster (32 x
  // 1088: 30.6 us against 40.6 us; 32 x 128..2048, max/mean 1.9: 36.4 us
  // against 40.0 us).
  if (num_seqs >= 2 && total_ctx_len > 0 &&
      static_cast<double>(max_ctx_len) * num_seqs > 3.0 * static_cast<double>(total_ctx_len))
    return PA_DECODE_BALANCED;
  return pa_decode_num_splits(num_seqs, num_kv_heads, max_ctx_len);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t num_splits) {
  if (num_seqs < 1 || num_q_heads < 1 || head_dim < 1 || num_splits <= 1) return 0;
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * num_splits;
  size_t o_bytes = rows * head_dim * sizeof(float);
  o_bytes = (o_bytes + 255) & ~static_cast<size_t>(255);
  return o_bytes + rows * sizeof(float);
}

size_t pa_decode_balanced_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t max_ctx_len) {
  if (num_seqs < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 || max_ctx_len < 1)
    return 0;
  return balanced_ws_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_ctx_len, 0);
}

pa_status pa_decode(const pa_kv_pool* pool, const void* q, pa_dtype q_dtype, void* o,
                    float* lse, const int32_t* ctx_lens, const int32_t* block_table,
                    int32_t bt_stride, int32_t num_seqs, int32_t num_q_heads,
                    int32_t max_ctx_len, float scale, int32_t num_splits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (num_seqs == 0 && pool) return check_pool(pool);
  pa_status s = check_attn(pool, q, q_dtype, o, ctx_lens, block_table, bt_stride, num_seqs,
                           num_q_heads, max_ctx_len, scale);
  if (s != PA_OK) return s;
  if (num_splits < PA_DECODE_BALANCED || num_splits > 256) return PA_ERR_INVALID_ARG;
  if (num_splits == 0) num_splits = pa_decode_num_splits(num_seqs, pool->num_kv_heads, max_ctx_len);
  AttnArgs a = make_args(pool, q, o, lse, ctx_lens, block_table, bt_stride, num_seqs,
                         num_q_heads, max_ctx_len, scale);
  a.num_splits = num_splits;
  if (num_splits == PA_DECODE_BALANCED) {
    if (pool->kv_dtype == PA_F32) return PA_ERR_UNSUPPORTED;
    const size_t need = balanced_ws_bytes(num_seqs, num_q_heads, pool->num_kv_heads,
                                          pool->head_dim, max_ctx_len, 0);
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_INVALID_ARG;
    const int64_t U = 4 * static_cast<int64_t>(
                              balanced_wgs(num_seqs, pool->num_kv_heads, max_ctx_len, 0));
    const size_t prow = static_cast<size_t>(num_q_heads) * (U + num_seqs);
    const size_t o_bytes = (prow * pool->head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
    a.ws_o = static_cast<float*>(workspace);
    a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
    return launched(launch_decode(a, static_cast<hipStream_t>(stream)));
  }
  if (num_splits > 1) {
    size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, pool->head_dim, num_splits);
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_INVALID_ARG;
    size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * num_splits;
    size_t o_bytes = (rows * pool->head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
    a.ws_o = static_cast<float*>(workspace);
    a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  }
  return launched(launch_decode(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ----------------------------------------------------------- decode without allocation
// pa_decode_noalloc keeps the split partials in this fixed device array instead
// of a caller's workspace.  Each GPU the library runs on holds its own copy
// (PA_SCRATCH_BYTES) until the process ends.  In host code `scratch` names a
// host-side stand-in, not the device array: its device address is looked up
// once per device with hipGetSymbolAddress and only that address is used.
static __device__ __align__(256) unsigned char scratch[PA_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (looked up on its first use).
pa_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
        return PA_ERR_LAUNCH;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_noalloc(const pa_kv_pool* pool, const void* q, pa_dtype q_dtype, void* o,
                            float* lse, const int32_t* ctx_lens, const int32_t* block_table,
                            int32_t bt_stride, int32_t num_seqs, int32_t num_q_heads,
                            int32_t max_ctx_len, float scale, int32_t num_splits, void* stream) {
  if (num_seqs == 0 && pool) return check_pool(pool);
  pa_status s = check_attn(pool, q, q_dtype, o, ctx_lens, block_table, bt_stride, num_seqs,
                           num_q_heads, max_ctx_len, scale);
  if (s != PA_OK) return s;
  if (num_splits < PA_DECODE_BALANCED || num_splits > 256) return PA_ERR_INVALID_ARG;
  if (num_splits == 0) num_splits = pa_decode_num_splits(num_seqs, pool->num_kv_heads, max_ctx_len);
  const size_t need =
      num_splits == PA_DECODE_BALANCED
          ? balanced_ws_bytes(num_seqs, num_q_heads, pool->num_kv_heads, pool->head_dim,
                              max_ctx_len, 0)
          : pa_decode_workspace_bytes(num_seqs, num_q_heads, pool->head_dim, num_splits);
  if (need > PA_SCRATCH_BYTES) return PA_ERR_WORKSPACE;  // beyond the fixed array
  void* ws = nullptr;
  if (need > 0) {
    s = device_scratch(&ws);
    if (s != PA_OK) return s;
  }
  return pa_decode(pool, q, q_dtype, o, lse, ctx_lens, block_table, bt_stride, num_seqs,
                   num_q_heads, max_ctx_len, scale, num_splits, ws, need, stream);
}

}  // extern "C"
