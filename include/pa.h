/*
 * pa.h -- paged attention for MI355X (gfx950): C ABI (the forward pass, its
 *         backward, the paged KV cache and its block allocator, measurement probes).
 *
 * Exact scaled-dot-product attention, softmax(scale * Q K^T) V, computed with
 * K/V tiles streamed from a paged KV cache and an online softmax (running max,
 * running sum, rescaled accumulator; the logsumexp is written out).
 *
 * Sources of the operations (web pages on FlashAttention and PagedAttention):
 *  - the attention itself: the FlashAttention/PagedAttention survey page
 *    ("FlashAttention与PagedAttention技术详解"), section 1, scaled dot-product
 *    self-attention with d_k the head dimension;
 *  - tiling, safe softmax and the kept statistics (max and logsumexp): the same
 *    page, section 2, "core principle"; FlashAttention-2 keeps only logsumexp
 *    (section 2, FlashAttention-2 improvements);
 *  - the paged KV cache: fixed 16-token physical blocks, a per-sequence block
 *    table mapping logical to physical blocks, blocks allocated on demand and
 *    freed when a request ends, and reference-counted sharing of a common
 *    prompt's blocks: the same page, section 3, "core principle", and the
 *    "core modules" chapter page, section 2.2 (its pseudocode loops over a
 *    sequence's logical blocks, looks up the physical block and merges each
 *    block's scores into running statistics).
 *
 * Conventions common to every entry point:
 *  - Device pointers are plain device addresses (e.g. from hipMalloc or a torch
 *    CUDA tensor's data_ptr()); the caller owns every buffer.  The library never
 *    allocates, frees or synchronises device memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued on it; calls return before the work is done.
 *  - Arguments that live on the host are checked before anything is enqueued;
 *    a failed check returns a negative pa_status and enqueues nothing.  A launch
 *    failure returns PA_ERR_LAUNCH.  No C++ exception crosses this boundary.
 *  - Metadata that lives on the device (lengths, block tables, slot mappings)
 *    is not read by the host.  The caller guarantees: 1 <= q_len_b <= ctx_len_b
 *    <= max_ctx_len, q_len_b <= max_q_len, and block_table[b][j] in
 *    [0, num_blocks) for every j < ceil(ctx_len_b / 16).  Entries past that,
 *    up to ceil(max_ctx_len / 16), may be read but their values are never used;
 *    so bt_stride >= ceil(max_ctx_len / 16) (checked).  A block id outside
 *    [0, num_blocks) is never dereferenced (the page is treated as empty), but
 *    the result is then unspecified.
 *  - Calls are reentrant; the library keeps no mutable global state (except
 *    pa_decode_noalloc's fixed device array, see there).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad alignment          */
  PA_ERR_UNSUPPORTED = -2, /* valid but not built: dtype / head_dim / group  */
  PA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required     */
  PA_ERR_OOM = -4,         /* host block allocator has no free block         */
  PA_ERR_LAUNCH = -5       /* a HIP launch or runtime call failed            */
} pa_status;

typedef enum {
  PA_F32 = 0,      /* IEEE binary32                                          */
  PA_BF16 = 1,     /* bfloat16                                               */
  PA_FP8_E4M3 = 2  /* OCP E4M3FN: bias 7, max +-448, NaN = S.1111.111; pool only */
} pa_dtype;

/*
 * The KV block pool (caller-owned device memory).
 *   k: [num_blocks, num_kv_heads, 16, head_dim]  token-major inside a page
 *   v: [num_blocks, num_kv_heads, head_dim, 16]  feature-major inside a page
 * Each (physical block, KV head) is one contiguous chunk of 16 * head_dim
 * elements (4 KiB for bf16 and head_dim 128).  Keeping V feature-major inside
 * the page lets the P.V product read its operand as 16-byte runs of keys.
 * For PA_FP8_E4M3 pools, k_scale/v_scale hold one float per physical block,
 * shared by all KV heads: stored value = code * scale.  Otherwise they are
 * ignored (may be NULL).  k and v must be 16-byte aligned.
 */
typedef struct {
  void* k;
  void* v;
  float* k_scale;
  float* v_scale;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;    /* 64 or 128 */
  int32_t block_size;  /* must be 16 */
  pa_dtype kv_dtype;
} pa_kv_pool;

/* Static text for a status code. */
const char* pa_status_string(pa_status s);

/* Version of this ABI (incremented on any signature or layout change). */
int32_t pa_abi_version(void);

/* ------------------------------------------------------------------ write
 * Scatter num_tokens new tokens into the pool (on-demand block use, as the
 * survey page's section 3 describes for newly generated tokens).
 *   k_new, v_new : [num_tokens, num_kv_heads, head_dim] in src_dtype (device)
 *   slot_mapping : int32 [num_tokens] (device); token t goes to physical block
 *                  slot_mapping[t] / 16, offset slot_mapping[t] % 16
 * Pool f32 <- src f32, pool bf16 <- src bf16: exact copy.
 * Pool fp8 <- src f32 or bf16: every block touched by this call gets one K and
 *   one V scale, s = amax / 448 (float32, correctly rounded; s = 1 when amax is
 *   0) where amax is the largest |value| this call writes into that block (all
 *   heads, dims, tokens), and each value becomes the nearest-even E4M3 code of
 *   clamp(x / s, -448, 448).  So a block must be written whole by one call;
 *   earlier codes of a block touched again are not re-quantised (use
 *   pa_append_kv for that).
 * workspace: device memory of pa_write_kv_workspace_bytes(pool) bytes
 *   (0 for non-fp8 pools; may then be NULL).  Slots must be distinct.
 */
size_t pa_write_kv_workspace_bytes(const pa_kv_pool* pool);
pa_status pa_write_kv(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                      pa_dtype src_dtype, const int32_t* slot_mapping, int32_t num_tokens,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ append
 * Like pa_write_kv, for tokens appended to sequences whose last page may be
 * partly filled (one new token per sequence per decode step, as the survey
 * page's section 3 describes: new tokens go to the sequence's current block,
 * and a new block is taken when it is full).  In every page this call writes,
 * the offsets below the lowest offset it writes are the page's existing
 * tokens and are kept; the call must write a page's new tokens as a run of
 * offsets from that lowest one.
 * Pool f32 / bf16: identical to pa_write_kv.
 * Pool fp8: each touched page gets a new K and V scale s' = amax' / 448 (1 when
 *   amax' is 0), where amax' is the largest |value| among the page's existing
 *   tokens as stored (code * old scale, float32) and the new tokens (all
 *   heads); the existing codes are re-encoded as the nearest-even E4M3 code of
 *   clamp(code * old scale / s'), then the new tokens are encoded with s'.
 * Same arguments, workspace and errors as pa_write_kv.
 */
pa_status pa_append_kv(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                       pa_dtype src_dtype, const int32_t* slot_mapping, int32_t num_tokens,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ copy
 * Copy whole physical blocks: block dst_blocks[i] becomes a bit-exact copy of
 * block src_blocks[i] (K and V of every KV head, and the fp8 scales).  The
 * copy a sequence needs before writing into a block it shares with others
 * (copy on write; see pa_plan_append).  src_blocks, dst_blocks: int32
 * [num_pairs] (device).  Destinations must be distinct and must not be
 * sources of the same call.  Ids outside [0, num_blocks) are skipped.
 */
pa_status pa_copy_blocks(const pa_kv_pool* pool, const int32_t* src_blocks,
                         const int32_t* dst_blocks, int32_t num_pairs, void* stream);

/* ------------------------------------------------------------------ gather
 * Copy each sequence's logical tokens out of the pool, through its block
 * table, into contiguous token-major buffers (bit-exact copy of the stored
 * bytes; fp8 codes are copied without scaling).  This is the lookup step of
 * the paged loop in the "core modules" chapter page, section 2.2 (logical
 * block j of a sequence -> physical block block_table[j] -> its K and V), and
 * of the block-table mapping in the survey page, section 3, "core
 * principle", done on its own.  Used to check the pool and block-table
 * addressing and as a bandwidth probe.
 *   block_table : int32 [num_seqs, bt_stride] (device)
 *   ctx_lens    : int32 [num_seqs] (device)
 *   cu_ctx      : int32 [num_seqs + 1] (device), prefix sums of ctx_lens
 *   k_out, v_out: [cu_ctx[num_seqs], num_kv_heads, head_dim] pool dtype (device)
 * max_ctx_len bounds every ctx_lens entry.
 */
pa_status pa_gather_kv(const pa_kv_pool* pool, const int32_t* block_table, int32_t bt_stride,
                       const int32_t* ctx_lens, const int32_t* cu_ctx, int32_t num_seqs,
                       int32_t max_ctx_len, void* k_out, void* v_out, void* stream);

/* ------------------------------------------------------------------ prefill
 * Causal (or full) attention of a batch of query chunks against the paged
 * cache: softmax(scale Q K^T) V (survey page, section 1) computed tile by tile
 * with a running max, a running exp-sum and a rescaled accumulator, only the
 * logsumexp kept (survey page, section 2, "core principle" and
 * FlashAttention-2 improvements; "core modules" chapter, section 2.1), the
 * K/V tiles found page by page through the block table (the paged loop of
 * the "core modules" chapter, section 2.2).  Sequence b has q_len_b = cu_q_lens[b+1] - cu_q_lens[b] query tokens
 * that are the LAST q_len_b of its ctx_len_b cached tokens (their K/V must
 * already be in the pool): query i of sequence b sits at position
 * ctx_len_b - q_len_b + i and, when causal, sees keys 0..that position.
 *   q   : [cu_q_lens[num_seqs], num_q_heads, head_dim], q_dtype (device)
 *   o   : same shape, q_dtype (device, written)
 *   lse : float [cu_q_lens[num_seqs], num_q_heads] natural-log logsumexp of the
 *         scaled scores of each row (device, written; may be NULL)
 *   cu_q_lens : int32 [num_seqs + 1]; ctx_lens : int32 [num_seqs] (device)
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).  scale must be
 * finite and > 0 (usually 1/sqrt(head_dim)).
 * Supported: q_dtype PA_F32 with an f32 pool; q_dtype PA_BF16 with a bf16 or
 * fp8 pool.  head_dim 64 or 128; num_q_heads / num_kv_heads in {1,2,4,8,16}.
 * q and o must be 16-byte aligned.  A sequence with q_len_b = 1 is a decode
 * row, so one call can serve a mixed batch of chunked prefills and decodes.
 * A row that sees no key (only possible when the device-resident contract is
 * broken: ctx_len_b = 0 or q_len_b > ctx_len_b) gets O = 0 and LSE = -inf.
 * Key splits: each query tile's visible keys can be cut into num_splits
 * contiguous ranges of 32-key tiles; each range gives a normalised partial
 * output and logsumexp in the workspace, and a second pass merges them by
 * their logsumexps (as pa_decode does).  num_splits: 0 = choose with
 * pa_prefill_num_splits(), 1 = none (no workspace needed), at most 16; fp32
 * pools always run with one.  workspace: device memory of at least
 * pa_prefill_workspace_bytes(num_seqs, max_q_len, num_q_heads, head_dim,
 * splits) bytes, 16-byte aligned, contents need not be initialised.
 */
int32_t pa_prefill_num_splits(int32_t num_seqs, int32_t num_kv_heads, int32_t num_q_heads,
                              int32_t max_q_len, int32_t max_ctx_len);
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads,
                                  int32_t head_dim, int32_t num_splits);
pa_status pa_prefill(const pa_kv_pool* pool, const void* q, pa_dtype q_dtype, void* o,
                     float* lse, const int32_t* cu_q_lens, const int32_t* ctx_lens,
                     const int32_t* block_table, int32_t bt_stride, int32_t num_seqs,
                     int32_t num_q_heads, int32_t max_q_len, int32_t max_ctx_len,
                     float scale, int32_t causal, int32_t num_splits, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ fp8 products
 * pa_prefill for an fp8 pool with both products on the fp8 matrix cores
 * (FlashAttention-3's low-precision forward: the survey page, FlashAttention-3
 * section), the cache's per-page scales kept exact:
 *   - each query row x gets one scale s = amax/448 and is split into two E4M3
 *     parts, hi = E4M3(x/s) and lo = E4M3(16 (x/s - hi)), so Q enters the
 *     scores to about 2^-8 relative;
 *   - S = Q . K codes * K page scale, in fp32;
 *   - the online softmax runs in fp32; each weight (<= 4 under a lazy
 *     rescale) times 112 times its key's V page scale over the largest V
 *     page scale of the workgroup's keys is rounded to E4M3 and multiplied
 *     with the V codes;
 *   - O is divided by the sum of those rounded weights, LSE uses the sum of
 *     the unrounded ones.
 * So every weight carries E4M3 rounding (relative 2^-4) on top of the pool's,
 * and O is the weighted mean of V under weights each within 2^-4 of exact:
 * per element |dO| <= (1/15) * the spread of the row's visible V values in
 * that feature, plus terms below 1e-2.  The error averages down with the keys
 * a row sees: on the library's tests rows that see 16 keys or more, and every
 * LSE, stay within the fp8-KV bound of 6e-2; rows that see fewer may not
 * (pa_prefill keeps them at the pool's own precision).
 * Arguments, layouts, key splits, workspace and errors as pa_prefill, except:
 * the pool must be PA_FP8_E4M3 (else PA_ERR_UNSUPPORTED), q bf16.
 */
pa_status pa_prefill_fp8(const pa_kv_pool* pool, const void* q, pa_dtype q_dtype, void* o,
                         float* lse, const int32_t* cu_q_lens, const int32_t* ctx_lens,
                         const int32_t* block_table, int32_t bt_stride, int32_t num_seqs,
                         int32_t num_q_heads, int32_t max_q_len, int32_t max_ctx_len,
                         float scale, int32_t causal, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ backward
 * Gradients of pa_prefill's attention for an upstream gradient dout, from the
 * forward's output o and logsumexp lse: the attention weights are recomputed
 * tile by tile instead of stored (the FlashAttention page, core-principle
 * section: the backward rebuilds them from the kept statistics).  With
 * P = softmax(scale Q K^T) (masked as the forward masks it):
 *   dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * O)),
 *   dQ = scale dS K,  dK = scale dS^T Q,
 * dK and dV summed over the G query heads of each KV head.
 *   q, o, dout : [cu_q_lens[num_seqs], num_q_heads, head_dim] bf16 (device)
 *   lse        : float [cu_q_lens[num_seqs], num_q_heads], as pa_prefill wrote it
 *   dq         : float [cu_q_lens[num_seqs], num_q_heads, head_dim] (written)
 *   dk         : float, the K pool's shape [num_blocks, num_kv_heads, 16, head_dim]
 *   dv         : float, the V pool's shape [num_blocks, num_kv_heads, head_dim, 16]
 * Every slot of every page a sequence uses is written (slots at or past its
 * context length with 0); other pages are not touched.  Other arguments as
 * pa_prefill.  Supported: bf16 pools with bf16 q, head_dim 64 or 128, and
 * max_q_len * (num_q_heads / num_kv_heads) * head_dim < 2^30.
 * Device-resident contract (not checked): no physical page is used by two
 * sequences (their gradients would race) or twice by one.
 * workspace: pa_backward_workspace_bytes(pool, num_seqs, num_q_heads,
 *   max_q_len) bytes of device memory, 16-byte aligned, contents need not be
 *   initialised (transposed copies of Q, dO and the used pages, rowsum(dO*O)
 *   and lse per query row).  dout, dq, dk, dv 16-byte aligned.
 */
size_t pa_backward_workspace_bytes(const pa_kv_pool* pool, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_q_len);
pa_status pa_prefill_backward(const pa_kv_pool* pool, const void* q, const void* o,
                              const float* lse, const void* dout, pa_dtype q_dtype, float* dq,
                              float* dk, float* dv, const int32_t* cu_q_lens,
                              const int32_t* ctx_lens, const int32_t* block_table,
                              int32_t bt_stride, int32_t num_seqs, int32_t num_q_heads,
                              int32_t max_q_len, int32_t max_ctx_len, float scale,
                              int32_t causal, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ------------------------------------------------------------ shared prefix
 * pa_prefill for a batch whose sequences all begin with the same prefix_len
 * tokens held in the same physical blocks (reference-counted sharing of a
 * common prompt's blocks: the survey page, section 3, "core principle"; the
 * saving it brings: same page, section 3, "performance advantages").  The
 * result is the same attention as pa_prefill with the same arguments; only
 * the work is arranged differently.  Two arrangements (pa_shared_plan.mode):
 *
 * PA_SHARED_PACKED, for the rows with q_len_b = 1 (decode rows):
 *   1. those rows of all sequences, packed into one virtual sequence (row b =
 *      sequence b's query), attend the prefix keys 0..prefix_len-1 once per
 *      KV head (no mask: every query lies past the prefix), read through
 *      block-table row 0, so the prefix is multiplied in a matrix tile for all
 *      of them together instead of streamed once per sequence;
 *   2. each such row attends its own keys prefix_len..ctx_len_b-1 (pa_decode's
 *      split pass over the pages past the prefix);
 *   3. the normalised partials of both passes are merged by their logsumexps
 *      (the combination of partial softmax statistics of the "core modules"
 *      chapter, section 2.1).
 *   Rows with q_len_b > 1 gain nothing from packing (each of their query
 *   tiles meets every prefix key either way): they take pa_prefill's pass
 *   over all their keys, before the packed passes.
 * PA_SHARED_PLAIN: the whole batch as pa_decode (max_q_len = 1) or pa_prefill
 *   would run it.
 * PA_SHARED_AUTO (to pa_shared_prefix_plan only) packs when the prefix bytes
 * that all but one of the q_len = 1 rows would read (bounded from the shapes:
 * with max_q_len > 1, at most (num_seqs * max_q_len - num_q_tokens) /
 * (max_q_len - 1) rows can have q_len = 1) reach 128 MiB, and otherwise runs
 * plain, so that packing is taken only where it pays.
 *
 * Arguments as pa_prefill, plus:
 *   prefix_len   : a multiple of 16, >= 16, and prefix_len + max_q_len <=
 *                  max_ctx_len (checked).
 *   num_q_tokens : cu_q_lens[num_seqs], the rows of q and o; 1 <= num_q_tokens
 *                  <= num_seqs * max_q_len (checked).  When max_q_len is 1
 *                  every sequence has exactly one query (q_len_b >= 1 as for
 *                  every call), so num_q_tokens must equal num_seqs (checked).
 *   plan         : from pa_shared_prefix_plan, whose split counts the caller
 *                  may change within their bounds (checked: packed 1..16
 *                  prefix splits, 1..64 own-key splits, 1..16 splits of the
 *                  q_len > 1 rows' pass; plain 1..64 for max_q_len = 1, else
 *                  1..16), or NULL for the PA_SHARED_AUTO plan.
 *   workspace    : at least pa_shared_prefix_workspace_bytes(pool, num_seqs,
 *                  num_q_heads, max_q_len, plan) bytes of device memory,
 *                  16-byte aligned (none needed when that is 0).
 * Device-resident contract (not checked): for every b, block_table[b][j] ==
 * block_table[0][j] for j < prefix_len / 16, and ctx_len_b - q_len_b >=
 * prefix_len (no query inside the prefix).  If it does not hold the result is
 * unspecified, but nothing outside the documented buffers is touched.
 * Supported: bf16 and fp8 pools (PA_ERR_UNSUPPORTED for fp32 pools).
 */
#define PA_SHARED_AUTO 0
#define PA_SHARED_PACKED 1
#define PA_SHARED_PLAIN 2

typedef struct pa_shared_plan {
  int32_t mode;            /* PA_SHARED_PACKED or PA_SHARED_PLAIN */
  int32_t prefix_splits;   /* packed: key splits of the packed prefix pass */
  int32_t suffix_splits;   /* packed: key splits of the q_len = 1 rows' own keys */
  int32_t plain_splits;    /* key splits of pa_prefill's / pa_decode's pass */
  size_t workspace_bytes;  /* filled by pa_shared_prefix_plan */
} pa_shared_plan;

/* Fill *plan for the given shapes: the arrangement (mode PA_SHARED_AUTO
 * chooses as above; PACKED and PLAIN force one), its split counts and its
 * workspace size.  PA_ERR_INVALID_ARG for shapes pa_prefill_shared_prefix
 * would refuse, PA_ERR_UNSUPPORTED for fp32 pools. */
pa_status pa_shared_prefix_plan(const pa_kv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                int32_t max_q_len, int32_t max_ctx_len, int32_t prefix_len,
                                int32_t num_q_tokens, int32_t mode, pa_shared_plan* plan);
/* Workspace bytes for a (possibly edited) plan; 0 for an invalid plan or
 * when none is needed. */
size_t pa_shared_prefix_workspace_bytes(const pa_kv_pool* pool, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_q_len,
                                        const pa_shared_plan* plan);
pa_status pa_prefill_shared_prefix(const pa_kv_pool* pool, const void* q, pa_dtype q_dtype,
                                   void* o, float* lse, const int32_t* cu_q_lens,
                                   const int32_t* ctx_lens, const int32_t* block_table,
                                   int32_t bt_stride, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_q_len, int32_t max_ctx_len, float scale,
                                   int32_t causal, int32_t prefix_len, int32_t num_q_tokens,
                                   const pa_shared_plan* plan, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ decode
 * One query token per sequence, at position ctx_len_b - 1 (it sees all
 * ctx_len_b cached keys).  Split-KV: each sequence's pages are cut into
 * num_splits contiguous page ranges; one pass computes, per (sequence, KV head,
 * range), the normalised partial output and logsumexp of all the group's query
 * heads into the workspace, and a second pass merges the ranges by their
 * logsumexps:  lse = M + ln sum_s exp(lse_s - M),  o = sum_s exp(lse_s - lse) o_s.
 * (The merge is the same combination of partial softmax statistics that the
 * online softmax applies block by block, "core modules" chapter, section 2.1.)
 *   q   : [num_seqs, num_q_heads, head_dim], q_dtype (device)
 *   o   : same shape and dtype (device, written)
 *   lse : float [num_seqs, num_q_heads] (device, written; may be NULL)
 * num_splits: 0 = choose with pa_decode_num_splits(); 1 = no merge pass, no
 *   workspace needed; at most 256.  workspace: device memory of at least
 *   pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, splits) bytes,
 *   16-byte aligned, contents need not be initialised.  Same dtype and group
 *   support as pa_prefill.
 * num_splits = PA_DECODE_BALANCED (bf16 and fp8 pools): the pages of all
 *   sequences of a KV head, taken in sequence order, are cut into equal
 *   chunks, one per wave, whatever the mix of lengths; a sequence inside one
 *   chunk is finished there, the others are merged from one partial per chunk
 *   they meet (same merge as above).  For batches whose longest sequence is
 *   far above the mean.  workspace: pa_decode_balanced_workspace_bytes(...)
 *   bytes, 16-byte aligned, contents need not be initialised.
 * pa_decode_choose_splits: the library's choice given the batch's total
 *   context length (sum of ctx_len_b; 0 = unknown): PA_DECODE_BALANCED when
 *   the longest sequence is over 3 times the mean, else pa_decode_num_splits.
 */
#define PA_DECODE_BALANCED (-1)
/* Workspace of pa_decode with num_splits > 1: one normalised fp32 partial
 * output row of head_dim floats and one fp32 logsumexp per (sequence, query
 * head, split), the state each split keeps before the merge (the partial
 * softmax statistics of the "core modules" chapter, section 2.1; the survey
 * page, section 2, "core principle", keeps the same max/sum pair per block).
 * Independent of the context lengths; 0 when num_splits <= 1. */
size_t pa_decode_balanced_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t max_ctx_len);
int32_t pa_decode_num_splits(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx_len);
int32_t pa_decode_choose_splits(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx_len,
                                int64_t total_ctx_len);
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t num_splits);
pa_status pa_decode(const pa_kv_pool* pool, const void* q, pa_dtype q_dtype, void* o,
                    float* lse, const int32_t* ctx_lens, const int32_t* block_table,
                    int32_t bt_stride, int32_t num_seqs, int32_t num_q_heads,
                    int32_t max_ctx_len, float scale, int32_t num_splits, void* workspace,
                    size_t workspace_bytes, void* stream);

/* ------------------------------------------------ decode without allocation
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same computation, kernels and results as pa_decode with the
 * same num_splits (bit for bit), but the split partials go to a fixed device
 * array of PA_SCRATCH_BYTES inside the library instead of a workspace.  Calls
 * no hipMalloc, hipFree or other allocating routine.
 *   - Each GPU the library runs on holds its own copy of the array until the
 *     process ends; its address is looked up on the first call on that GPU.
 *     The current device (hipGetDevice) must be the one `stream` and all
 *     buffers belong to.
 *   - Every call on one GPU shares that GPU's array: calls that may overlap
 *     on one GPU (different streams, other threads) race and must not be
 *     issued.  Stream-ordered calls on one stream are fine.
 *   - The array keeps the last call's partials; no call needs it cleared.
 * Arguments as pa_decode without the workspace.  Errors as pa_decode, plus
 * PA_ERR_WORKSPACE (before anything is enqueued) when the partials of the
 * chosen split count would need more than PA_SCRATCH_BYTES
 * (pa_decode_workspace_bytes, or pa_decode_balanced_workspace_bytes for
 * PA_DECODE_BALANCED).  Breaks the "no mutable global state" convention above
 * only through that array.
 */
#define PA_SCRATCH_BYTES (8u << 20)
pa_status pa_decode_noalloc(const pa_kv_pool* pool, const void* q, pa_dtype q_dtype, void* o,
                            float* lse, const int32_t* ctx_lens, const int32_t* block_table,
                            int32_t bt_stride, int32_t num_seqs, int32_t num_q_heads,
                            int32_t max_ctx_len, float scale, int32_t num_splits, void* stream);

/* ------------------------------------------------------------------ blocks
 * Host-side block allocator for a pool of num_blocks physical blocks: a free
 * list plus one reference count per block (survey page section 3: on-demand
 * allocation, freeing at request end, reference counts for blocks shared by
 * sequences with a common prompt).  Not thread-safe; one allocator per pool.
 *   pa_alloc_block      : a free block with refcount 1, or -1 when none is free
 *                         (lowest free id first, so allocation is deterministic)
 *   pa_block_incref     : one more owner of an allocated block (sharing)
 *   pa_block_decref     : one owner fewer; the block is free again at 0.
 *                         PA_ERR_INVALID_ARG on a free block (double free) or a
 *                         bad id.
 *   pa_block_refcount   : current count (0 = free), -1 for a bad id
 *   pa_num_free_blocks  : number of free blocks
 */
typedef struct pa_allocator pa_allocator;
pa_allocator* pa_allocator_create(int32_t num_blocks);  /* NULL if num_blocks < 1 */
void pa_allocator_destroy(pa_allocator* a);
int32_t pa_alloc_block(pa_allocator* a);
pa_status pa_block_incref(pa_allocator* a, int32_t block);
pa_status pa_block_decref(pa_allocator* a, int32_t block);
int32_t pa_block_refcount(const pa_allocator* a, int32_t block);
int32_t pa_num_free_blocks(const pa_allocator* a);

/*
 * Plan appending num_new[b] tokens to each sequence b (host memory throughout;
 * survey page section 3: blocks on demand, copy of a shared block before a
 * sequence writes into it).  Position p = ctx_lens[b] + i of sequence b goes to
 * page p / 16, offset p % 16.  A position that starts a page takes a fresh
 * block (lowest free id).  When the partly filled last page of a sequence is
 * shared (refcount > 1), the sequence first gets a fresh block: the pair
 * (shared, fresh) is written to copy_src / copy_dst (copy it with
 * pa_copy_blocks before appending) and the shared block loses one reference.
 * On success block_table rows and ctx_lens are updated in place,
 * slot_mapping[sum of num_new] holds the slots in sequence order (the order of
 * the rows of k_new / v_new for pa_append_kv), and *num_copies the pairs
 * written.  Checks come first: PA_ERR_INVALID_ARG (bad length, table too
 * narrow, last page not allocated, more copies than max_copies),
 * PA_ERR_OOM (not enough free blocks); on any error nothing is changed.
 */
pa_status pa_plan_append(pa_allocator* a, int32_t* block_table, int32_t bt_stride,
                         int32_t* ctx_lens, const int32_t* num_new, int32_t num_seqs,
                         int32_t* slot_mapping, int32_t* copy_src, int32_t* copy_dst,
                         int32_t max_copies, int32_t* num_copies);

/* ------------------------------------------------------------ measurement probes
 * Not part of the attention path.  Kernels that measure what this GPU
 * sustains, so that each attention kernel's rate can be read against a
 * measured ceiling as well as the spec peak (bench.py runs these beside the
 * attention kernels).
 *
 * pa_probe_stream_read: every 16-byte word of buf (device memory, bytes a
 *   multiple of 16) is read once with non-temporal loads by `blocks`
 *   workgroups of 256 threads in a grid-stride loop; out (device,
 *   blocks * 256 uint32) receives one XOR per thread of the words it read.
 * pa_probe_page_stream: the bf16 d = 128 decode's read pattern with no
 *   arithmetic.  buf is cut into `blocks` equal runs of 8 KiB pages (bytes a
 *   multiple of blocks * 8192); workgroup i (4 waves) reads run i, each wave
 *   every fourth page with two pages in flight, a page as a 4 KiB K page
 *   (16 keys x 64-byte pieces per 16-byte-per-lane load) then a 4 KiB V page
 *   (8 bytes per lane), the decode kernel's loads.  out (device, blocks * 256
 *   uint32) receives one XOR per thread.  The time for a volume with the work
 *   evenly spread: the floor of that pattern, below which a decode that
 *   streams its pages this way cannot go.
 * pa_probe_mfma: `blocks` workgroups of 4 waves; each wave runs 4 independent
 *   chains of `iters` MFMAs on register operands.  PA_BF16 uses
 *   v_mfma_f32_32x32x16_bf16 (32768 FLOP each), PA_FP8_E4M3
 *   v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales (131072 FLOP
 *   each); out (device, blocks * 256 float) receives each thread's sum of its
 *   accumulators.  FLOP per call: blocks * 16 * iters * the instruction's.
 * Errors: PA_ERR_INVALID_ARG for null pointers, bytes 0 or not a multiple of
 * 16 (of blocks * 8192 for the page stream), blocks outside [1, 65535],
 * iters < 1; PA_ERR_UNSUPPORTED for another
 * dtype; PA_ERR_LAUNCH when the launch fails.  Stream-ordered on `stream`.
 */
pa_status pa_probe_stream_read(const void* buf, size_t bytes, uint32_t* out, int32_t blocks,
                               void* stream);
pa_status pa_probe_page_stream(const void* buf, size_t bytes, uint32_t* out, int32_t blocks,
                               void* stream);
pa_status pa_probe_mfma(pa_dtype dtype, float* out, int32_t blocks, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
