// Internal declarations shared by the HIP sources of libpa (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kPage = 16;          // tokens per physical block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 packed in one dword (low = a), round to nearest even
// (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16_bits(float a) {
  return static_cast<uint16_t>(pack_bf16x2(a, 0.f));
}

// Four fp8 codes in a dword -> four bf16 packed in two dwords (exact: every
// E4M3 value is a bfloat16 value).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  float f0 = __builtin_amdgcn_cvt_f32_fp8(w, 0);
  float f1 = __builtin_amdgcn_cvt_f32_fp8(w, 1);
  float f2 = __builtin_amdgcn_cvt_f32_fp8(w, 2);
  float f3 = __builtin_amdgcn_cvt_f32_fp8(w, 3);
  u32x2 r;
  r.x = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
  r.y = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xffff0000u);
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resources.  A buffer load whose byte offset is at or past
// num_records returns zero without touching memory, so a descriptor with
// num_records = 0 makes a "dummy" load that can stay unconditional.
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit data format
constexpr int kLoadNT = 2;              // non-temporal (streaming) cache policy
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           kRsrcWord3);
}

// Symmetric pairwise combine of lane l with lane l ^ 32 / l ^ 16 through
// v_permlane32_swap / v_permlane16_swap (no LDS round trip): with both
// operands equal to x, the two results hold x[l] and x[l ^ k] in some order.
__device__ __forceinline__ float max_xor32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// the same with IEEE maximum (NaN-propagating; no operand canonicalisation)
__device__ __forceinline__ float maxm_xor32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ----------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already checked.
hipError_t launch_write_kv(const pa_kv_pool& pool, const void* k_new, const void* v_new,
                           pa_dtype src, const int32_t* slots, int32_t n, uint32_t* amax_ws,
                           bool append, hipStream_t st);
hipError_t launch_copy_blocks(const pa_kv_pool& pool, const int32_t* src, const int32_t* dst,
                              int32_t n, hipStream_t st);
hipError_t launch_gather_kv(const pa_kv_pool& pool, const int32_t* bt, int32_t bt_stride,
                            const int32_t* ctx, const int32_t* cu_ctx, int32_t B,
                            int32_t max_ctx, void* k_out, void* v_out, hipStream_t st);

struct AttnArgs {
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;
  pa_dtype kv_dtype;
  const void* q;
  void* o;
  float* lse;
  const int32_t* cu_q_lens;   // prefill only
  const int32_t* ctx_lens;
  const int32_t* block_table;
  int32_t bt_stride;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t max_q_len;
  int32_t max_ctx_len;
  float scale;
  int32_t causal;
  int32_t num_splits;          // key splits of this launch (blockIdx.y carries them)
  float* ws_o;                 // decode: [B, Hq, S, D] partial outputs; prefill: see below
  float* ws_lse;               // decode: [B, Hq, S] partial logsumexp
  // Prefill partials (ws_o != nullptr): split s of this launch writes the
  // normalised fp32 row of query token t, head h at
  // ((split_base + s) * part_rows + t) * Hq + h, t the token's index in q.
  // A decode launch uses this layout too (token t = sequence t) when
  // part_rows > 0, else its own [B, Hq, S].
  int32_t split_base;
  int64_t part_rows;
  // Prefill: packed_q > 0 makes the launch one virtual sequence of packed_q
  // query tokens (all of q) over the first max_ctx_len keys of block-table
  // row 0; cu_q_lens and ctx_lens are not read.
  int32_t packed_q;
  // Keys below this position (a multiple of 16) are left out.
  int32_t key_begin;
  // Prefill of an fp8 pool with Q and P quantised to E4M3 and both products
  // on the fp8 MFMA (no packed_q or key_begin).
  int32_t fp8_mma;
  // Row filter by query count q_len_b = cu_q_lens[b+1] - cu_q_lens[b]
  // (kQAll: every sequence).  kQOne: only sequences with q_len_b = 1 (the
  // decode split pass and the merge); kQMany: only sequences with
  // q_len_b > 1 (the prefill pass and the merge).  The others are skipped:
  // nothing is read or written for them.
  int32_t q_filter;
};

constexpr int32_t kQAll = 0, kQOne = 1, kQMany = 2;

// One buffer load of 16 bytes per lane straight into LDS: lane i's bytes
// [voffset, voffset + 16) of the buffer [base, base + nbytes) land at
// lds_addr + 16 * i; bytes at or past nbytes read as zero.  Written as inline
// asm so the compiler's wait-count pass does not drain all outstanding loads
// before each write of M0 (the hardware latches M0 when the load issues);
// callers wait with wait_vmcnt<>() before the data is used.  The instruction
// writes no register.  The compiler's hazard pass does not look inside inline
// asm, so the asm carries its own wait states: s_nop 4 (five) covers both a
// VALU write of a descriptor SGPR (v_readfirstlane) before a vector-memory
// read of it (five wait states) and an M0 write before an LDS DMA (one).
__device__ __forceinline__ void dma16(const void* base, int32_t nbytes, uint32_t voffset,
                                      uint32_t lds_addr) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const i32x4 rs = {__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b))),
                    __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b >> 32) & 0xffff)),
                    __builtin_amdgcn_readfirstlane(nbytes), kRsrcWord3};
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rs), "{m0}"(m0)
               : "memory");
}

// The LDS address (offset in the workgroup's LDS) of a __shared__ object.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

// Wait until at most n of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Full-wave max and sum (64 lanes).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) x = fmaxf(x, __shfl_xor(x, s));
  return x;
}
__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) x += __shfl_xor(x, s);
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) x += __shfl_xor(x, s);
  return x;
}

// fp32 pools: one wave folds keys [t0, t1) of one sequence (t0 a multiple of
// 16, so 64 keys are four whole pages) into the online-softmax state of one
// query row q (d floats in LDS, read by every lane).  Scores take one key per
// lane; P.V takes one feature per lane (two for d = 128), the key weights
// broadcast from their lanes.  o is unnormalised, m is in log2 units of the
// scaled scores.  Keys on invalid pages or at or past t1 get weight 0 and
// their V values are replaced by 0 before use (the pool may hold NaN there).
template <int D>
__device__ __forceinline__ void f32_attend(const AttnArgs& a, const int32_t* bt, int g,
                                           const float* q, int t0, int t1, int lane,
                                           float (&o)[D / 64], float& m, float& l) {
  const float* kb = static_cast<const float*>(a.k);
  const float* vb = static_cast<const float*>(a.v);
  const int Hkv = a.num_kv_heads;
  const float sc = a.scale * kLog2e;
  for (int base = t0; base < t1; base += 64) {
    const int t = base + lane;
    const int32_t phys = t < t1 ? bt[t / kPage] : -1;
    const bool ok = t < t1 && phys >= 0 && phys < a.num_blocks;
    float s = -INFINITY;
    if (ok) {
      const float* kr = kb + ((static_cast<int64_t>(phys) * Hkv + g) * kPage + t % kPage) * D;
      float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll 8
      for (int i = 0; i < D; i += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(kr + i);
        const float4 qv = *reinterpret_cast<const float4*>(q + i);
        d0 = __builtin_fmaf(kv.x, qv.x, d0);
        d1 = __builtin_fmaf(kv.y, qv.y, d1);
        d2 = __builtin_fmaf(kv.z, qv.z, d2);
        d3 = __builtin_fmaf(kv.w, qv.w, d3);
      }
      s = ((d0 + d1) + (d2 + d3)) * sc;
    }
    const float m_new = fmaxf(m, wave_max(s));
    if (m_new == -INFINITY) continue;  // nothing visible yet (uniform)
    const float alpha = fast_exp2(m - m_new);
    const float p = fast_exp2(s - m_new);
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int j = 0; j < D / 64; ++j) o[j] *= alpha;
    m = m_new;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int start = base + pp * kPage;
      if (start >= t1) break;
      const int nv = min(kPage, t1 - start);
      const int32_t pid = __builtin_amdgcn_readlane(phys, pp * kPage);
      if (pid < 0 || pid >= a.num_blocks) continue;
#pragma unroll
      for (int j = 0; j < D / 64; ++j) {
        const float* vr = vb + ((static_cast<int64_t>(pid) * Hkv + g) * D + lane + 64 * j) * kPage;
        float v[kPage];
#pragma unroll
        for (int c = 0; c < kPage; c += 4) {
          const float4 x = *reinterpret_cast<const float4*>(vr + c);
          v[c] = x.x; v[c + 1] = x.y; v[c + 2] = x.z; v[c + 3] = x.w;
        }
        float acc = o[j];
#pragma unroll
        for (int k = 0; k < kPage; ++k) {
          const float pk = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), pp * kPage + k));
          acc = __builtin_fmaf(pk, k < nv ? v[k] : 0.f, acc);
        }
        o[j] = acc;
      }
    }
  }
}

// Workgroups per KV head of the balanced decode (4 waves each): about 512 in
// all (two per compute unit), and no more waves than half the pages.
inline int balanced_wgs(int num_seqs, int num_kv_heads, int max_ctx_len, int key_begin) {
  const int64_t per_seq = (max_ctx_len + 15) / 16 - key_begin / 16;
  const int64_t pages = static_cast<int64_t>(num_seqs) * (per_seq > 0 ? per_seq : 0);
  int64_t w = (512 + num_kv_heads - 1) / num_kv_heads;
  const int64_t by_pages = (pages + 7) / 8;
  if (w > by_pages) w = by_pages;
  return static_cast<int>(w < 1 ? 1 : w);
}
// Workspace of the balanced decode: per KV head, U + B partial slots (U =
// 4 * balanced_wgs waves) of G rows: fp32 rows of head_dim, then one lse each.
inline size_t balanced_ws_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                int max_ctx_len, int key_begin) {
  const int64_t U = 4 * static_cast<int64_t>(
                            balanced_wgs(num_seqs, num_kv_heads, max_ctx_len, key_begin));
  const size_t rows = static_cast<size_t>(num_q_heads) * (U + num_seqs);
  const size_t o_bytes = (rows * head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
  return o_bytes + rows * sizeof(float);
}

// Arguments of the backward kernels (bf16 pool, q, o, dO; fp32 gradients).
struct BwdArgs {
  const uint16_t* k;        // pool K [NB, Hkv, 16, D]
  const uint16_t* v;        // pool V [NB, Hkv, D, 16]
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;
  const uint16_t* q;        // [T, Hq, D]
  const uint16_t* o;        // forward output [T, Hq, D]
  const float* lse;         // forward logsumexp [T, Hq]
  const uint16_t* dout;     // upstream gradient [T, Hq, D]
  float* dq;                // [T, Hq, D]
  float* dk;                // [NB, Hkv, 16, D]
  float* dv;                // [NB, Hkv, D, 16]
  const int32_t* cu_q_lens;
  const int32_t* ctx_lens;
  const int32_t* block_table;
  int32_t bt_stride;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t max_q_len;
  int32_t max_ctx_len;
  float scale;
  int32_t causal;
  int32_t lpad;             // query rows per (KV head, sequence) in the row workspaces
  uint16_t* qt;             // Q^T  [Hkv][B][D][lpad]
  uint16_t* dot;            // dO^T [Hkv][B][D][lpad]
  float* delta;             // rowsum(dO * O) [Hkv][B][lpad]
  float* lse2;              // lse * log2(e)  [Hkv][B][lpad]
  uint16_t* kfm;            // K pages feature-major [NB, Hkv, D, 16]
  uint16_t* vtm;            // V pages token-major   [NB, Hkv, 16, D]
};

// Workspace of the backward: the six regions of BwdArgs, each 256-byte aligned.
struct BwdLayout {
  int lpad;
  size_t off[6];  // qt, dot, delta, lse2, kfm, vtm
  size_t total;
};
inline BwdLayout backward_layout(int num_seqs, int max_q_len, int num_q_heads, int num_kv_heads,
                                 int head_dim, int num_blocks) {
  BwdLayout L;
  const int G = num_q_heads / num_kv_heads;
  L.lpad = ((max_q_len * G + 31) / 32) * 32;
  const size_t rows = static_cast<size_t>(num_kv_heads) * num_seqs * L.lpad;
  const size_t pages = static_cast<size_t>(num_blocks) * num_kv_heads * 16 * head_dim;
  const size_t sz[6] = {rows * head_dim * 2, rows * head_dim * 2, rows * 4, rows * 4,
                        pages * 2, pages * 2};
  size_t o = 0;
  for (int i = 0; i < 6; ++i) {
    L.off[i] = o;
    o += (sz[i] + 255) & ~static_cast<size_t>(255);
  }
  L.total = o;
  return L;
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t st);
hipError_t launch_prefill(const AttnArgs& a, hipStream_t st);
// The decode split pass alone (bf16 or fp8 pool), partials as a's workspace says.
hipError_t launch_decode_split(const AttnArgs& a, hipStream_t st);
// The packed passes of a shared-prefix call: the rows with q_len = 1 attend
// the prefix packed together (one row per sequence) and their own keys
// through the decode split pass, and the two are merged; in a batch that
// also holds rows with q_len > 1, those take the ordinary prefill pass first.
struct SharedLaunch {
  int prefix_len;
  int s_prefix, s_suffix, s_plain;  // key splits of the three passes
  void* qd;                         // q_len = 1 rows gathered ([B][Hq][D] bf16), mixed batches
  float* ws_o;                      // partials of the prefix and own-key passes,
  float* ws_lse;                    //   (s_prefix + s_suffix) x B x Hq rows
  float* ws_o2;                     // partials of the q_len > 1 rows when s_plain > 1
  float* ws_lse2;
};
hipError_t launch_prefill_shared_prefix(const AttnArgs& a, const SharedLaunch& L, hipStream_t st);
hipError_t launch_decode(const AttnArgs& a, hipStream_t st);

}  // namespace pa
