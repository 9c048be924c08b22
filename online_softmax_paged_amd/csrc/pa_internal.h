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
                           hipStream_t st);
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
  int32_t num_splits;          // decode only
  float* ws_o;                 // decode: [B, Hq, S, D] partial outputs
  float* ws_lse;               // decode: [B, Hq, S] partial logsumexp
};

hipError_t launch_prefill(const AttnArgs& a, hipStream_t st);
hipError_t launch_decode(const AttnArgs& a, hipStream_t st);

}  // namespace pa
