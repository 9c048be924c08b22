// Writing new tokens into the paged KV pool, and reading them back out.
//
// Pool layout (one contiguous chunk per physical block and KV head):
//   K [num_blocks, Hkv, 16, D]   token-major inside the page
//   V [num_blocks, Hkv, D, 16]   feature-major inside the page
// A token's slot is physical_block * 16 + offset (the block-table scheme of
// the survey page's PagedAttention section: logical blocks map to physical
// blocks that need not be contiguous).
//
// fp8 pools hold OCP E4M3 codes with one float scale per physical block for K
// and one for V, shared by all heads: s = amax / 448, code = RNE(clamp(x / s)).
// Quantising takes three passes: clear the per-block amax words, take the amax
// of every written token into its block's word (atomic max on the float bits,
// which order like the values for non-negative floats), then encode.
//
// Appending to a partly filled fp8 page changes its scale: the page's tokens
// below the lowest offset the call writes are its existing tokens; their
// stored values (code * old scale) join the amax, and they are re-encoded
// with the new scale before the new tokens are encoded.
#include "pa_internal.h"

namespace pa {
namespace {

template <typename T>
__global__ void write_copy_kernel(T* __restrict__ kp, T* __restrict__ vp,
                                  const T* __restrict__ kn, const T* __restrict__ vn,
                                  const int32_t* __restrict__ slots, int32_t n, int32_t Hkv,
                                  int32_t D, int32_t num_blocks) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  const int chunks = D / EPC;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(n) * Hkv * chunks;
  if (gid >= total) return;
  const int c = static_cast<int>(gid % chunks);
  const int h = static_cast<int>((gid / chunks) % Hkv);
  const int64_t t = gid / (static_cast<int64_t>(chunks) * Hkv);
  const int32_t slot = slots[t];
  const int32_t phys = slot >> 4, off = slot & 15;
  if (slot < 0 || phys >= num_blocks) return;
  const int64_t src = (t * Hkv + h) * D + c * EPC;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(kn + src);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(vn + src);
  const int64_t chunk_base = (static_cast<int64_t>(phys) * Hkv + h) * kPage * D;
  *reinterpret_cast<u32x4*>(kp + chunk_base + off * D + c * EPC) = kv;
  T vals[EPC];
  *reinterpret_cast<u32x4*>(vals) = vv;
#pragma unroll
  for (int e = 0; e < EPC; ++e) vp[chunk_base + (c * EPC + e) * kPage + off] = vals[e];
}

// p[0, n0) = v0, p[n0, n) = v1.
__global__ void fill_u32_kernel(uint32_t* p, int64_t n0, int64_t n, uint32_t v0, uint32_t v1) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = i < n0 ? v0 : v1;
}

template <typename S>
__device__ __forceinline__ float load_src(const S* p, int64_t i);
template <>
__device__ __forceinline__ float load_src<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_src<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

// One workgroup per token: amax of its K values and of its V values (and,
// when appending, the lowest offset written to its page).
template <typename S>
__global__ void fp8_amax_kernel(const S* __restrict__ kn, const S* __restrict__ vn,
                                const int32_t* __restrict__ slots, int32_t Hkv, int32_t D,
                                int32_t num_blocks, uint32_t* __restrict__ amax_ws,
                                uint32_t* __restrict__ min_off) {
  const int64_t t = blockIdx.x;
  const int32_t slot = slots[t];
  const int32_t phys = slot >> 4;
  if (slot < 0 || phys >= num_blocks) return;
  if (min_off && threadIdx.x == 0) atomicMin(&min_off[phys], static_cast<uint32_t>(slot & 15));
  const int64_t row = Hkv * D;
  float mk = 0.f, mv = 0.f;
  for (int64_t i = threadIdx.x; i < row; i += blockDim.x) {
    mk = fmaxf(mk, fabsf(load_src(kn, t * row + i)));
    mv = fmaxf(mv, fabsf(load_src(vn, t * row + i)));
  }
  for (int s = 32; s >= 1; s >>= 1) {
    mk = fmaxf(mk, __shfl_xor(mk, s));
    mv = fmaxf(mv, __shfl_xor(mv, s));
  }
  __shared__ float red[2][16];
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) {
    red[0][w] = mk;
    red[1][w] = mv;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < static_cast<int>(blockDim.x / 64); ++i) {
      mk = fmaxf(mk, red[0][i]);
      mv = fmaxf(mv, red[1][i]);
    }
    atomicMax(&amax_ws[phys], __float_as_uint(mk));
    atomicMax(&amax_ws[num_blocks + phys], __float_as_uint(mv));
  }
}

__device__ __forceinline__ float fp8_scale_of(uint32_t amax_bits) {
  const float amax = __uint_as_float(amax_bits);
  return amax > 0.f ? amax / 448.0f : 1.0f;  // correctly rounded division
}

__device__ __forceinline__ uint32_t encode_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

__device__ __forceinline__ float to_code_domain(float x, float s) {
  return fminf(fmaxf(x / s, -448.0f), 448.0f);
}

// One thread per (token, head, 8 consecutive dims).
template <typename S>
__global__ void fp8_encode_kernel(uint8_t* __restrict__ kp, uint8_t* __restrict__ vp,
                                  float* __restrict__ k_scale, float* __restrict__ v_scale,
                                  const S* __restrict__ kn, const S* __restrict__ vn,
                                  const int32_t* __restrict__ slots, int32_t n, int32_t Hkv,
                                  int32_t D, int32_t num_blocks,
                                  const uint32_t* __restrict__ amax_ws) {
  const int groups = D / 8;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(n) * Hkv * groups;
  if (gid >= total) return;
  const int c = static_cast<int>(gid % groups);
  const int h = static_cast<int>((gid / groups) % Hkv);
  const int64_t t = gid / (static_cast<int64_t>(groups) * Hkv);
  const int32_t slot = slots[t];
  const int32_t phys = slot >> 4, off = slot & 15;
  if (slot < 0 || phys >= num_blocks) return;
  const float sk = fp8_scale_of(amax_ws[phys]);
  const float sv = fp8_scale_of(amax_ws[num_blocks + phys]);
  const int64_t src = (t * Hkv + h) * D + c * 8;
  float kx[8], vx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kx[e] = to_code_domain(load_src(kn, src + e), sk);
    vx[e] = to_code_domain(load_src(vn, src + e), sv);
  }
  const int64_t chunk_base = (static_cast<int64_t>(phys) * Hkv + h) * kPage * D;
  u32x2 kc;
  kc.x = encode_fp8x4(kx[0], kx[1], kx[2], kx[3]);
  kc.y = encode_fp8x4(kx[4], kx[5], kx[6], kx[7]);
  *reinterpret_cast<u32x2*>(kp + chunk_base + off * D + c * 8) = kc;
  const uint32_t v0 = encode_fp8x4(vx[0], vx[1], vx[2], vx[3]);
  const uint32_t v1 = encode_fp8x4(vx[4], vx[5], vx[6], vx[7]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w = e < 4 ? v0 : v1;
    vp[chunk_base + (c * 8 + e) * kPage + off] = static_cast<uint8_t>(w >> (8 * (e & 3)));
  }
  if (h == 0 && c == 0) {  // every token of the block stores the same value
    k_scale[phys] = sk;
    v_scale[phys] = sv;
  }
}

// Appending, pass 3: the token at the lowest offset written to its page leads
// the page.  The new tokens' amax is final (pass 2); the leader adds the
// page's existing values (offsets below it, all heads, as stored: code * old
// scale), stores the page's final amax for pass 4, and re-encodes the existing
// codes with the new scale (the old scale is still in the scale arrays; pass
// 4, which stores the new one, runs after this).
__global__ __launch_bounds__(256) void fp8_requant_kernel(
    uint8_t* __restrict__ kp, uint8_t* __restrict__ vp, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ slots, int32_t Hkv, int32_t D,
    int32_t num_blocks, const uint32_t* __restrict__ min_off, uint32_t* __restrict__ amax_ws) {
  const int32_t slot = slots[blockIdx.x];
  const int32_t phys = slot >> 4, off = slot & 15;
  if (slot < 0 || phys >= num_blocks || static_cast<uint32_t>(off) != min_off[phys] || off == 0)
    return;
  const float sk_old = k_scale[phys], sv_old = v_scale[phys];
  const int64_t base = static_cast<int64_t>(phys) * Hkv * kPage * D;
  const int n = Hkv * off * D;  // existing values per pool
  float mk = 0.f, mv = 0.f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int d = i % D, t = (i / D) % off, h = i / (D * off);
    const int64_t chunk = base + static_cast<int64_t>(h) * kPage * D;
    mk = fmaxf(mk, fabsf(__builtin_amdgcn_cvt_f32_fp8(kp[chunk + t * D + d], 0) * sk_old));
    mv = fmaxf(mv, fabsf(__builtin_amdgcn_cvt_f32_fp8(vp[chunk + d * kPage + t], 0) * sv_old));
  }
  for (int s = 32; s >= 1; s >>= 1) {
    mk = fmaxf(mk, __shfl_xor(mk, s));
    mv = fmaxf(mv, __shfl_xor(mv, s));
  }
  __shared__ float red[2][4];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = mk;
    red[1][w] = mv;
  }
  __syncthreads();
  mk = fmaxf(__uint_as_float(amax_ws[phys]), fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3])));
  mv = fmaxf(__uint_as_float(amax_ws[num_blocks + phys]),
             fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3])));
  __syncthreads();  // every thread has read the new tokens' amax
  if (threadIdx.x == 0) {
    amax_ws[phys] = __float_as_uint(mk);
    amax_ws[num_blocks + phys] = __float_as_uint(mv);
  }
  const float sk = fp8_scale_of(__float_as_uint(mk)), sv = fp8_scale_of(__float_as_uint(mv));
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int d = i % D, t = (i / D) % off, h = i / (D * off);
    const int64_t chunk = base + static_cast<int64_t>(h) * kPage * D;
    uint8_t* kq = kp + chunk + t * D + d;
    uint8_t* vq = vp + chunk + d * kPage + t;
    const float xk = __builtin_amdgcn_cvt_f32_fp8(*kq, 0) * sk_old;
    const float xv = __builtin_amdgcn_cvt_f32_fp8(*vq, 0) * sv_old;
    *kq = static_cast<uint8_t>(encode_fp8x4(to_code_domain(xk, sk), 0.f, 0.f, 0.f) & 0xff);
    *vq = static_cast<uint8_t>(encode_fp8x4(to_code_domain(xv, sv), 0.f, 0.f, 0.f) & 0xff);
  }
}

// Copy whole physical blocks (all heads, K and V, and the fp8 scales): one
// thread per 16 bytes of a block's K (and the same 16 bytes of its V).
__global__ void copy_blocks_kernel(char* __restrict__ kp, char* __restrict__ vp,
                                   float* __restrict__ k_scale, float* __restrict__ v_scale,
                                   const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
                                   int32_t n, int64_t block_bytes, int32_t num_blocks) {
  const int64_t per = block_bytes / 16;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= per * n) return;
  const int64_t pair = gid / per, c = gid % per;
  const int32_t s = src[pair], d = dst[pair];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return;
  const int64_t so = s * block_bytes + c * 16, dof = d * block_bytes + c * 16;
  *reinterpret_cast<u32x4*>(kp + dof) = *reinterpret_cast<const u32x4*>(kp + so);
  *reinterpret_cast<u32x4*>(vp + dof) = *reinterpret_cast<const u32x4*>(vp + so);
  if (c == 0 && k_scale) {
    k_scale[d] = k_scale[s];
    v_scale[d] = v_scale[s];
  }
}

// One workgroup per (logical page j, sequence b).
template <typename T>
__global__ void gather_kernel(const T* __restrict__ kp, const T* __restrict__ vp,
                              const int32_t* __restrict__ bt, int32_t bt_stride,
                              const int32_t* __restrict__ ctx, const int32_t* __restrict__ cu,
                              int32_t Hkv, int32_t D, int32_t num_blocks, T* __restrict__ ko,
                              T* __restrict__ vo) {
  const int j = blockIdx.x, b = blockIdx.y;
  const int32_t c = ctx[b];
  if (j * kPage >= c) return;
  const int32_t phys = bt[static_cast<int64_t>(b) * bt_stride + j];
  if (phys < 0 || phys >= num_blocks) return;
  const int n = min(kPage, c - j * kPage);
  const int64_t out0 = static_cast<int64_t>(cu[b]) + j * kPage;
  const int per_page = Hkv * n * D;
  for (int i = threadIdx.x; i < per_page; i += blockDim.x) {
    const int d = i % D;
    const int t = (i / D) % n;
    const int h = i / (D * n);
    const int64_t chunk = (static_cast<int64_t>(phys) * Hkv + h) * kPage * D;
    const int64_t o = ((out0 + t) * Hkv + h) * D + d;
    ko[o] = kp[chunk + t * D + d];
    vo[o] = vp[chunk + d * kPage + t];
  }
}

unsigned blocks_for(int64_t threads, int per_block) {
  return static_cast<unsigned>((threads + per_block - 1) / per_block);
}

}  // namespace

hipError_t launch_write_kv(const pa_kv_pool& pool, const void* k_new, const void* v_new,
                           pa_dtype src, const int32_t* slots, int32_t n, uint32_t* amax_ws,
                           bool append, hipStream_t st) {
  const int Hkv = pool.num_kv_heads, D = pool.head_dim, NB = pool.num_blocks;
  if (pool.kv_dtype == PA_F32 || pool.kv_dtype == PA_BF16) {
    const int epc = pool.kv_dtype == PA_F32 ? 4 : 8;
    const int64_t threads = static_cast<int64_t>(n) * Hkv * (D / epc);
    if (pool.kv_dtype == PA_F32) {
      write_copy_kernel<uint32_t><<<blocks_for(threads, 256), 256, 0, st>>>(
          static_cast<uint32_t*>(pool.k), static_cast<uint32_t*>(pool.v),
          static_cast<const uint32_t*>(k_new), static_cast<const uint32_t*>(v_new), slots, n,
          Hkv, D, NB);
    } else {
      write_copy_kernel<uint16_t><<<blocks_for(threads, 256), 256, 0, st>>>(
          static_cast<uint16_t*>(pool.k), static_cast<uint16_t*>(pool.v),
          static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), slots, n,
          Hkv, D, NB);
    }
    return hipGetLastError();
  }
  // amax words (K then V) to 0 and, when appending, the lowest-offset words to 16
  const int64_t words = (append ? 3 : 2) * static_cast<int64_t>(NB);
  fill_u32_kernel<<<blocks_for(words, 256), 256, 0, st>>>(amax_ws, 2 * static_cast<int64_t>(NB),
                                                          words, 0u, static_cast<uint32_t>(kPage));
  uint32_t* min_off = append ? amax_ws + 2 * static_cast<int64_t>(NB) : nullptr;
  const int64_t threads = static_cast<int64_t>(n) * Hkv * (D / 8);
  uint8_t* kp = static_cast<uint8_t*>(pool.k);
  uint8_t* vp = static_cast<uint8_t*>(pool.v);
  if (src == PA_F32)
    fp8_amax_kernel<float><<<n, 256, 0, st>>>(static_cast<const float*>(k_new),
                                              static_cast<const float*>(v_new), slots, Hkv, D,
                                              NB, amax_ws, min_off);
  else
    fp8_amax_kernel<uint16_t><<<n, 256, 0, st>>>(static_cast<const uint16_t*>(k_new),
                                                 static_cast<const uint16_t*>(v_new), slots, Hkv,
                                                 D, NB, amax_ws, min_off);
  if (append)
    fp8_requant_kernel<<<n, 256, 0, st>>>(kp, vp, pool.k_scale, pool.v_scale, slots, Hkv, D, NB,
                                          min_off, amax_ws);
  if (src == PA_F32)
    fp8_encode_kernel<float><<<blocks_for(threads, 256), 256, 0, st>>>(
        kp, vp, pool.k_scale, pool.v_scale, static_cast<const float*>(k_new),
        static_cast<const float*>(v_new), slots, n, Hkv, D, NB, amax_ws);
  else
    fp8_encode_kernel<uint16_t><<<blocks_for(threads, 256), 256, 0, st>>>(
        kp, vp, pool.k_scale, pool.v_scale, static_cast<const uint16_t*>(k_new),
        static_cast<const uint16_t*>(v_new), slots, n, Hkv, D, NB, amax_ws);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const pa_kv_pool& pool, const int32_t* src, const int32_t* dst,
                              int32_t n, hipStream_t st) {
  const int64_t es = pool.kv_dtype == PA_F32 ? 4 : (pool.kv_dtype == PA_BF16 ? 2 : 1);
  const int64_t block_bytes = static_cast<int64_t>(pool.num_kv_heads) * kPage * pool.head_dim * es;
  const bool fp8 = pool.kv_dtype == PA_FP8_E4M3;
  copy_blocks_kernel<<<blocks_for(block_bytes / 16 * n, 256), 256, 0, st>>>(
      static_cast<char*>(pool.k), static_cast<char*>(pool.v), fp8 ? pool.k_scale : nullptr,
      fp8 ? pool.v_scale : nullptr, src, dst, n, block_bytes, pool.num_blocks);
  return hipGetLastError();
}

hipError_t launch_gather_kv(const pa_kv_pool& pool, const int32_t* bt, int32_t bt_stride,
                            const int32_t* ctx, const int32_t* cu_ctx, int32_t B,
                            int32_t max_ctx, void* k_out, void* v_out, hipStream_t st) {
  const dim3 grid((max_ctx + kPage - 1) / kPage, B);
  const int Hkv = pool.num_kv_heads, D = pool.head_dim, NB = pool.num_blocks;
  switch (pool.kv_dtype) {
    case PA_F32:
      gather_kernel<uint32_t><<<grid, 256, 0, st>>>(
          static_cast<const uint32_t*>(pool.k), static_cast<const uint32_t*>(pool.v), bt,
          bt_stride, ctx, cu_ctx, Hkv, D, NB, static_cast<uint32_t*>(k_out),
          static_cast<uint32_t*>(v_out));
      break;
    case PA_BF16:
      gather_kernel<uint16_t><<<grid, 256, 0, st>>>(
          static_cast<const uint16_t*>(pool.k), static_cast<const uint16_t*>(pool.v), bt,
          bt_stride, ctx, cu_ctx, Hkv, D, NB, static_cast<uint16_t*>(k_out),
          static_cast<uint16_t*>(v_out));
      break;
    default:
      gather_kernel<uint8_t><<<grid, 256, 0, st>>>(
          static_cast<const uint8_t*>(pool.k), static_cast<const uint8_t*>(pool.v), bt,
          bt_stride, ctx, cu_ctx, Hkv, D, NB, static_cast<uint8_t*>(k_out),
          static_cast<uint8_t*>(v_out));
      break;
  }
  return hipGetLastError();
}

}  // namespace pa
