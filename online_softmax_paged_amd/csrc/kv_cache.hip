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

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t value) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

template <typename S>
__device__ __forceinline__ float load_src(const S* p, int64_t i);
template <>
__device__ __forceinline__ float load_src<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_src<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

// One workgroup per token: amax of its K values and of its V values.
template <typename S>
__global__ void fp8_amax_kernel(const S* __restrict__ kn, const S* __restrict__ vn,
                                const int32_t* __restrict__ slots, int32_t Hkv, int32_t D,
                                int32_t num_blocks, uint32_t* __restrict__ amax_ws) {
  const int64_t t = blockIdx.x;
  const int32_t slot = slots[t];
  const int32_t phys = slot >> 4;
  if (slot < 0 || phys >= num_blocks) return;
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
                           hipStream_t st) {
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
  fill_u32_kernel<<<blocks_for(2 * static_cast<int64_t>(NB), 256), 256, 0, st>>>(
      amax_ws, 2 * static_cast<int64_t>(NB), 0u);
  const int64_t threads = static_cast<int64_t>(n) * Hkv * (D / 8);
  uint8_t* kp = static_cast<uint8_t*>(pool.k);
  uint8_t* vp = static_cast<uint8_t*>(pool.v);
  if (src == PA_F32) {
    const float* kn = static_cast<const float*>(k_new);
    const float* vn = static_cast<const float*>(v_new);
    fp8_amax_kernel<float><<<n, 256, 0, st>>>(kn, vn, slots, Hkv, D, NB, amax_ws);
    fp8_encode_kernel<float><<<blocks_for(threads, 256), 256, 0, st>>>(
        kp, vp, pool.k_scale, pool.v_scale, kn, vn, slots, n, Hkv, D, NB, amax_ws);
  } else {
    const uint16_t* kn = static_cast<const uint16_t*>(k_new);
    const uint16_t* vn = static_cast<const uint16_t*>(v_new);
    fp8_amax_kernel<uint16_t><<<n, 256, 0, st>>>(kn, vn, slots, Hkv, D, NB, amax_ws);
    fp8_encode_kernel<uint16_t><<<blocks_for(threads, 256), 256, 0, st>>>(
        kp, vp, pool.k_scale, pool.v_scale, kn, vn, slots, n, Hkv, D, NB, amax_ws);
  }
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
