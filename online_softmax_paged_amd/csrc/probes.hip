// Measurement probes: a streaming read of a device buffer, the same read in
// the decode's page pattern, and MFMA loops on register operands.  They are not part of the attention path; they measure
// what this GPU sustains so that each attention kernel's rate can be read
// against a measured ceiling as well as against the spec peak.
#include "pa_internal.h"

namespace pa {
namespace {

// Every 16-byte word of p read once, grid-stride, with non-temporal loads;
// one XOR per thread is written so the loads cannot be dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ out) {
  const size_t tid = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  u32x4 acc = {0, 0, 0, 0};
  for (size_t i = tid; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  out[tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// The decode's read pattern without its arithmetic: each workgroup (four
// waves) streams its own run of pages of 8 KiB (a bf16 d = 128 K page of 4 KiB
// read as 16 keys x 64-byte pieces per 16-byte-per-lane load, then the V page
// of 4 KiB read 8 bytes per lane), each wave taking every fourth page with two
// pages in flight, as decode_split_kernel loads them.  All workgroups get the
// same number of pages, so this is the time that pattern needs for a given
// volume with the work perfectly balanced.
__global__ __launch_bounds__(256) void page_stream_kernel(const char* __restrict__ base,
                                                          int pages_per_wg,
                                                          uint32_t* __restrict__ out) {
  constexpr int kRingP = 2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, c = lane & 15, grp = lane >> 4;
  const char* wg = base + static_cast<size_t>(blockIdx.x) * pages_per_wg * 8192;
  u32x4 acc = {0, 0, 0, 0};
  for (int p0 = wave * kRingP; p0 < pages_per_wg; p0 += 4 * kRingP) {
    u32x4 k[kRingP][4];
    u32x2 v[kRingP][8];
#pragma unroll
    for (int r = 0; r < kRingP; ++r) {
      const int p = min(p0 + r, pages_per_wg - 1);
      const char* kp = wg + static_cast<size_t>(p) * 8192;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        k[r][ks] = *reinterpret_cast<const u32x4*>(kp + (c * 128 + ks * 32 + grp * 8) * 2);
#pragma unroll
      for (int db = 0; db < 8; ++db)
        v[r][db] = *reinterpret_cast<const u32x2*>(kp + 4096 + ((db * 16 + c) * 16 + grp * 4) * 2);
    }
#pragma unroll
    for (int r = 0; r < kRingP; ++r) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc ^= k[r][ks];
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        acc.x ^= v[r][db].x;
        acc.y ^= v[r][db].y;
      }
    }
  }
  out[static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Each wave: four independent accumulator chains of iters MFMAs each.
template <bool FP8>
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ out, int iters) {
  const int t = threadIdx.x;
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  if constexpr (FP8) {
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x38383838 + (t & 3);  // E4M3 codes near 1.0
      b[i] = 0x30303030 + i;
    }
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 127, 0, 127);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 127, 0, 127);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 127, 0, 127);
    }
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = static_cast<__bf16>(t * 1e-3f + i);
      b[i] = static_cast<__bf16>(i * 0.5f);
    }
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += (c0[i] + c1[i]) + (c2[i] + c3[i]);
  out[static_cast<size_t>(blockIdx.x) * 256 + t] = s;
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" {

pa_status pa_probe_stream_read(const void* buf, size_t bytes, uint32_t* out, int32_t blocks,
                               void* stream) {
  if (!buf || !out || bytes == 0 || bytes % 16 != 0 || blocks < 1 || blocks > 65535)
    return PA_ERR_INVALID_ARG;
  stream_read_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(buf), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_probe_page_stream(const void* buf, size_t bytes, uint32_t* out, int32_t blocks,
                               void* stream) {
  if (!buf || !out || blocks < 1 || blocks > 65535 || bytes == 0 ||
      bytes % (static_cast<size_t>(blocks) * 8192) != 0 ||
      bytes / (static_cast<size_t>(blocks) * 8192) > (1u << 30))
    return PA_ERR_INVALID_ARG;
  const int pages = static_cast<int>(bytes / (static_cast<size_t>(blocks) * 8192));
  page_stream_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const char*>(buf), pages, out);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_probe_mfma(pa_dtype dtype, float* out, int32_t blocks, int32_t iters, void* stream) {
  if (!out || blocks < 1 || blocks > 65535 || iters < 1) return PA_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == PA_BF16)
    mfma_loop_kernel<false><<<blocks, 256, 0, st>>>(out, iters);
  else if (dtype == PA_FP8_E4M3)
    mfma_loop_kernel<true><<<blocks, 256, 0, st>>>(out, iters);
  else
    return PA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"
