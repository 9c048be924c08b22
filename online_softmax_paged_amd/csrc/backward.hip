// Backward of the paged attention for bf16 pools: dQ, dK, dV from the
// forward's output O and logsumexp, recomputing the attention weights tile by
// tile instead of storing them (the FlashAttention page, core-principle
// section: the backward rebuilds what it needs from the kept statistics).
//
// With S = scale Q K^T (masked as in the forward), P = exp(S - LSE) row by
// row, and the upstream gradient dO:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D) with D = rowsum(dO * O),
//   dQ = scale dS K,  dK = scale dS^T Q.
// (rowsum(dO * O) equals rowsum(P * dP), the softmax Jacobian's row term.)
//
// Every product runs on v_mfma_f32_32x32x16_bf16.  An MFMA operand lane
// holds 8 consecutive elements along the contracted dimension, so each input
// is needed in the layout that makes its contracted dimension contiguous:
//   S    = Q K^T   contracts features:  Q, K row-major (K pages are)
//   dP   = dO V^T  contracts features:  dO row-major, V token-major
//   dV^T = dO^T P  contracts query rows: dO^T feature-major
//   dK^T = Q^T dS  contracts query rows: Q^T feature-major
//   dQ^T = K^T dS^T contracts keys:     K feature-major
// Two prep kernels write the missing layouts once (Q^T and dO^T per sequence,
// padded to 32-row tiles; each referenced page's K feature-major and V
// token-major, with slots past the context zeroed), plus D and LSE * log2(e)
// per query row.  Then one kernel owns 128 keys per workgroup (32 per wave)
// and walks the query tiles that see them, accumulating dK and dV in
// registers; another owns 128 query rows per workgroup and walks the key
// tiles, accumulating dQ.  Neither needs atomics: results are deterministic.
//
// Query rows of a KV head g are the (token, head) pairs of its G query heads,
// row R = t * G + (h - g * G) within a sequence, as in the forward.
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kBT = 32;  // rows (or keys) per tile

// 16-byte chunk reads of the two LDS tile layouts.
//  Row tile [32 rows][D]: chunk j of row r at j ^ (r % (D/8)).
//  Col tile [2 halves][D][16]: rows 16c..16c+15 of feature d, 8-row chunk e
//  at e ^ ((d / 8) % 2).
template <int D>
__device__ __forceinline__ bf16x8 row_read(const uint16_t* t, int r, int j) {
  constexpr int CPR = D / 8;
  return *reinterpret_cast<const bf16x8*>(t + (r * CPR + (j ^ (r % CPR))) * 8);
}
template <int D>
__device__ __forceinline__ int row_pos(int r, int j) {
  constexpr int CPR = D / 8;
  return (r * CPR + (j ^ (r % CPR))) * 8;
}
template <int D>
__device__ __forceinline__ bf16x8 col_read(const uint16_t* t, int d, int c, int e) {
  return *reinterpret_cast<const bf16x8*>(t + c * (D * 16) + d * 16 + ((e ^ ((d >> 3) & 1)) * 8));
}
template <int D>
__device__ __forceinline__ int col_pos(int d, int c, int e) {
  return c * (D * 16) + d * 16 + ((e ^ ((d >> 3) & 1)) * 8);
}

// The 16 fp32 values a lane holds of a 32x32 MFMA result (value v is row
// 8*(v/4) + 4*half + v%4 of its column) rounded to bf16 and rearranged
// across the two lane halves into the B operand of a product that contracts
// those rows: k-step c covers rows 16c..16c+15, half 0 taking rows 16c..+7.
__device__ __forceinline__ bf16x8 rows_to_b(const float (&x)[16], int c) {
  const uint32_t A0 = pack_bf16x2(x[8 * c + 0], x[8 * c + 1]);
  const uint32_t A1 = pack_bf16x2(x[8 * c + 2], x[8 * c + 3]);
  const uint32_t B0 = pack_bf16x2(x[8 * c + 4], x[8 * c + 5]);
  const uint32_t B1 = pack_bf16x2(x[8 * c + 6], x[8 * c + 7]);
  const auto r0 = __builtin_amdgcn_permlane32_swap(A0, B0, false, false);
  const auto r1 = __builtin_amdgcn_permlane32_swap(A1, B1, false, false);
  return __builtin_bit_cast(bf16x8, u32x4{r0[0], r1[0], r0[1], r1[1]});
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ int clamp_ctx(const BwdArgs& a, int b) {
  const int c = a.ctx_lens[b];
  return c < 0 ? 0 : (c > a.max_ctx_len ? a.max_ctx_len : c);
}

__device__ __forceinline__ int32_t page_id(const BwdArgs& a, int b, int page, int n_pages) {
  if (page >= n_pages) return -1;
  const int32_t p = a.block_table[static_cast<int64_t>(b) * a.bt_stride + page];
  return p >= 0 && p < a.num_blocks ? p : -1;
}

// ---------------------------------------------------------------------------
// Prep 1: per (sequence, KV head, 64 query rows): D = rowsum(dO * O), LSE *
// log2(e), and Q^T, dO^T into [Hkv][D][B][lpad] (rows past the sequence 0).
template <int D>
__global__ __launch_bounds__(256) void bwd_rows_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;
  constexpr int LD = D + 8;  // padded LDS row
  __shared__ uint16_t sq[64 * LD];
  __shared__ uint16_t sd[64 * LD];
  const int tid = threadIdx.x;
  const int R0 = blockIdx.x * 64, g = blockIdx.y, b = blockIdx.z;
  const int Hq = a.num_q_heads, G = Hq / a.num_kv_heads, B = a.num_seqs;
  const int q0 = a.cu_q_lens[b];
  const int nrows = (a.cu_q_lens[b + 1] - q0) * G;
  const int64_t rowbase = (static_cast<int64_t>(g) * B + b) * a.lpad;
  for (int idx = tid; idx < 64 * CPR; idx += 256) {  // 256 % CPR == 0: a row's chunks share a wave
    const int r = idx / CPR, c = idx % CPR, R = R0 + r;
    u32x4 qv = {0, 0, 0, 0}, dv = {0, 0, 0, 0}, ov = {0, 0, 0, 0};
    int64_t row = 0;
    if (R < nrows) {
      row = static_cast<int64_t>(q0 + R / G) * Hq + (g * G + R % G);
      qv = *reinterpret_cast<const u32x4*>(a.q + row * D + c * 8);
      dv = *reinterpret_cast<const u32x4*>(a.dout + row * D + c * 8);
      ov = *reinterpret_cast<const u32x4*>(a.o + row * D + c * 8);
    }
    *reinterpret_cast<u32x4*>(sq + r * LD + c * 8) = qv;
    *reinterpret_cast<u32x4*>(sd + r * LD + c * 8) = dv;
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      dot += bf16lo(dv[k]) * bf16lo(ov[k]) + bf16hi(dv[k]) * bf16hi(ov[k]);
#pragma unroll
    for (int s = 1; s < CPR; s <<= 1) dot += __shfl_xor(dot, s);
    if (c == 0 && R < a.lpad) {
      a.delta[rowbase + R] = R < nrows ? dot : 0.f;
      a.lse2[rowbase + R] = R < nrows ? a.lse[row] * kLog2e : 0.f;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < D * 8; idx += 256) {
    const int d = idx / 8, e = idx % 8;
    const int R = R0 + 8 * e;
    if (R >= a.lpad) continue;
    u32x4 wq, wd;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 8 * e + 2 * k;
      wq[k] = static_cast<uint32_t>(sq[r * LD + d]) | (static_cast<uint32_t>(sq[(r + 1) * LD + d]) << 16);
      wd[k] = static_cast<uint32_t>(sd[r * LD + d]) | (static_cast<uint32_t>(sd[(r + 1) * LD + d]) << 16);
    }
    const int64_t off = ((static_cast<int64_t>(g) * D + d) * B + b) * a.lpad + R;
    *reinterpret_cast<u32x4*>(a.qt + off) = wq;
    *reinterpret_cast<u32x4*>(a.dot + off) = wd;
  }
}

// Prep 2: per (sequence, KV head, page): the page's K feature-major into
// kfm [NB][Hkv][D][16] and its V token-major into vtm [NB][Hkv][16][D],
// slots at or past the context zeroed.
template <int D>
__global__ __launch_bounds__(256) void bwd_pages_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;
  __shared__ uint16_t sk[16 * (D + 8)];
  __shared__ uint16_t sv[D * 24];
  const int tid = threadIdx.x, j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int ctx = clamp_ctx(a, b);
  const int n_pages = (ctx + kPage - 1) / kPage;
  const int32_t phys = page_id(a, b, j, n_pages);
  if (phys < 0) return;
  const int nv = min(kPage, ctx - j * kPage);  // slots in use
  const int64_t chunk = (static_cast<int64_t>(phys) * a.num_kv_heads + g) * (kPage * D);
  for (int idx = tid; idx < kPage * CPR; idx += 256) {
    const int s = idx / CPR, c = idx % CPR;
    u32x4 w = {0, 0, 0, 0};
    if (s < nv) w = *reinterpret_cast<const u32x4*>(a.k + chunk + s * D + c * 8);
    *reinterpret_cast<u32x4*>(sk + s * (D + 8) + c * 8) = w;
  }
  for (int idx = tid; idx < 2 * D; idx += 256) {
    const int d = idx / 2, e = idx % 2;
    u32x4 w = *reinterpret_cast<const u32x4*>(a.v + chunk + d * kPage + e * 8);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = e * 8 + 2 * k;
      const uint32_t lo = s < nv ? 0xffffu : 0u, hi = s + 1 < nv ? 0xffff0000u : 0u;
      w[k] &= lo | hi;
    }
    *reinterpret_cast<u32x4*>(sv + d * 24 + e * 8) = w;
  }
  __syncthreads();
  for (int idx = tid; idx < 2 * D; idx += 256) {  // kfm chunk (feature d, slots 8e..8e+7)
    const int d = idx / 2, e = idx % 2;
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = e * 8 + 2 * k;
      w[k] = static_cast<uint32_t>(sk[s * (D + 8) + d]) |
             (static_cast<uint32_t>(sk[(s + 1) * (D + 8) + d]) << 16);
    }
    *reinterpret_cast<u32x4*>(a.kfm + chunk + d * kPage + e * 8) = w;
  }
  for (int idx = tid; idx < kPage * CPR; idx += 256) {  // vtm chunk (slot s, features 8c..8c+7)
    const int s = idx / CPR, c = idx % CPR;
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = c * 8 + 2 * k;
      w[k] = static_cast<uint32_t>(sv[d * 24 + s]) | (static_cast<uint32_t>(sv[(d + 1) * 24 + s]) << 16);
    }
    *reinterpret_cast<u32x4*>(a.vtm + chunk + s * D + c * 8) = w;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (sequence, KV head, 128 keys); wave w owns keys
// 32w..32w+31 of them, K and V of its keys held as MFMA operands.  The query
// tiles (32 rows) that see any of the keys are staged in LDS for all four
// waves: Q and dO row-major, Q^T and dO^T feature-major, D and LSE*log2(e).
template <int D>
struct RowsStage {
  uint16_t q[kBT * D], d[kBT * D], qt[kBT * D], dt[kBT * D];
  float lse2[kBT], delta[kBT];
};

template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;
  __shared__ RowsStage<D> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv, B = a.num_seqs;
  const int b = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int ctx = clamp_ctx(a, b);
  const int k0 = blockIdx.y * 128;
  if (k0 >= ctx) return;
  const int q0 = a.cu_q_lens[b], qlen = a.cu_q_lens[b + 1] - q0;
  const int nrows = qlen * G, pos_base = ctx - qlen;
  const int n_pages = (ctx + kPage - 1) / kPage;
  const float sc = a.scale * kLog2e;

  // this lane's key (its MFMA column) and the operands of the wave's keys
  const int key = k0 + 32 * wave + col;
  const int32_t phys = page_id(a, b, key / kPage, n_pages);
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const int64_t base = (static_cast<int64_t>(phys < 0 ? 0 : phys) * Hkv + g) * (kPage * D) +
                         (key % kPage) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(a.k + base + ks * 16);
      bf16x8 y = *reinterpret_cast<const bf16x8*>(a.vtm + base + ks * 16);
      kf[ks] = phys < 0 ? bf16x8{} : x;
      vf[ks] = phys < 0 ? bf16x8{} : y;
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

  // query tiles that see a key of this workgroup (causal: from the token at
  // position k0 on)
  const int t_first = a.causal ? max(0, k0 - pos_base) : 0;
  const int tile0 = (t_first * G) / kBT, n_tiles = (nrows + kBT - 1) / kBT;
  const int64_t rowbase = (static_cast<int64_t>(g) * B + b) * a.lpad;
  for (int it = tile0; it < n_tiles; ++it) {
    const int R0 = it * kBT;
    __syncthreads();  // the previous tile's reads are done
    for (int idx = tid; idx < kBT * CPR; idx += 256) {
      const int r = idx / CPR, c = idx % CPR, R = R0 + r;
      u32x4 qv = {0, 0, 0, 0}, dv_ = {0, 0, 0, 0};
      if (R < nrows) {
        const int64_t row = static_cast<int64_t>(q0 + R / G) * Hq + (g * G + R % G);
        qv = *reinterpret_cast<const u32x4*>(a.q + row * D + c * 8);
        dv_ = *reinterpret_cast<const u32x4*>(a.dout + row * D + c * 8);
      }
      *reinterpret_cast<u32x4*>(sm.q + row_pos<D>(r, c)) = qv;
      *reinterpret_cast<u32x4*>(sm.d + row_pos<D>(r, c)) = dv_;
    }
    for (int idx = tid; idx < D * 4; idx += 256) {
      const int d = idx / 4, c = (idx / 2) % 2, e = idx % 2;
      const int64_t off = ((static_cast<int64_t>(g) * D + d) * B + b) * a.lpad + R0 + 16 * c + 8 * e;
      *reinterpret_cast<u32x4*>(sm.qt + col_pos<D>(d, c, e)) = *reinterpret_cast<const u32x4*>(a.qt + off);
      *reinterpret_cast<u32x4*>(sm.dt + col_pos<D>(d, c, e)) = *reinterpret_cast<const u32x4*>(a.dot + off);
    }
    if (tid < kBT) sm.lse2[tid] = a.lse2[rowbase + R0 + tid];
    else if (tid < 2 * kBT) sm.delta[tid - kBT] = a.delta[rowbase + R0 + tid - kBT];
    __syncthreads();

    // S and dP for (query rows x this lane's key)
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(sm.q, col, 2 * ks + half), kf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(sm.d, col, 2 * ks + half), vf[ks], dp, 0, 0, 0);
    }
    float p[16], ds[16];
#pragma unroll
    for (int bq = 0; bq < 4; ++bq) {
      const f32x4 l2 = *reinterpret_cast<const f32x4*>(sm.lse2 + 8 * bq + 4 * half);
      const f32x4 dl = *reinterpret_cast<const f32x4*>(sm.delta + 8 * bq + 4 * half);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = 4 * bq + r, R = R0 + 8 * bq + 4 * half + r;
        const bool vis = R < nrows && key < ctx && (!a.causal || key <= pos_base + R / G);
        p[v] = vis ? fast_exp2(__builtin_fmaf(s[v], sc, -l2[r])) : 0.f;
        ds[v] = vis ? p[v] * (dp[v] - dl[r]) : 0.f;
      }
    }
    // dV^T += dO^T P,  dK^T += Q^T dS  (contract the 32 query rows)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 pb = rows_to_b(p, c), sb = rows_to_b(ds, c);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = db * 32 + col;
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_read<D>(sm.dt, d, c, half), pb, dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_read<D>(sm.qt, d, c, half), sb, dk[db], 0, 0, 0);
      }
    }
  }

  // write this lane's key: dK token-major, dV feature-major (the pool's layouts)
  if (phys < 0) return;
  const int slot = key % kPage;
  const int64_t chunk = (static_cast<int64_t>(phys) * Hkv + g) * (kPage * D);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int bq = 0; bq < 4; ++bq) {
      const int f = db * 32 + 8 * bq + 4 * half;
      const f32x4 w = {dk[db][4 * bq] * a.scale, dk[db][4 * bq + 1] * a.scale,
                       dk[db][4 * bq + 2] * a.scale, dk[db][4 * bq + 3] * a.scale};
      *reinterpret_cast<f32x4*>(a.dk + chunk + slot * D + f) = w;
#pragma unroll
      for (int r = 0; r < 4; ++r) a.dv[chunk + (f + r) * kPage + slot] = dv[db][4 * bq + r];
    }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (sequence, KV head, 128 query rows), wave w owning
// rows 32w..32w+31 with its Q and dO rows as MFMA operands; the key tiles
// (32 keys, two pages) it sees are staged in LDS: K and V token-major, K
// feature-major.
template <int D>
struct KeysStage {
  uint16_t k[kBT * D], v[kBT * D], kt[kBT * D];
};

template <int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;
  __shared__ KeysStage<D> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv, B = a.num_seqs;
  const int b = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int q0 = a.cu_q_lens[b], qlen = a.cu_q_lens[b + 1] - q0;
  const int nrows = qlen * G;
  const int W0 = blockIdx.y * 128;
  if (W0 >= nrows) return;
  const int ctx = clamp_ctx(a, b);
  const int pos_base = ctx - qlen;
  const int n_pages = (ctx + kPage - 1) / kPage;
  const float sc = a.scale * kLog2e;

  const int R = W0 + 32 * wave + col;  // this lane's query row
  const bool row_ok = R < nrows;
  const int qpos = pos_base + R / G;
  const int64_t qrow = static_cast<int64_t>(q0 + (row_ok ? R / G : 0)) * Hq + g * G + R % G;
  bf16x8 qf[D / 16], dof[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(a.q + qrow * D + ks * 16 + half * 8);
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(a.dout + qrow * D + ks * 16 + half * 8);
    qf[ks] = row_ok ? x : bf16x8{};
    dof[ks] = row_ok ? y : bf16x8{};
  }
  const int64_t rowbase = (static_cast<int64_t>(g) * B + b) * a.lpad;
  const float l2 = row_ok ? a.lse2[rowbase + R] : 0.f;
  const float dl = row_ok ? a.delta[rowbase + R] : 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const int t_last = min(W0 + 127, nrows - 1) / G;
  const int kmax = a.causal ? min(ctx, pos_base + t_last + 1) : ctx;
  const int n_kt = (kmax + kBT - 1) / kBT;
  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();
    for (int idx = tid; idx < kBT * CPR; idx += 256) {  // K, V rows of keys 32kt + r
      const int r = idx / CPR, c = idx % CPR;
      const int32_t phys = page_id(a, b, 2 * kt + r / kPage, n_pages);
      u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (phys >= 0) {
        const int64_t off = (static_cast<int64_t>(phys) * Hkv + g) * (kPage * D) + (r % kPage) * D + c * 8;
        kv = *reinterpret_cast<const u32x4*>(a.k + off);
        vv = *reinterpret_cast<const u32x4*>(a.vtm + off);
      }
      *reinterpret_cast<u32x4*>(sm.k + row_pos<D>(r, c)) = kv;
      *reinterpret_cast<u32x4*>(sm.v + row_pos<D>(r, c)) = vv;
    }
    for (int idx = tid; idx < D * 4; idx += 256) {  // K^T of page c of the tile
      const int d = idx / 4, c = (idx / 2) % 2, e = idx % 2;
      const int32_t phys = page_id(a, b, 2 * kt + c, n_pages);
      u32x4 w = {0, 0, 0, 0};
      if (phys >= 0)
        w = *reinterpret_cast<const u32x4*>(a.kfm + (static_cast<int64_t>(phys) * Hkv + g) * (kPage * D) +
                                            d * kPage + e * 8);
      *reinterpret_cast<u32x4*>(sm.kt + col_pos<D>(d, c, e)) = w;
    }
    __syncthreads();

    // S^T and dP^T for (keys x this lane's row)
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(sm.k, col, 2 * ks + half), qf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(sm.v, col, 2 * ks + half), dof[ks], dp, 0, 0, 0);
    }
    float ds[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = kt * kBT + 8 * (v >> 2) + 4 * half + (v & 3);
      const bool vis = row_ok && key < ctx && (!a.causal || key <= qpos);
      const float p = vis ? fast_exp2(__builtin_fmaf(s[v], sc, -l2)) : 0.f;
      ds[v] = vis ? p * (dp[v] - dl) : 0.f;
    }
    // dQ^T += K^T dS^T  (contract the 32 keys)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 sb = rows_to_b(ds, c);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_read<D>(sm.kt, db * 32 + col, c, half), sb,
                                                          acc[db], 0, 0, 0);
    }
  }
  if (!row_ok) return;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int bq = 0; bq < 4; ++bq) {
      const f32x4 w = {acc[db][4 * bq] * a.scale, acc[db][4 * bq + 1] * a.scale,
                       acc[db][4 * bq + 2] * a.scale, acc[db][4 * bq + 3] * a.scale};
      *reinterpret_cast<f32x4*>(a.dq + qrow * D + db * 32 + 8 * bq + 4 * half) = w;
    }
}

template <int D>
hipError_t launch_backward_d(const BwdArgs& a, hipStream_t st) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int max_pages = (a.max_ctx_len + kPage - 1) / kPage;
  bwd_rows_kernel<D><<<dim3((a.lpad + 63) / 64, a.num_kv_heads, a.num_seqs), 256, 0, st>>>(a);
  bwd_pages_kernel<D><<<dim3(max_pages, a.num_kv_heads, a.num_seqs), 256, 0, st>>>(a);
  bwd_dkdv_kernel<D><<<dim3(a.num_seqs * a.num_kv_heads, (a.max_ctx_len + 127) / 128), 256, 0, st>>>(a);
  bwd_dq_kernel<D><<<dim3(a.num_seqs * a.num_kv_heads, (a.max_q_len * G + 127) / 128), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t st) {
  return a.head_dim == 64 ? launch_backward_d<64>(a, st) : launch_backward_d<128>(a, st);
}

}  // namespace pa
