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
#include <climits>

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

// Workgroups are dealt to the 8 dies (each with its own L2) round robin by
// linear id.  When the (sequence, KV head) pairs split evenly over the dies,
// die k takes pairs k*P .. k*P+P-1 with all their tiles (tile index y from 0,
// the longest first), so the workgroups of a pair share the die's L2.
__device__ __forceinline__ void die_task(int& pair, int& y) {
  const int n_pair = gridDim.x;
  pair = blockIdx.x;
  y = blockIdx.y;
  if (n_pair % 8 == 0) {
    const int lin = blockIdx.y * n_pair + blockIdx.x, P = n_pair / 8, j = lin / 8;
    pair = (lin % 8) * P + j % P;
    y = j / P;
  }
}

// ---------------------------------------------------------------------------
// Prep 1: per (sequence, KV head, 64 query rows): D = rowsum(dO * O), LSE *
// log2(e), and Q^T, dO^T into [Hkv][B][D][lpad] (rows past the sequence 0).
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
  // a feature pair (2 dp, 2 dp + 1) of 8 rows per lane: 8 four-byte LDS reads
  // give two 16-byte chunks of the transposed rows
  for (int idx = tid; idx < (D / 2) * 8; idx += 256) {
    const int dp = idx / 8, e = idx % 8;
    const int R = R0 + 8 * e;
    if (R >= a.lpad) continue;
    uint32_t q2[8], d2[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      q2[k] = *reinterpret_cast<const uint32_t*>(sq + (8 * e + k) * LD + 2 * dp);
      d2[k] = *reinterpret_cast<const uint32_t*>(sd + (8 * e + k) * LD + 2 * dp);
    }
    u32x4 q0, q1, w0, w1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      q0[k] = (q2[2 * k] & 0xffffu) | (q2[2 * k + 1] << 16);
      q1[k] = (q2[2 * k] >> 16) | (q2[2 * k + 1] & 0xffff0000u);
      w0[k] = (d2[2 * k] & 0xffffu) | (d2[2 * k + 1] << 16);
      w1[k] = (d2[2 * k] >> 16) | (d2[2 * k + 1] & 0xffff0000u);
    }
    const int64_t off = ((static_cast<int64_t>(g) * B + b) * D + 2 * dp) * a.lpad + R;
    *reinterpret_cast<u32x4*>(a.qt + off) = q0;
    *reinterpret_cast<u32x4*>(a.qt + off + a.lpad) = q1;
    *reinterpret_cast<u32x4*>(a.dot + off) = w0;
    *reinterpret_cast<u32x4*>(a.dot + off + a.lpad) = w1;
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
  // each lane reads a pair of features (or of slots) with 4-byte LDS reads
  // and writes the two transposed 16-byte chunks they hold
  auto split2 = [](const uint32_t (&x)[8], u32x4& lo, u32x4& hi) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo[k] = (x[2 * k] & 0xffffu) | (x[2 * k + 1] << 16);
      hi[k] = (x[2 * k] >> 16) | (x[2 * k + 1] & 0xffff0000u);
    }
  };
  for (int idx = tid; idx < D; idx += 256) {  // kfm chunks (features 2dp, 2dp+1; slots 8e..8e+7)
    const int dp = idx / 2, e = idx % 2;
    uint32_t x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = *reinterpret_cast<const uint32_t*>(sk + (e * 8 + k) * (D + 8) + 2 * dp);
    u32x4 w0, w1;
    split2(x, w0, w1);
    *reinterpret_cast<u32x4*>(a.kfm + chunk + (2 * dp) * kPage + e * 8) = w0;
    *reinterpret_cast<u32x4*>(a.kfm + chunk + (2 * dp + 1) * kPage + e * 8) = w1;
  }
  for (int idx = tid; idx < (kPage / 2) * CPR; idx += 256) {  // vtm chunks (slots 2sp, 2sp+1; features 8c..8c+7)
    const int sp = idx / CPR, c = idx % CPR;
    uint32_t x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = *reinterpret_cast<const uint32_t*>(sv + (c * 8 + k) * 24 + 2 * sp);
    u32x4 w0, w1;
    split2(x, w0, w1);
    *reinterpret_cast<u32x4*>(a.vtm + chunk + (2 * sp) * D + c * 8) = w0;
    *reinterpret_cast<u32x4*>(a.vtm + chunk + (2 * sp + 1) * D + c * 8) = w1;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (sequence, KV head, 32 * NW keys); wave w owns
// keys 32w..32w+31 of them, K and V of its keys held as MFMA operands.  The
// query tiles (32 rows) that see any of the keys are staged in LDS for all
// the waves: Q and dO row-major, Q^T and dO^T feature-major, D and
// LSE*log2(e).  Staging is by buffer loads straight into LDS (dma16) into two
// stages, so the next tile moves while one is multiplied: waves w and w + 4
// share operand tile w % 4 (their lanes' source offsets chosen so that the
// linear LDS writes land in the swizzled layout), waves 0 and 1 also move the
// row statistics.
template <int D>
struct RowsStage {
  uint16_t q[kBT * D], d[kBT * D], qt[kBT * D], dt[kBT * D];
  float lse2[256], delta[256];  // one 1 KiB load each; the first 32 floats used
};

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;
  constexpr int NI = kBT * D * 2 / 1024;  // 1 KiB loads per operand tile
  constexpr int KW = kBT * NW;            // keys per workgroup
  constexpr int NP = NW / 4;              // waves moving each operand tile
  static_assert(NW % 4 == 0 && NI % NP == 0, "operand tiles split evenly over the waves");
  // d = 128: V of the workgroup's keys in LDS, each lane keeping its own
  // key's operands there (written and read by that lane only), which leaves
  // the registers for two waves per SIMD; 8 waves (256 keys) share each staged
  // query tile, in two stages (132 KiB of LDS, one workgroup per CU).  d = 64
  // keeps V in registers.
  constexpr bool kVL = D == 128;
  constexpr int NS = 2;
  __shared__ RowsStage<D> sm[NS];
  __shared__ uint16_t vsm[kVL ? NW * kBT * D : 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv, B = a.num_seqs;
  int pair, y;
  die_task(pair, y);
  const int b = pair / Hkv, g = pair % Hkv;
  const int ctx = clamp_ctx(a, b);
  const int k0 = y * KW;
  if (k0 >= ctx) return;
  const int q0 = a.cu_q_lens[b], qlen = a.cu_q_lens[b + 1] - q0;
  const int nrows = qlen * G, pos_base = ctx - qlen;
  const int n_pages = (ctx + kPage - 1) / kPage;
  const float sc = a.scale * kLog2e;

  // this lane's key (its MFMA column) and the operands of the wave's keys
  const int key = k0 + 32 * wave + col;
  const int32_t phys = page_id(a, b, key / kPage, n_pages);
  bf16x8 kf[D / 16], vf[kVL ? 1 : D / 16];
  uint16_t* const vw = vsm + (kVL ? wave * (kBT * D) : 0);  // this wave's keys, row-tile layout
  {
    const int64_t base = (static_cast<int64_t>(phys < 0 ? 0 : phys) * Hkv + g) * (kPage * D) +
                         (key % kPage) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(a.k + base + ks * 16);
      bf16x8 y = *reinterpret_cast<const bf16x8*>(a.vtm + base + ks * 16);
      kf[ks] = phys < 0 ? bf16x8{} : x;
      if constexpr (kVL)
        *reinterpret_cast<bf16x8*>(vw + row_pos<D>(col, 2 * ks + half)) = phys < 0 ? bf16x8{} : y;
      else
        vf[ks] = phys < 0 ? bf16x8{} : y;
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

  // per-lane source offsets of this wave's loads (the same for every tile):
  // operand tile ot = wave % 4, its 1 KiB loads part * NI / NP onwards
  const int ot = wave % 4, part = wave / 4;
  constexpr int NL = NI / NP;
  uint32_t voff[NL];
#pragma unroll
  for (int il = 0; il < NL; ++il) {
    const int i = part * NL + il;
    const int m = i * 64 + lane;  // 16-byte slot of the operand tile
    if (ot < 2) {                 // row tile: slot m holds chunk pos of row r
      const int r = m / CPR, pos = m % CPR, j = pos ^ (r % CPR);
      voff[il] = static_cast<uint32_t>(((r / G) * Hq + (r % G)) * D * 2 + j * 16);
    } else {                      // col tile: half c, feature d, 8-row chunk
      const int c = m / (D * 2), w2 = m % (D * 2), d = w2 / 2, e = (w2 % 2) ^ ((d >> 3) & 1);
      voff[il] = static_cast<uint32_t>((d * a.lpad + 16 * c + 8 * e) * 2);
    }
  }
  const int64_t rowbase = (static_cast<int64_t>(g) * B + b) * a.lpad;
  const int64_t colbase = (static_cast<int64_t>(g) * B + b) * D * a.lpad;
  const int32_t col_bytes = ((D - 1) * a.lpad + kBT) * 2;
  auto stage_tile = [&](int it, int s) {
    const int R0 = it * kBT;
    RowsStage<D>& st = sm[s];
    const void* src;
    int32_t nb;
    uint32_t lds;
    if (ot < 2) {
      const int t0 = R0 / G;
      src = (ot == 0 ? a.q : a.dout) + (static_cast<int64_t>(q0 + t0) * Hq + g * G) * D;
      nb = max(0, min(qlen - t0, kBT / G)) * Hq * D * 2;  // the tile's tokens; past the sequence: 0
      lds = lds_address(ot == 0 ? st.q : st.d);
    } else {
      src = (ot == 2 ? a.qt : a.dot) + colbase + R0;
      nb = col_bytes;
      lds = lds_address(ot == 2 ? st.qt : st.dt);
    }
#pragma unroll
    for (int il = 0; il < NL; ++il) dma16(src, nb, voff[il], lds + (part * NL + il) * 1024);
    if (wave < 2)
      dma16((wave == 0 ? a.lse2 : a.delta) + rowbase + R0, kBT * 4, lane * 16,
            lds_address(wave == 0 ? st.lse2 : st.delta));
  };

  // query tiles that see a key of this workgroup (causal: from the token at
  // position k0 on), walked from the last one down: the workgroups of one
  // pair then read the same tiles at about the same time
  const int t_first = a.causal ? max(0, k0 - pos_base) : 0;
  const int tile0 = (t_first * G) / kBT, n_tiles = (nrows + kBT - 1) / kBT;
  // a query row R (token R / G) sees this lane's key when R >= lo_row
  const int lo_row = a.causal ? (key - pos_base) * G : INT_MIN;
  const bool key_ok = key < ctx;
  // this wave's first key; tiles wholly before it (causal) or a wave with no
  // key in the context skip the arithmetic and only stage
  const int wkey0 = k0 + kBT * wave;
  const int wave_lo_row = a.causal ? (wkey0 - pos_base) * G : INT_MIN;
  const bool wave_keys = wkey0 < ctx;
  if (tile0 < n_tiles) stage_tile(n_tiles - 1, 0);
  wait_vmcnt<0>();
  for (int it = n_tiles - 1; it >= tile0; --it) {
    const int R0 = it * kBT;
    const int s = (n_tiles - 1 - it) & 1;
    __syncthreads();  // tile it has landed; the stage of the tile before is free
    if (it > tile0) stage_tile(it - 1, s ^ 1);
    const RowsStage<D>& st = sm[s];
    if (!wave_keys || R0 + kBT - 1 < wave_lo_row) {
      wait_vmcnt<0>();
      continue;
    }

    // S and dP for (query rows x this lane's key)
    f32x16 sv = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(st.q, col, 2 * ks + half), kf[ks], sv, 0, 0, 0);
      bf16x8 vk;
      if constexpr (kVL)
        vk = row_read<D>(vw, col, 2 * ks + half);
      else
        vk = vf[ks];
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(st.d, col, 2 * ks + half), vk, dp, 0, 0, 0);
    }
    float p[16], ds[16];
    // one wave-uniform test: every (row, key) of the tile visible to every lane
    if (__all(key_ok & (R0 + kBT <= nrows) & (R0 >= lo_row))) {
#pragma unroll
      for (int bq = 0; bq < 4; ++bq) {
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(st.lse2 + 8 * bq + 4 * half);
        const f32x4 dl = *reinterpret_cast<const f32x4*>(st.delta + 8 * bq + 4 * half);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = 4 * bq + r;
          p[v] = fast_exp2(__builtin_fmaf(sv[v], sc, -l2[r]));
          ds[v] = p[v] * (dp[v] - dl[r]);
        }
      }
    } else {
#pragma unroll
      for (int bq = 0; bq < 4; ++bq) {
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(st.lse2 + 8 * bq + 4 * half);
        const f32x4 dl = *reinterpret_cast<const f32x4*>(st.delta + 8 * bq + 4 * half);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = 4 * bq + r, R = R0 + 8 * bq + 4 * half + r;
          const bool vis = key_ok & (R < nrows) & (R >= lo_row);
          p[v] = vis ? fast_exp2(__builtin_fmaf(sv[v], sc, -l2[r])) : 0.f;
          ds[v] = vis ? p[v] * (dp[v] - dl[r]) : 0.f;
        }
      }
    }
    // dV^T += dO^T P,  dK^T += Q^T dS  (contract the 32 query rows)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 pb = rows_to_b(p, c), sb = rows_to_b(ds, c);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = db * 32 + col;
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_read<D>(st.dt, d, c, half), pb, dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_read<D>(st.qt, d, c, half), sb, dk[db], 0, 0, 0);
      }
    }
    wait_vmcnt<0>();  // this wave's loads of the next tile are in LDS
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
// dQ: one workgroup per (sequence, KV head, 32 * NW query rows), wave w
// owning rows 32w..32w+31 with its Q and dO rows as MFMA operands; the key
// tiles (32 keys, two pages) it sees are staged in LDS, two stages deep: K
// and V token-major, K feature-major -- six page groups, the waves sharing
// their loads evenly.
template <int D>
struct KeysStage {
  uint16_t k[kBT * D], v[kBT * D], kt[kBT * D];
};

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_dq_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;
  constexpr int PER = kPage * D * 2 / 1024;  // 1 KiB loads per page group
  constexpr int RW = kBT * NW;               // query rows per workgroup
  __shared__ KeysStage<D> sm[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv, B = a.num_seqs;
  int pair, y;
  die_task(pair, y);
  const int b = pair / Hkv, g = pair % Hkv;
  const int q0 = a.cu_q_lens[b], qlen = a.cu_q_lens[b + 1] - q0;
  const int nrows = qlen * G;
  // row blocks from the last one down: under a causal mask the last rows see
  // the most keys, so the longest tasks start first
  const int W0 = (gridDim.y - 1 - y) * RW;
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

  // this wave's instructions of the six page groups: K page 0/1 and V page
  // 0/1 (row layout), K^T page 0/1 (col layout); PER instructions per group,
  // instruction u = i*NW + wave
  static_assert(6 * PER % NW == 0, "page groups split evenly over the waves");
  constexpr int NI = 6 * PER / NW;
  uint32_t voff[NI], ldso[NI];
  int grp[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int u = i * NW + wave, gr = u / PER, sub = u % PER;
    const int m = sub * 64 + lane, p = gr & 1;
    grp[i] = gr;
    if (gr < 4) {
      const int r1 = m / CPR, pos = m % CPR, r = 16 * p + r1, j = pos ^ (r % CPR);
      voff[i] = static_cast<uint32_t>(r1 * D * 2 + j * 16);
      ldso[i] = static_cast<uint32_t>((16 * p * CPR + m) * 16);
    } else {
      const int d = m / 2, e = (m % 2) ^ ((d >> 3) & 1);
      voff[i] = static_cast<uint32_t>((d * kPage + 8 * e) * 2);
      ldso[i] = static_cast<uint32_t>(p * D * 32 + m * 16);
    }
  }
  // page ids, 64 pages (32 key tiles) per lane vector, read out with readlane:
  // one table read per 32 tiles instead of one wait per tile
  int id_chunk = -1;
  int32_t idv = -1;
  auto page_at = [&](int pg) -> int32_t {
    if ((pg >> 6) != id_chunk) {
      id_chunk = pg >> 6;
      idv = page_id(a, b, 64 * id_chunk + lane, n_pages);
    }
    return __builtin_amdgcn_readlane(idv, pg & 63);
  };
  auto stage_tile = [&](int kt, int s) {
    int64_t chunk[2];
    int32_t nb[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int32_t ph = page_at(2 * kt + p);
      chunk[p] = (static_cast<int64_t>(ph < 0 ? 0 : ph) * Hkv + g) * (kPage * D);
      nb[p] = ph < 0 ? 0 : kPage * D * 2;
    }
    const uint32_t base_k = lds_address(sm[s].k), base_v = lds_address(sm[s].v),
                   base_t = lds_address(sm[s].kt);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int gr = grp[i], p = gr & 1;
      const uint16_t* src = gr < 2 ? a.k : (gr < 4 ? a.vtm : a.kfm);
      const uint32_t lb = gr < 2 ? base_k : (gr < 4 ? base_v : base_t);
      dma16(src + chunk[p], nb[p], voff[i], lb + ldso[i]);
    }
  };

  const int t_last = min(W0 + RW - 1, nrows - 1) / G;
  const int kmax = a.causal ? min(ctx, pos_base + t_last + 1) : ctx;
  const int n_kt = (kmax + kBT - 1) / kBT;
  if (n_kt > 0) stage_tile(0, 0);
  wait_vmcnt<0>();
  // the last key this lane's row sees (none when the row is past the sequence)
  const int key_lim = row_ok ? (a.causal ? min(qpos, ctx - 1) : ctx - 1) : -1;
  for (int kt = 0; kt < n_kt; ++kt) {
    const int s = kt & 1;
    __syncthreads();  // tile kt has landed; the stage of tile kt-1 is free
    if (kt + 1 < n_kt) stage_tile(kt + 1, s ^ 1);
    const KeysStage<D>& st = sm[s];
    if (__all(kt * kBT > key_lim)) {  // no key of the tile seen by a row of this wave
      wait_vmcnt<0>();
      continue;
    }

    // S^T and dP^T for (keys x this lane's row)
    f32x16 sv = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(st.k, col, 2 * ks + half), qf[ks], sv, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(st.v, col, 2 * ks + half), dof[ks], dp, 0, 0, 0);
    }
    float ds[16];
    // one wave-uniform test: every key of the tile visible to every lane's row
    if (__all(kt * kBT + kBT - 1 <= key_lim)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) ds[v] = fast_exp2(__builtin_fmaf(sv[v], sc, -l2)) * (dp[v] - dl);
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kt * kBT + 8 * (v >> 2) + 4 * half + (v & 3);
        const bool vis = key <= key_lim;
        const float p = vis ? fast_exp2(__builtin_fmaf(sv[v], sc, -l2)) : 0.f;
        ds[v] = vis ? p * (dp[v] - dl) : 0.f;
      }
    }
    // dQ^T += K^T dS^T  (contract the 32 keys)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 sb = rows_to_b(ds, c);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_read<D>(st.kt, db * 32 + col, c, half), sb,
                                                          acc[db], 0, 0, 0);
    }
    wait_vmcnt<0>();  // tile kt+1 is in LDS
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
  constexpr int NW = D == 128 ? 8 : 4;
  bwd_dkdv_kernel<D, NW><<<dim3(a.num_seqs * a.num_kv_heads, (a.max_ctx_len + 32 * NW - 1) / (32 * NW)),
                           64 * NW, 0, st>>>(a);
  bwd_dq_kernel<D, NW><<<dim3(a.num_seqs * a.num_kv_heads, (a.max_q_len * G + 32 * NW - 1) / (32 * NW)),
                         64 * NW, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t st) {
  return a.head_dim == 64 ? launch_backward_d<64>(a, st) : launch_backward_d<128>(a, st);
}

}  // namespace pa
