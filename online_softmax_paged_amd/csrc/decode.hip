// Split-KV decode: one query token per sequence against its paged K/V.
//
// Pass 1 (split kernel): workgroup = (page range s, KV head g, sequence b),
// four waves.  Each wave walks every fourth page of the range; per 16-token
// page it reads the K page and the V page straight from HBM into MFMA operand
// registers (16-byte / 8-byte loads), computes the scores of all the group's
// query heads at once on the matrix cores, and folds them into a running max,
// running sum and rescaled accumulator (the online softmax of the "core
// modules" chapter, section 2.1; deferred division as in FlashAttention-2).
// The four waves then combine through LDS and write one normalised partial
// output and logsumexp per query head (or the final result when there is a
// single range).
//
// Pass 2 (merge kernel): per (sequence, query head), combine the ranges by
// their logsumexps.
//
// Operand layouts (v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x16_bf16,
// lane l, c = l % 16, grp = l / 16):
//   scores S^T = K . Q^T : A = K rows (key c), B = Q^T columns (head c);
//                          D[4*grp + i][c] = score of key 4*grp+i, head c
//   O^T += V^T . P^T     : A = V^T rows (feature c), B = P^T (the lane's own
//                          4 scores, head c); D[4*grp + i][c] = O[head c][feat]
// so each lane keeps the softmax state of head c and no transpose is needed.
// Scores are kept in the log2 domain (scale * log2(e) folded in) and
// exponentiated with the hardware exp2.
#include <float.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
#ifndef PA_DECODE_RING
#define PA_DECODE_RING 2
#endif
// Pages in flight per wave.  Two pages keep the split kernel within 168
// VGPRs, so three workgroups fit per compute unit instead of two.  Measured
// (batched 32 x 128..2048 / long 8 x 32768 / fp8 mixed / 64 x 512, split
// heuristic of the time): 2 pages at 3 waves per SIMD 41.0 / 171.1 / 19.1 /
// 29.5 us; 3 pages at 2 waves per SIMD 42.8 / 172.4 / 19.5 / 30.8 us; 3 pages
// at 3 waves per SIMD 42.3 / 172.1 / 33.1 (fp8 spills) / 30.0 us; 4 and 5
// pages at 2 waves per SIMD no faster than 3.
constexpr int kRing = PA_DECODE_RING;

template <int D>
struct KVFrag {
  bf16x8 k[D / 32];  // A operand of the score MFMA, one per 32-feature step
  bf16x4 v[D / 16];  // A operand of the PV MFMA, one per 16-feature block
  float ks, vs;      // fp8 page scales
};

// Load one page's K and V operands for this lane.  phys outside
// [0, num_blocks) gives a zero-length buffer: the loads return zeros and read
// nothing, so callers can issue them unconditionally.  NT selects streaming
// (non-temporal) loads: right when the call reads far more K/V than the
// last-level cache holds (measured ~7% more bandwidth), wrong when pages are
// shared between sequences and could be served from cache.
template <int D, bool FP8, bool NT>
__device__ __forceinline__ void load_page(KVFrag<D>& f, const AttnArgs& a, int32_t phys, int g,
                                          int lane) {
  constexpr int kPol = NT ? kLoadNT : 0;
  constexpr int ES = FP8 ? 1 : 2;
  constexpr int BYTES = kPage * D * ES;
  const bool ok = phys >= 0 && phys < a.num_blocks;
  const int64_t chunk = ok ? static_cast<int64_t>(phys) * a.num_kv_heads + g : 0;
  const auto rk = make_rsrc(static_cast<const char*>(a.k) + chunk * BYTES, ok ? BYTES : 0);
  const auto rv = make_rsrc(static_cast<const char*>(a.v) + chunk * BYTES, ok ? BYTES : 0);
  const int c = lane & 15, grp = lane >> 4;
  if constexpr (!FP8) {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      f.k[ks] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, (c * D + ks * 32 + grp * 8) * ES, 0,
                                                        kPol));
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      f.v[db] = __builtin_bit_cast(
          bf16x4, __builtin_amdgcn_raw_buffer_load_b64(rv, ((db * 16 + c) * kPage + grp * 4) * ES,
                                                       0, kPol));
  } else {
    const auto rs = make_rsrc(a.k_scale, ok ? 4 * a.num_blocks : 0);
    const auto rt = make_rsrc(a.v_scale, ok ? 4 * a.num_blocks : 0);
    f.ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? phys * 4 : 0, 0, 0));
    f.vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rt, ok ? phys * 4 : 0, 0, 0));
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const u32x2 w = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, c * D + ks * 32 + grp * 8, 0, kPol));
      const u32x2 lo = fp8x4_to_bf16x4(w.x), hi = fp8x4_to_bf16x4(w.y);
      f.k[ks] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const uint32_t w = __builtin_bit_cast(
          uint32_t,
          __builtin_amdgcn_raw_buffer_load_b32(rv, (db * 16 + c) * kPage + grp * 4, 0, kPol));
      f.v[db] = __builtin_bit_cast(bf16x4, fp8x4_to_bf16x4(w));
    }
  }
}

__device__ __forceinline__ bool valid_block(int32_t phys, int32_t nb) {
  return phys >= 0 && phys < nb;
}

// Q^T operand of the score MFMA for sequence b's query heads g*G .. g*G+G-1:
// lane column c = head g*G + c (zero for c >= G), lane group grp = features
// ks*32 + grp*8 .. +7.
template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[D / 32], const AttnArgs& a, int b, int g,
                                       int G, int c, int grp) {
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                       (static_cast<int64_t>(b) * a.num_q_heads + g * G + (c < G ? c : 0)) * D;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + ks * 32 + grp * 8);
    if (c >= G) v = bf16x8{};
    qf[ks] = v;
  }
}

// One wave's online-softmax state over some pages of one (sequence, KV head),
// for the G query heads: lane column c = lane % 16 is head c; lane group grp =
// lane / 16 holds keys grp*4 .. grp*4+3 of every page and features
// db*16 + grp*4 + i of the accumulator.  m (log2 domain) is the same in the
// four groups; l is the group's share of the running sum.
template <int D>
struct DecodeState {
  float m = -INFINITY, l = 0.f;
  f32x4 acc[D / 16];
  __device__ __forceinline__ DecodeState() {
#pragma unroll
    for (int db = 0; db < D / 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// Fold page p of the sequence (keys 16p .. 16p+15; keys >= ctx masked), loaded
// in f, into the state.  sc = scale * log2(e).
template <int D, bool FP8>
__device__ __forceinline__ void fold_page(DecodeState<D>& st, KVFrag<D>& f,
                                          const bf16x8 (&qf)[D / 32], int p, int ctx, float sc,
                                          int grp) {
  f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k[ks], qf[ks], s4, 0, 0, 0);
  float scl = sc, vscl = 1.f;
  if constexpr (FP8) {
    scl *= f.ks;
    vscl = f.vs;
  }
  const int key0 = p * kPage + grp * 4;
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = (key0 + i < ctx) ? s4[i] * scl : -INFINITY;
  float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  mt = max_xor16(mt);
  mt = max_xor32(mt);
  const float m_new = fmaxf(st.m, mt);
  const float alpha = fast_exp2(st.m - m_new);
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(s[i] - m_new);
  st.l = st.l * alpha + (pr[0] + pr[1]) + (pr[2] + pr[3]);
  st.m = m_new;
  u32x2 pp;
  pp.x = pack_bf16x2(pr[0] * vscl, pr[1] * vscl);
  pp.y = pack_bf16x2(pr[2] * vscl, pr[3] * vscl);
  const bf16x4 pf = __builtin_bit_cast(bf16x4, pp);
  if (p * kPage + kPage > ctx) {
    // Last, partly filled page: slots past the context hold unspecified
    // bytes (possibly NaN); replace them so that 0 * NaN cannot occur.
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      u32x2 w = __builtin_bit_cast(u32x2, f.v[db]);
      if (key0 + 0 >= ctx) w.x &= 0xffff0000u;
      if (key0 + 1 >= ctx) w.x &= 0x0000ffffu;
      if (key0 + 2 >= ctx) w.y &= 0xffff0000u;
      if (key0 + 3 >= ctx) w.y &= 0x0000ffffu;
      f.v[db] = __builtin_bit_cast(bf16x4, w);
    }
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    st.acc[db] *= alpha;
    st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(i16x4, f.v[db]), __builtin_bit_cast(i16x4, pf), st.acc[db], 0, 0, 0);
  }
}

#ifndef PA_DECODE_WAVES_PER_EU
#define PA_DECODE_WAVES_PER_EU 3
#endif

template <int D, bool FP8, bool NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PA_DECODE_WAVES_PER_EU)))
void decode_split_kernel(AttnArgs a) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = lane & 15, grp = lane >> 4;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
  const int S = a.num_splits;
  // the q_len = 1 rows of a mixed batch: q row b is sequence b's query
  if (a.q_filter == kQOne && a.cu_q_lens[b + 1] - a.cu_q_lens[b] != 1) return;

  int ctx = a.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx_len ? a.max_ctx_len : ctx);
  const int n_pages = (ctx + kPage - 1) / kPage;
  const int max_pages = (a.max_ctx_len + kPage - 1) / kPage;
  // pages [key_begin / 16, max_pages) cut into S ranges
  const int pg0 = a.key_begin / kPage;
  const int pps = max(0, (max_pages - pg0 + S - 1) / S);
  const int p_begin = pg0 + split * pps;
  const int p_end = min(p_begin + pps, n_pages);

  bf16x8 qf[D / 32];
  load_q<D>(qf, a, b, g, G, c, grp);
  const float sc = a.scale * kLog2e;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.bt_stride;

  DecodeState<D> st;
  auto process = [&](KVFrag<D>& f, int p, bool valid) {
    if (valid) fold_page<D, FP8>(st, f, qf, p, ctx, sc, grp);
  };

  // This wave's pages are p_begin + wave + 4*i.  Their block ids are read up
  // front, one per lane (64 at a time), and three pages are kept in flight in
  // a register ring: while one is folded in, the next two are loading.  The
  // ids are read for the split's whole range without waiting for the context
  // length (entries past the sequence's last page are read, never used), and
  // ring slots past the last page load from an empty buffer (no traffic), so
  // every load is unconditional and the compiler can count those in flight.
  // The ids of the first 64 pages and the first three pages are requested
  // before the context length arrives, so the first data waits for two
  // dependent reads (table, page) rather than three.
  const int first = p_begin + wave;
  const int range_end = min(p_begin + pps, max_pages);
  const int n_spec = first < range_end ? (range_end - first + kWaves - 1) / kWaves : 0;
  const int32_t id0 = lane < min(64, n_spec) ? bt[first + kWaves * lane] : -1;
  KVFrag<D> ring[kRing];
  {
    auto spec_at = [&](int i) -> int32_t {
      return i < n_spec ? __builtin_amdgcn_readlane(id0, i) : -1;
    };
#pragma unroll
    for (int r = 0; r < kRing; ++r) load_page<D, FP8, NT>(ring[r], a, spec_at(r), g, lane);
  }
  const int n_mine = first < p_end ? (p_end - first + kWaves - 1) / kWaves : 0;
  for (int i0 = 0; i0 < n_mine; i0 += 64) {
    const int n = min(64, n_mine - i0);
    int32_t my_id = i0 == 0 ? id0
                            : (lane < min(64, n_spec - i0) ? bt[first + kWaves * (i0 + lane)] : -1);
    my_id = lane < n ? my_id : -1;
    auto id_at = [&](int i) -> int32_t {
      return i < n ? __builtin_amdgcn_readlane(my_id, min(i, 63)) : -1;
    };
    if (i0 > 0) {
#pragma unroll
      for (int r = 0; r < kRing; ++r) load_page<D, FP8, NT>(ring[r], a, id_at(r), g, lane);
    }
    for (int i = 0; i < n; i += kRing) {
      const int pa_ = first + kWaves * (i0 + i);
#pragma unroll
      for (int r = 0; r < kRing; ++r) {
        process(ring[r], pa_ + r * kWaves, valid_block(id_at(i + r), a.num_blocks));
        load_page<D, FP8, NT>(ring[r], a, id_at(i + r + kRing), g, lane);
      }
    }
  }

  // Row sums: each lane group holds a quarter of the keys of head c.
  const float l = sum_xor32(sum_xor16(st.l));

  __shared__ float sm_m[kWaves][16], sm_l[kWaves][16];
  __shared__ float sm_o[kWaves][D][17];
  if (grp == 0) {
    sm_m[wave][c] = st.m;
    sm_l[wave][c] = l;
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[wave][db * 16 + grp * 4 + i][c] = st.acc[db][i];
  __syncthreads();

  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int hd = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][hd]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm_m[w][hd];
        if (mw != -INFINITY) {
          const float f = fast_exp2(mw - M);
          L += sm_l[w][hd] * f;
          O += sm_o[w][d][hd] * f;
        }
      }
    }
    const bool empty = !(L > 0.f);
    const float out = empty ? 0.f : O / L;
    const float lse = empty ? -INFINITY : (M + __log2f(L)) * kLn2;
    const int64_t row = static_cast<int64_t>(b) * Hq + g * G + hd;
    if (a.ws_o == nullptr) {
      static_cast<uint16_t*>(a.o)[row * D + d] = to_bf16_bits(out);
      if (d == 0 && a.lse) a.lse[row] = lse;
    } else if (a.part_rows > 0) {
      // partial rows laid out as the prefill's, sequence b being token b
      if (b >= a.part_rows) continue;
      const int64_t prow = static_cast<int64_t>(a.split_base + split) * a.part_rows * Hq + row;
      a.ws_o[prow * D + d] = out;
      if (d == 0) a.ws_lse[prow] = lse;
    } else {
      a.ws_o[(row * S + split) * D + d] = out;
      if (d == 0) a.ws_lse[row * S + split] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// Balanced decode.  For one KV head, the pages of all sequences taken in order
// (sequence 0's, then sequence 1's, ...) form one list of N pages, cut into
// U = 4 * gridDim.x equal chunks of ppw = ceil(N / U) pages, one per wave.  A
// chunk may hold the end of one sequence and the start of the next, so every
// wave does the same amount of work whatever the mix of lengths.  A wave folds
// each sequence it meets separately: a sequence that lies inside one chunk is
// finished there (output row and logsumexp written directly); otherwise each
// chunk that meets it writes a normalised partial, into slot chunk + sequence
// of the KV head's U + B slots (unique: a chunk meeting sequence b+1 has
// passed sequence b), and decode_bal_merge_kernel combines them.
// Pages are counted from key_begin / 16 (the shared-prefix suffix pass).

// Pages of sequence b past key_begin (0 when the sequence is shorter).
__device__ __forceinline__ int bal_pages(const AttnArgs& a, int b, int pg0) {
  int ctx = a.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx_len ? a.max_ctx_len : ctx);
  return max(0, (ctx + kPage - 1) / kPage - pg0);
}

// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    x += lane >= o ? y : 0;
  }
  return x;
}

// Pages per chunk, from the total page count of all sequences.  The first
// 64 sequences' counts are returned in n0 (lane j: sequence j).
__device__ __forceinline__ int bal_chunk_pages(const AttnArgs& a, int U, int pg0, int lane,
                                               int& n0) {
  int N = 0;
  n0 = 0;
  for (int k0 = 0; k0 < a.num_seqs; k0 += 64) {
    const int n = k0 + lane < a.num_seqs ? bal_pages(a, k0 + lane, pg0) : 0;
    if (k0 == 0) n0 = n;
    N += wave_sum_i32(n);
  }
  N = __builtin_amdgcn_readfirstlane(N);
  return (N + U - 1) / U;
}

template <int D, bool FP8, bool NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PA_DECODE_WAVES_PER_EU)))
void decode_bal_kernel(AttnArgs a) {
  const int g = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = lane & 15, grp = lane >> 4;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv, B = a.num_seqs;
  const int U = gridDim.x * kWaves, u = blockIdx.x * kWaves + wave;
  const int pg0 = a.key_begin / kPage;
  const float sc = a.scale * kLog2e;

  int n0;
  const int ppw = bal_chunk_pages(a, U, pg0, lane, n0);
  if (ppw == 0) return;
  const int c0 = u * ppw, c1 = c0 + ppw;  // this wave's chunk [c0, c1) of the page list

  int base = 0;  // pages of the sequences before k0
  for (int k0 = 0; k0 < B; k0 += 64) {
    if (base >= c1) break;
    const int n = k0 == 0 ? n0 : (k0 + lane < B ? bal_pages(a, k0 + lane, pg0) : 0);
    const int incl = wave_incl_scan(n, lane), excl = incl - n;
    // sequences of this block that overlap the chunk
    uint64_t meet = __ballot(n > 0 && base + excl < c1 && base + incl > c0);
    while (meet) {
      const int j = __builtin_ctzll(meet);
      meet &= meet - 1;
      const int b = k0 + j;
      const int sb = base + __builtin_amdgcn_readlane(excl, j);
      const int nb = __builtin_amdgcn_readlane(n, j);
      const int lp0 = max(c0, sb) - sb, lp1 = min(c1, sb + nb) - sb;
      const bool whole = sb / ppw == (sb + nb - 1) / ppw;
      int ctx = a.ctx_lens[b];
      ctx = ctx < 0 ? 0 : (ctx > a.max_ctx_len ? a.max_ctx_len : ctx);

      bf16x8 qf[D / 32];
      load_q<D>(qf, a, b, g, G, c, grp);
      DecodeState<D> st;
      const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.bt_stride + pg0 + lp0;
      KVFrag<D> ring[kRing];
      for (int i0 = 0; i0 < lp1 - lp0; i0 += 64) {
        const int np = min(64, lp1 - lp0 - i0);
        const int32_t my_id = lane < np ? bt[i0 + lane] : -1;
        auto id_at = [&](int i) -> int32_t {
          return i < np ? __builtin_amdgcn_readlane(my_id, min(i, 63)) : -1;
        };
#pragma unroll
        for (int r = 0; r < kRing; ++r) load_page<D, FP8, NT>(ring[r], a, id_at(r), g, lane);
        for (int i = 0; i < np; i += kRing) {
#pragma unroll
          for (int r = 0; r < kRing; ++r) {
            if (valid_block(id_at(i + r), a.num_blocks))
              fold_page<D, FP8>(st, ring[r], qf, pg0 + lp0 + i0 + i + r, ctx, sc, grp);
            load_page<D, FP8, NT>(ring[r], a, id_at(i + r + kRing), g, lane);
          }
        }
      }

      const float l = sum_xor32(sum_xor16(st.l));
      const bool empty = !(l > 0.f);
      const float inv = empty ? 0.f : 1.f / l;
      const float lse = empty ? -INFINITY : (st.m + __log2f(l)) * kLn2;
      if (c < G) {
        const int64_t row = static_cast<int64_t>(b) * Hq + g * G + c;
        if (whole) {
          uint16_t* op = static_cast<uint16_t*>(a.o) + row * D + grp * 4;
#pragma unroll
          for (int db = 0; db < D / 16; ++db) {
            u32x2 w;
            w.x = pack_bf16x2(st.acc[db][0] * inv, st.acc[db][1] * inv);
            w.y = pack_bf16x2(st.acc[db][2] * inv, st.acc[db][3] * inv);
            *reinterpret_cast<u32x2*>(op + db * 16) = w;
          }
          if (grp == 0 && a.lse) a.lse[row] = lse;
        } else {
          const int64_t prow = (static_cast<int64_t>(g) * (U + B) + u + b) * G + c;
          float* op = a.ws_o + prow * D + grp * 4;
#pragma unroll
          for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4*>(op + db * 16) = st.acc[db] * inv;
          if (grp == 0) a.ws_lse[prow] = lse;
        }
      }
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
}

// Merge of the balanced decode's partials: one wave per (sequence, query
// head).  Sequences that lie inside one chunk were finished by the decode
// kernel; a sequence with no pages gets a zero row and lse = -inf.
template <int D>
__global__ __launch_bounds__(256) void decode_bal_merge_kernel(AttnArgs a, int U) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv, B = a.num_seqs;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  if (row >= static_cast<int64_t>(B) * Hq) return;
  const int b = static_cast<int>(row / Hq), h = static_cast<int>(row % Hq);
  const int g = h / G, c = h % G;
  const int pg0 = a.key_begin / kPage;
  int n0;
  const int ppw = bal_chunk_pages(a, U, pg0, lane, n0);
  // first page sb and page count nb of sequence b in the list
  int sb = 0, nb = 0;
  for (int k0 = 0; k0 < B; k0 += 64) {
    const int n = k0 == 0 ? n0 : (k0 + lane < B ? bal_pages(a, k0 + lane, pg0) : 0);
    if (b < k0 + 64) {
      const int j = b - k0;
      sb += wave_sum_i32(lane < j ? n : 0);
      nb = __builtin_amdgcn_readlane(n, j);
      break;
    }
    sb += wave_sum_i32(n);
  }
  constexpr int NPL = D / 64;
  uint16_t* orow = static_cast<uint16_t*>(a.o) + row * D + lane;
  if (nb == 0) {
#pragma unroll
    for (int j = 0; j < NPL; ++j) orow[64 * j] = 0;
    if (lane == 0 && a.lse) a.lse[row] = -INFINITY;
    return;
  }
  const int u0 = sb / ppw, u1 = (sb + nb - 1) / ppw;
  if (u0 == u1) return;
  const int S = u1 - u0 + 1;
  const int64_t p0 = (static_cast<int64_t>(g) * (U + B) + u0 + b) * G + c;  // slot u0 + b
  // partial s of this row: p0 + s * G
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, a.ws_lse[p0 + static_cast<int64_t>(s) * G]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float Mu = M == -INFINITY ? 0.f : M;
  float acc[NPL] = {};
  float W = 0.f;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int s = s0 + lane;
    const float lt = s < S ? a.ws_lse[p0 + static_cast<int64_t>(s) * G] : -INFINITY;
    const float w = lt == -INFINITY ? 0.f : fast_exp2((lt - Mu) * kLog2e);
    W += w;
    const int n = min(64, S - s0);
    const float* op = a.ws_o + (p0 + static_cast<int64_t>(s0) * G) * D + lane;
    const int wbits = __builtin_bit_cast(int, w);
    int k = 0;
    for (; k + 8 <= n; k += 8) {  // 8 partials' loads in flight at once
      float x[8][NPL];
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int j = 0; j < NPL; ++j) x[q][j] = op[static_cast<int64_t>(k + q) * G * D + 64 * j];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wbits, k + q));
#pragma unroll
        for (int j = 0; j < NPL; ++j) acc[j] += wk * x[q][j];
      }
    }
    for (; k < n; ++k) {
      const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wbits, k));
#pragma unroll
      for (int j = 0; j < NPL; ++j) acc[j] += wk * op[static_cast<int64_t>(k) * G * D + 64 * j];
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) W += __shfl_xor(W, o);
  const bool empty = !(W > 0.f);
  const float inv = empty ? 0.f : 1.f / W;
#pragma unroll
  for (int j = 0; j < NPL; ++j) orow[64 * j] = to_bf16_bits(acc[j] * inv);
  if (lane == 0 && a.lse) a.lse[row] = empty ? -INFINITY : M + __logf(W);
}

// fp32 pools: one wave per (query head, sequence, page range), 64 keys per
// step (see f32_attend).
template <int D>
__global__ __launch_bounds__(256) void decode_f32_kernel(AttnArgs a) {
  __shared__ float qs[kWaves][D];
  const int split = blockIdx.x, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y * kWaves + wave;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv, S = a.num_splits;
  if (h >= Hq) return;
  const int g = h / G;
  int ctx = a.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx_len ? a.max_ctx_len : ctx);
  const int max_pages = (a.max_ctx_len + kPage - 1) / kPage;
  const int pps = (max_pages + S - 1) / S;
  const int t_begin = split * pps * kPage;
  const int t_end = min(t_begin + pps * kPage, ctx);
  constexpr int NPL = D / 64;  // features per lane
  const int64_t row = static_cast<int64_t>(b) * Hq + h;
  const float* qp = static_cast<const float*>(a.q) + row * D;
  float o[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    qs[wave][lane + 64 * j] = qp[lane + 64 * j];
    o[j] = 0.f;
  }
  __builtin_amdgcn_wave_barrier();
  float m = -INFINITY, l = 0.f;
  f32_attend<D>(a, a.block_table + static_cast<int64_t>(b) * a.bt_stride, g, qs[wave], t_begin,
                t_end, lane, o, m, l);
  const bool empty = !(l > 0.f);
  const float lse = empty ? -INFINITY : (m + __log2f(l)) * kLn2;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const float out = empty ? 0.f : o[j] / l;
    if (S == 1)
      static_cast<float*>(a.o)[row * D + lane + 64 * j] = out;
    else
      a.ws_o[(row * S + split) * D + lane + 64 * j] = out;
  }
  if (lane == 0) {
    if (S == 1) {
      if (a.lse) a.lse[row] = lse;
    } else {
      a.ws_lse[row * S + split] = lse;
    }
  }
}

// One wave per (sequence, query head): logsumexp-weighted sum of the ranges.
// The range weights are computed by the lanes in parallel (lane s holds range
// s, up to 64 per pass) and broadcast with readlane, so the partial outputs of
// all ranges are independent loads.  Empty ranges carry lse = -inf, weight 0
// and a zero partial output.
template <int D, typename OutT>
__global__ __launch_bounds__(256) void decode_merge_kernel(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  if (row >= rows) return;
  const int S = a.num_splits;
  const float* ls = a.ws_lse + row * S;
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, ls[s]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  constexpr int NPL = D / 64;
  float acc[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) acc[j] = 0.f;
  float W = 0.f;
  const float Mu = M == -INFINITY ? 0.f : M;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int s = s0 + lane;
    const float lsv = s < S ? ls[s] : -INFINITY;
    const float w = lsv == -INFINITY ? 0.f : fast_exp2((lsv - Mu) * kLog2e);
    W += w;
    const int n = min(64, S - s0);
    const float* op = a.ws_o + (row * S + s0) * D + lane;
    const int wbits = __builtin_bit_cast(int, w);
    int i = 0;
    for (; i + 8 <= n; i += 8) {  // 8 ranges' loads in flight at once
      float x[8][NPL];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < NPL; ++j) x[u][j] = op[(i + u) * D + 64 * j];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wbits, i + u));
#pragma unroll
        for (int j = 0; j < NPL; ++j) acc[j] += wi * x[u][j];
      }
    }
    for (; i < n; ++i) {
      const float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wbits, i));
#pragma unroll
      for (int j = 0; j < NPL; ++j) acc[j] += wi * op[i * D + 64 * j];
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) W += __shfl_xor(W, o);
  const bool empty = !(W > 0.f);
  const float inv = empty ? 0.f : 1.f / W;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const float out = acc[j] * inv;
    if constexpr (sizeof(OutT) == 2)
      static_cast<uint16_t*>(a.o)[row * D + lane + 64 * j] = to_bf16_bits(out);
    else
      static_cast<float*>(a.o)[row * D + lane + 64 * j] = out;
  }
  if (lane == 0 && a.lse) a.lse[row] = empty ? -INFINITY : M + __logf(W);
}

// The split pass of a bf16 or fp8 pool (partials, or the output when a has no
// workspace).
template <int D>
hipError_t launch_split_d(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(a.num_splits, a.num_kv_heads, a.num_seqs);
  // Stream (non-temporal loads) when the largest possible K/V read of the
  // call is well beyond the 256 MB last-level cache.
  const double es = a.kv_dtype == PA_FP8_E4M3 ? 1.0 : 2.0;
  const double max_bytes = 2.0 * es * D * a.num_kv_heads * static_cast<double>(a.num_seqs) *
                           (a.max_ctx_len - a.key_begin);
  const bool nt = max_bytes > 512.0 * (1 << 20);
  if (a.kv_dtype == PA_FP8_E4M3) {
    if (nt) decode_split_kernel<D, true, true><<<grid, 256, 0, st>>>(a);
    else decode_split_kernel<D, true, false><<<grid, 256, 0, st>>>(a);
  } else {
    if (nt) decode_split_kernel<D, false, true><<<grid, 256, 0, st>>>(a);
    else decode_split_kernel<D, false, false><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_balanced_d(const AttnArgs& a, hipStream_t st) {
  const int wgs = balanced_wgs(a.num_seqs, a.num_kv_heads, a.max_ctx_len, a.key_begin);
  const dim3 grid(wgs, a.num_kv_heads);
  const double es = a.kv_dtype == PA_FP8_E4M3 ? 1.0 : 2.0;
  const double max_bytes = 2.0 * es * D * a.num_kv_heads * static_cast<double>(a.num_seqs) *
                           (a.max_ctx_len - a.key_begin);
  const bool nt = max_bytes > 512.0 * (1 << 20);
  if (a.kv_dtype == PA_FP8_E4M3) {
    if (nt) decode_bal_kernel<D, true, true><<<grid, 256, 0, st>>>(a);
    else decode_bal_kernel<D, true, false><<<grid, 256, 0, st>>>(a);
  } else {
    if (nt) decode_bal_kernel<D, false, true><<<grid, 256, 0, st>>>(a);
    else decode_bal_kernel<D, false, false><<<grid, 256, 0, st>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  decode_bal_merge_kernel<D><<<static_cast<unsigned>((rows + kWaves - 1) / kWaves), 256, 0, st>>>(
      a, 4 * wgs);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const AttnArgs& a, hipStream_t st) {
  const int S = a.num_splits;
  if (S < 0) return launch_balanced_d<D>(a, st);
  hipError_t e;
  if (a.kv_dtype == PA_F32) {
    const dim3 grid(S, (a.num_q_heads + kWaves - 1) / kWaves, a.num_seqs);
    decode_f32_kernel<D><<<grid, 256, 0, st>>>(a);
    e = hipGetLastError();
  } else {
    e = launch_split_d<D>(a, st);
  }
  if (e != hipSuccess || S == 1) return e;
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  const unsigned blocks = static_cast<unsigned>((rows + kWaves - 1) / kWaves);
  if (a.kv_dtype == PA_F32)
    decode_merge_kernel<D, float><<<blocks, 256, 0, st>>>(a);
  else
    decode_merge_kernel<D, uint16_t><<<blocks, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const AttnArgs& a, hipStream_t st) {
  return a.head_dim == 64 ? launch_decode_d<64>(a, st) : launch_decode_d<128>(a, st);
}

hipError_t launch_decode_split(const AttnArgs& a, hipStream_t st) {
  return a.head_dim == 64 ? launch_split_d<64>(a, st) : launch_split_d<128>(a, st);
}

}  // namespace pa
