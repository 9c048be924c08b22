// Causal (or full) prefill over the paged KV cache.
//
// FlashAttention-style tiling (survey page, section 2, core principle: Q in
// row blocks, K/V in column blocks, one block at a time on chip, combined
// through running max and exp-sum statistics; FlashAttention-2's deferred
// division and parallelism over the sequence).  Here:
//
//  * Workgroup = 4 waves = 128 query rows of one KV head group: 128/G query
//    tokens times the G query heads that share KV head g (grouped-query
//    packing, so every K/V tile read from HBM serves all G heads).
//  * K/V tiles of 32 keys = two 16-token physical pages, found through the
//    block table, staged in LDS (double-buffered: the next tile's global loads
//    are in flight while the current one is multiplied).
//  * Per wave, v_mfma_f32_32x32x16_bf16 computes S^T = K . Q^T (keys x 32
//    queries; Q^T stays in registers for the whole kernel) so that each lane
//    owns one query column: its softmax state (m, l) and its column of
//    O^T = V^T . P^T need no cross-lane traffic except one swap with lane^32.
//  * fp8 pools are expanded to bf16 on the way into LDS (exact); the page's K
//    scale multiplies the score columns and its V scale the probabilities.
//  * Grid = (sequence x KV head, query tile) with tiles launched longest
//    first, so the long diagonal tiles start early and each (sequence, KV
//    head)'s tiles spread over all dies while their K/V stays L2-resident.
#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kRows = 128;   // query rows per workgroup
constexpr int kKeys = 32;    // keys per tile (2 pages)

template <int D>
struct Smem {
  static constexpr int KS = D + 8;        // K row stride (bf16), 16 B pad
  static constexpr int VS = kKeys + 4;    // V^T row stride (bf16), 8 B pad
  uint16_t k[2][kKeys * KS];
  uint16_t vt[2][D * VS];
};

// The two physical pages of one 32-key tile (uniform across the workgroup),
// looked up two tiles ahead so the block-table read latency stays hidden.
struct TilePages {
  int32_t phys[2];
  bool ok[2];        // page holds keys of this sequence and its id is valid
  float ks[2], vs[2];  // fp8 page scales (1 for other pools)
};

template <bool FP8>
__device__ __forceinline__ TilePages pages_of(const AttnArgs& a, const int32_t* bt, int t,
                                              int n_pages) {
  TilePages tp;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int pidx = 2 * t + j;
    int32_t phys = pidx < n_pages ? bt[pidx] : -1;
    phys = __builtin_amdgcn_readfirstlane(phys);
    const bool ok = phys >= 0 && phys < a.num_blocks;
    tp.phys[j] = phys;
    tp.ok[j] = ok;
    tp.ks[j] = 1.f;
    tp.vs[j] = 1.f;
    if constexpr (FP8) {
      tp.ks[j] = ok ? a.k_scale[phys] : 0.f;
      tp.vs[j] = ok ? a.v_scale[phys] : 0.f;
    }
  }
  return tp;
}

// Global -> register staging of one 32-key tile: each thread moves 16-byte
// chunks of the two K pages and the two V pages.  Which page a chunk belongs
// to is uniform per wave, so the page checks are scalar branches.
template <int D, bool FP8>
struct Stage {
  static constexpr int CPP = FP8 ? kPage * D / 16 : kPage * D / 8;  // chunks per page
  static constexpr int KCH = (2 * CPP + 255) / 256;
  u32x4 k[KCH];
  u32x4 v[KCH];
};

template <int D, bool FP8>
__device__ __forceinline__ void stage_load(Stage<D, FP8>& st, const AttnArgs& a, int g,
                                           const TilePages& tp, int tid) {
  constexpr int CPP = Stage<D, FP8>::CPP;
  constexpr int ES = FP8 ? 16 : 8;  // elements per chunk
#pragma unroll
  for (int r = 0; r < Stage<D, FP8>::KCH; ++r) {
    const int e = min(r * 256 + tid, 2 * CPP - 1);
    const int pg = e / CPP, within = e % CPP;
    // Loads are unconditional so they stay in flight across the tile's math;
    // a page that is not part of the sequence reads physical page 0 instead
    // (always a valid address) and is zeroed when stored to LDS.
    const bool ok = pg ? tp.ok[1] : tp.ok[0];
    const int32_t phys = ok ? (pg ? tp.phys[1] : tp.phys[0]) : 0;
    const int64_t base = (static_cast<int64_t>(phys) * a.num_kv_heads + g) * (kPage * D);
    if constexpr (FP8) {
      st.k[r] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.k) + base + within * ES);
      st.v[r] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.v) + base + within * ES);
    } else {
      st.k[r] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.k) + base + within * ES);
      st.v[r] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.v) + base + within * ES);
    }
  }
}

__device__ __forceinline__ uint32_t zero_lo_hi(uint32_t w, bool lo_dead, bool hi_dead) {
  if (lo_dead) w &= 0xffff0000u;
  if (hi_dead) w &= 0x0000ffffu;
  return w;
}

// Register -> LDS without any masking (tile fully inside the context).
template <int D, bool FP8>
__device__ __forceinline__ void stage_store_plain(const Stage<D, FP8>& st, Smem<D>& sm, int buf,
                                                  int tid) {
  constexpr int KS = Smem<D>::KS, VS = Smem<D>::VS;
  constexpr int CPP = Stage<D, FP8>::CPP;
#pragma unroll
  for (int r = 0; r < Stage<D, FP8>::KCH; ++r) {
    const int e = r * 256 + tid;
    if (e >= 2 * CPP) break;
    const int pg = e / CPP, within = e % CPP;
    if constexpr (!FP8) {
      const int tk = within / (D / 8), dc = within % (D / 8);
      *reinterpret_cast<u32x4*>(&sm.k[buf][(pg * kPage + tk) * KS + dc * 8]) = st.k[r];
      const int d = within >> 1, hf = within & 1;
      uint16_t* dst = &sm.vt[buf][d * VS + pg * kPage + hf * 8];
      *reinterpret_cast<u32x2*>(dst) = u32x2{st.v[r].x, st.v[r].y};
      *reinterpret_cast<u32x2*>(dst + 4) = u32x2{st.v[r].z, st.v[r].w};
    } else {
      const int tk = within / (D / 16), dc = within % (D / 16);
      const u32x4 kw = st.k[r];
      const u32x2 k0 = fp8x4_to_bf16x4(kw.x), k1 = fp8x4_to_bf16x4(kw.y);
      const u32x2 k2 = fp8x4_to_bf16x4(kw.z), k3 = fp8x4_to_bf16x4(kw.w);
      uint16_t* kd = &sm.k[buf][(pg * kPage + tk) * KS + dc * 16];
      *reinterpret_cast<u32x4*>(kd) = u32x4{k0.x, k0.y, k1.x, k1.y};
      *reinterpret_cast<u32x4*>(kd + 8) = u32x4{k2.x, k2.y, k3.x, k3.y};
      const u32x4 vw = st.v[r];
      uint16_t* vd = &sm.vt[buf][within * VS + pg * kPage];
      *reinterpret_cast<u32x2*>(vd) = fp8x4_to_bf16x4(vw.x);
      *reinterpret_cast<u32x2*>(vd + 4) = fp8x4_to_bf16x4(vw.y);
      *reinterpret_cast<u32x2*>(vd + 8) = fp8x4_to_bf16x4(vw.z);
      *reinterpret_cast<u32x2*>(vd + 12) = fp8x4_to_bf16x4(vw.w);
    }
  }
}

// Register -> LDS.  Slots at or past the context end are written as zeros so
// that unspecified pool bytes (possibly NaN) never meet a zero probability.
template <int D, bool FP8>
__device__ __forceinline__ void stage_store(const Stage<D, FP8>& st, Smem<D>& sm, int buf, int kt,
                                            int ctx, const TilePages& tp, int tid) {
  // Common case: both pages are whole and inside the context; no masking.
  if (tp.ok[0] && tp.ok[1] && (kt + 1) * kKeys <= ctx) {
    stage_store_plain<D, FP8>(st, sm, buf, tid);
    return;
  }
  constexpr int KS = Smem<D>::KS, VS = Smem<D>::VS;
  constexpr int CPP = Stage<D, FP8>::CPP;
#pragma unroll
  for (int r = 0; r < Stage<D, FP8>::KCH; ++r) {
    const int e = r * 256 + tid;
    if (e >= 2 * CPP) break;
    const int pg = e / CPP, within = e % CPP;
    // first token of this page; a page that is not part of the sequence is
    // treated as lying past the context end, so all of it is zeroed
    const int page_tok = (pg ? tp.ok[1] : tp.ok[0]) ? kt * kKeys + pg * kPage : ctx;
    if constexpr (!FP8) {
      // K chunk: token within / (D/8), features (within % (D/8)) * 8
      const int tk = within / (D / 8), dc = within % (D / 8);
      const int key = pg * kPage + tk;
      u32x4 kv = st.k[r];
      if (page_tok + tk >= ctx) kv = u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(&sm.k[buf][key * KS + dc * 8]) = kv;
      // V^T chunk: feature within / 2, tokens (within % 2) * 8 .. + 8
      const int d = within >> 1, hf = within & 1;
      const int t0 = page_tok + hf * 8;
      u32x4 vv = st.v[r];
      if (t0 + 8 > ctx) {
        vv.x = zero_lo_hi(vv.x, t0 + 0 >= ctx, t0 + 1 >= ctx);
        vv.y = zero_lo_hi(vv.y, t0 + 2 >= ctx, t0 + 3 >= ctx);
        vv.z = zero_lo_hi(vv.z, t0 + 4 >= ctx, t0 + 5 >= ctx);
        vv.w = zero_lo_hi(vv.w, t0 + 6 >= ctx, t0 + 7 >= ctx);
      }
      uint16_t* dst = &sm.vt[buf][d * VS + pg * kPage + hf * 8];
      *reinterpret_cast<u32x2*>(dst) = u32x2{vv.x, vv.y};
      *reinterpret_cast<u32x2*>(dst + 4) = u32x2{vv.z, vv.w};
    } else {
      // K chunk: 16 features of one token
      const int tk = within / (D / 16), dc = within % (D / 16);
      const int key = pg * kPage + tk;
      const u32x4 kw = st.k[r];
      u32x2 k0 = fp8x4_to_bf16x4(kw.x), k1 = fp8x4_to_bf16x4(kw.y);
      u32x2 k2 = fp8x4_to_bf16x4(kw.z), k3 = fp8x4_to_bf16x4(kw.w);
      u32x4 ka = {k0.x, k0.y, k1.x, k1.y}, kb = {k2.x, k2.y, k3.x, k3.y};
      if (page_tok + tk >= ctx) ka = kb = u32x4{0, 0, 0, 0};
      uint16_t* kd = &sm.k[buf][key * KS + dc * 16];
      *reinterpret_cast<u32x4*>(kd) = ka;
      *reinterpret_cast<u32x4*>(kd + 8) = kb;
      // V^T chunk: all 16 tokens of one feature row
      const int d = within;
      const u32x4 vw = st.v[r];
      u32x2 w[4] = {fp8x4_to_bf16x4(vw.x), fp8x4_to_bf16x4(vw.y), fp8x4_to_bf16x4(vw.z),
                    fp8x4_to_bf16x4(vw.w)};
      if (page_tok + kPage > ctx) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          w[j].x = zero_lo_hi(w[j].x, page_tok + 4 * j + 0 >= ctx, page_tok + 4 * j + 1 >= ctx);
          w[j].y = zero_lo_hi(w[j].y, page_tok + 4 * j + 2 >= ctx, page_tok + 4 * j + 3 >= ctx);
        }
      }
      uint16_t* vd = &sm.vt[buf][d * VS + pg * kPage];
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2*>(vd + 4 * j) = w[j];
    }
  }
}

// Epilogue of one lane (query row qrow = token * Hq + head, its half of the
// features): without a workspace, the output row (bf16) and its logsumexp;
// with one, this split's normalised fp32 partial row and logsumexp at
// (split_base + split) * part_rows * Hq + qrow.
template <int D>
__device__ __forceinline__ void write_rows(const AttnArgs& a, const f32x16 (&acc)[D / 32],
                                           float m, float l, int64_t qrow, int split, int half) {
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.f / l;
  const float lse = empty ? -INFINITY : (m + __log2f(l)) * kLn2;
  if (a.ws_o == nullptr) {
    uint16_t* op = static_cast<uint16_t*>(a.o) + qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w.x = pack_bf16x2(acc[db][4 * j + 0] * inv, acc[db][4 * j + 1] * inv);
        w.y = pack_bf16x2(acc[db][4 * j + 2] * inv, acc[db][4 * j + 3] * inv);
        *reinterpret_cast<u32x2*>(op + db * 32 + 8 * j + 4 * half) = w;
      }
    if (half == 0 && a.lse) a.lse[qrow] = lse;
    return;
  }
  if (qrow >= a.part_rows * a.num_q_heads) return;  // token past the partials' rows
  const int64_t prow =
      static_cast<int64_t>(a.split_base + split) * a.part_rows * a.num_q_heads + qrow;
  float* op = a.ws_o + prow * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 w = {acc[db][4 * j + 0] * inv, acc[db][4 * j + 1] * inv,
                       acc[db][4 * j + 2] * inv, acc[db][4 * j + 3] * inv};
      *reinterpret_cast<f32x4*>(op + db * 32 + 8 * j + 4 * half) = w;
    }
  if (half == 0) a.ws_lse[prow] = lse;
}

template <int D, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void prefill_kernel(AttnArgs a, int n_tiles) {
  __shared__ Smem<D> sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
  const int bg = blockIdx.x;
  const int b = bg / Hkv, g = bg % Hkv;
  const int S = a.num_splits;
  const int tile = n_tiles - 1 - static_cast<int>(blockIdx.y) / S;
  const int split = static_cast<int>(blockIdx.y) % S;
  const int TQ = kRows / G;

  int q0 = 0, qlen = a.packed_q, ctx = a.max_ctx_len;
  if (a.packed_q == 0) {
    q0 = a.cu_q_lens[b];
    qlen = a.cu_q_lens[b + 1] - q0;
    ctx = a.ctx_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > a.max_ctx_len ? a.max_ctx_len : ctx);
  }
  const int t0 = tile * TQ;
  if (t0 >= qlen || (a.q_filter == kQMany && qlen == 1)) return;
  const int pos_base = ctx - qlen;            // position of query token 0
  const int t_last = min(t0 + TQ, qlen) - 1;  // last token of this tile
  // Inconsistent lengths (ctx = 0, or q_len > ctx) leave some or all rows
  // nothing to see: those rows still get O = 0 and LSE = -inf (or an empty
  // partial) from the epilogue, with no key tile visited.
  const int kmax = max(0, a.causal ? min(ctx, pos_base + t_last + 1) : ctx);
  const int n_kt_all = (kmax + kKeys - 1) / kKeys;
  // this split's key tiles [kt_begin, n_kt), from the tile holding key_begin
  const int kt_first = a.key_begin / kKeys;
  const int per_split = max(0, (n_kt_all - kt_first + S - 1) / S);
  const int kt_begin = kt_first + split * per_split;
  const int n_kt = min(n_kt_all, kt_begin + per_split);
  const int n_pages = (ctx + kPage - 1) / kPage;
  // Tiles whose keys are all visible to every row need no mask.
  const int first_pos = pos_base + t0;
  const int n_full = a.causal ? max(0, min((first_pos + 1) / kKeys, ctx / kKeys))
                              : ctx / kKeys;

  // This lane's query row, and the last key it may see.
  const int r = wave * 32 + col;
  const int tt = t0 + r / G, hg = r % G;
  const bool row_ok = tt < qlen;
  const int qpos = pos_base + tt;
  const int key_lim = a.causal ? min(qpos, ctx - 1) : ctx - 1;
  const int64_t qrow = static_cast<int64_t>(q0 + (row_ok ? tt : 0)) * Hq + g * G + hg;

  bf16x8 qf[D / 16];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + half * 8);
      qf[ks] = row_ok ? v : bf16x8{};
    }
  }

  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.bt_stride;
  const float sc = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f, mu = 0.f;  // mu: the max used in exponents (0 while m = -inf)
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  TilePages cur = pages_of<FP8>(a, bt, kt_begin, n_pages);
  TilePages nxt = pages_of<FP8>(a, bt, kt_begin + 1, n_pages);
  Stage<D, FP8> st;
  if (kt_begin < n_kt) {
    stage_load<D, FP8>(st, a, g, cur, tid);
    stage_store<D, FP8>(st, sm, 0, kt_begin, ctx, cur, tid);
  }
  __syncthreads();

  constexpr int KS = Smem<D>::KS, VS = Smem<D>::VS;
  for (int kt = kt_begin; kt < n_kt; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    const TilePages nn = pages_of<FP8>(a, bt, kt + 2, n_pages);
    if (kt + 1 < n_kt) stage_load<D, FP8>(st, a, g, nxt, tid);

    // S^T = K . Q^T  (32 keys x 32 queries)
    f32x16 s = {};
    const uint16_t* kb = &sm.k[buf][col * KS + half * 8];
    bf16x8 kf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kf[ks] = *reinterpret_cast<const bf16x8*>(kb + ks * 16);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
    // Score value i of this lane is key 8*(i/4) + 4*half + i%4 of the tile.
    // Raw scores (fp8: times the page's K scale); invisible keys -> -inf.
    float sv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = FP8 ? s[i] * (i < 8 ? cur.ks[0] : cur.ks[1]) : s[i];
    if (kt >= n_full) {
      const int lim = key_lim - kt * kKeys - 4 * half;
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[i] = 8 * (i >> 2) + (i & 3) <= lim ? sv[i] : -INFINITY;
    }
    if (kt * kKeys < a.key_begin) {  // key_begin % 32 == 16: the tile's first page is left out
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = -INFINITY;
    }
    float mt = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mt = fmaxf(fmaxf(mt, sv[i]), sv[i + 1]);
    mt = fmaxf(mt, sv[15]);
    mt = max_xor32(mt);
    const float mt_s = mt * sc;  // scaled, log2 domain (sc > 0 keeps -inf)
    // Lazy rescaling: the running max (and with it O and l) is only moved when
    // some row's tile max exceeds it by more than 8, so exponents stay <= 2^8
    // and the common case skips the O rescale; the final division by l makes
    // the result independent of which max was used.
    if (__any(mt_s > m + 8.f)) {
      const float m_new = fmaxf(m, mt_s);
      const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
      m = m_new;
      mu = m == -INFINITY ? 0.f : m;
    }
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = fast_exp2(__builtin_fmaf(sv[i], sc, -mu));
      psum += sv[i];
    }
    l += psum;

    // O^T += V^T . P^T ; chunk c covers page c of the tile (keys 16c..16c+15)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = FP8 ? sv[8 * c + i] * cur.vs[c] : sv[8 * c + i];
      u32x4 pw;
      pw.x = pack_bf16x2(pv[0], pv[1]);
      pw.y = pack_bf16x2(pv[2], pv[3]);
      pw.z = pack_bf16x2(pv[4], pv[5]);
      pw.w = pack_bf16x2(pv[6], pv[7]);
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t* vp = &sm.vt[buf][(db * 32 + col) * VS + c * kPage + half * 4];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 8);
        const u32x4 vw = {lo.x, lo.y, hi.x, hi.y};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pf,
                                                          acc[db], 0, 0, 0);
      }
    }
    if (kt + 1 < n_kt) stage_store<D, FP8>(st, sm, buf ^ 1, kt + 1, ctx, nxt, tid);
    __syncthreads();
    cur = nxt;
    nxt = nn;
  }

  l = sum_xor32(l);
  if (!row_ok) return;
  write_rows<D>(a, acc, m, l, qrow, split, half);
}

// ---------------------------------------------------------------------------
// bf16 pools: K/V tiles go from HBM straight into LDS (buffer loads with the
// LDS modifier; each wave instruction fills 1 KiB = 64 lanes x 16 B), so the
// staging needs no registers and no LDS store instructions.  Three LDS stages:
// tile kt+2 is loading while tile kt is multiplied.
//
// LDS layouts (16-byte chunks, swizzled so the MFMA operand reads are free of
// bank conflicts while each DMA instruction still writes 1 KiB contiguously):
//   K   [32 keys][D/8 chunks]: logical chunk j of key row r sits at j ^ (r % (D/8)).
//   V^T per page c: [D rows][2 chunks of 8 keys]: chunk e of row d sits at
//       e ^ ((d / 8) % 2).
// The P.V product reads V^T chunks of 8 consecutive keys (one ds_read_b128),
// so the P operand is rearranged with two v_permlane32_swap per page to the
// same key order.
// Tail handling: pages outside the sequence and K rows past the context end
// come from a shortened buffer range (zero-filled by the hardware); V^T slots
// past the context end of the last page are zeroed in LDS before use.

// Block ids of one tile, read raw (clamped index, no checks) so nothing waits
// on the load until the ids are used an iteration later.
// Pairs a die runs interleaved: all of them up to 8, else the largest power
// of two up to 8 that divides their count.
__device__ __forceinline__ int pair_group(int P) {
  return P <= 8 ? P : ((P % 8 == 0) ? 8 : ((P % 4 == 0) ? 4 : ((P % 2 == 0) ? 2 : 1)));
}

template <int D>
struct DmaSmem {
  static constexpr int KB = kKeys * D * 2;      // K tile bytes
  static constexpr int VB = kKeys * D * 2;      // V^T tile bytes (2 pages)
  static constexpr int STAGE = KB + VB;
  char buf[3 * STAGE];
};


// The DMA instructions of one tile form four groups of D/32 (1 KiB each):
// K page 0, K page 1, V^T page 0, V^T page 1.  Instruction u = i*NW + wave
// is this wave's i-th.  Its lane offset inside the page chunk and its LDS
// offset inside a stage are the same for every tile, so they are computed
// once; per tile only the two page addresses and valid lengths change.
template <int D, int NW>
struct DmaPlan {
  static constexpr int PER = D / 32;              // instructions per group
  static constexpr int TOT = 4 * PER;             // instructions per tile
  static constexpr int NI = (TOT + NW - 1) / NW;  // instructions per wave
  uint32_t voff[NI];
  int group[NI];
  int lds[NI];
  int count;

  __device__ __forceinline__ DmaPlan(int wave, int lane) {
    constexpr int CPR = D / 8;  // 16-byte chunks per K row
    constexpr int PAGE_BYTES = kPage * D * 2;
    count = 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int u = i * NW + wave;
      // with PER == NW the group of instruction i does not depend on the wave
      const int grp = (PER == NW) ? i : u / PER;
      const int sub = (PER == NW) ? wave : u % PER;
      const int m = sub * 64 + lane;  // 16-byte slot inside the group's LDS region
      uint32_t vo;
      if (grp < 2) {
        // K row rr of page grp, LDS position pos holds logical chunk pos ^ (row % CPR)
        const int rr = m / CPR, pos = m % CPR;
        vo = (rr * CPR + (pos ^ ((grp * kPage + rr) % CPR))) * 16;
      } else {
        // V^T row d of the page: slot e' holds keys 8e..8e+7, e = e' ^ ((d / 8) % 2)
        const int d = m >> 1, e = (m & 1) ^ ((d >> 3) & 1);
        vo = (d * 2 + e) * 16;
      }
      voff[i] = vo;
      group[i] = grp;
      lds[i] = grp * PAGE_BYTES + sub * 1024;
      count += u < TOT ? 1 : 0;
    }
  }
};


// One tile's DMA: off[j] is page j's (page, KV head) byte offset in the
// pools, knb[j] / vnb[j] the bytes of its K rows / V^T page to move (0 for an
// absent page; reads past them return zero).
template <int D, int NW>
__device__ __forceinline__ void dma_tile(const AttnArgs& a, const uint64_t (&off)[2],
                                         const int (&knb)[2], const int (&vnb)[2], uint32_t stage,
                                         const DmaPlan<D, NW>& plan) {
#pragma unroll
  for (int i = 0; i < DmaPlan<D, NW>::NI; ++i) {
    if (DmaPlan<D, NW>::NI * NW != DmaPlan<D, NW>::TOT && i >= plan.count) break;
    const int grp = plan.group[i];
    const bool is_v = grp >= 2, hi = grp & 1;
    const char* base = (is_v ? static_cast<const char*>(a.v) : static_cast<const char*>(a.k)) +
                       (hi ? off[1] : off[0]);
    const int nb = is_v ? (hi ? vnb[1] : vnb[0]) : (hi ? knb[1] : knb[0]);
    dma16(base, nb, plan.voff[i], stage + plan.lds[i]);
  }
}


// Same, for a wave-uniform count known only at run time (0..4).
[[maybe_unused]] __device__ __forceinline__ void wait_vmcnt_upto4(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    default: wait_vmcnt<4>(); break;
  }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW >= 8 ? 2 : 3)))
void prefill_dma_kernel(AttnArgs a, int n_tiles) {
  __shared__ DmaSmem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int krow = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);  // col, bits 2 and 3 swapped
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
  // Workgroups are dealt to the 8 dies (XCDs, each with its own 4 MB L2)
  // round robin by linear id.  When the (sequence, KV head) pairs split evenly
  // over the dies, die k takes pairs k*P .. k*P+P-1 and runs them in groups of
  // GP (all P of them up to 8), longest query tiles first across a group's
  // pairs, so every die ends on short tiles.  Measured at steady state, one
  // group of all 4 pairs per die beats groups of 2 by 1.3% on 4 x 4096 tokens
  // with 8 KV heads (groups of 1: 2.5% slower).
  // (With key splits, the task index along y is tile-from-end * S + split,
  // so a tile's splits stay together.)
  const int S = a.num_splits;
  const int n_bg = gridDim.x, n_y = gridDim.y;  // n_y = n_tiles * S
  const int lin = blockIdx.y * n_bg + blockIdx.x;
  int bg = blockIdx.x, y = blockIdx.y;
  if (n_bg % 8 == 0) {
    const int P = n_bg / 8, GP = pair_group(P);
    const int j = lin / 8, per_group = GP * n_y;
    const int grp = j / per_group, i = j % per_group;
    bg = (lin % 8) * P + grp * GP + i % GP;
    y = i / GP;
  }
  const int b = bg / Hkv, g = bg % Hkv;
  const int tile = n_tiles - 1 - y / S, split = y % S;
  constexpr int ROWS = 32 * NW;   // query rows per workgroup
  const int TQ = ROWS / G;
  constexpr int STAGE = DmaSmem<D>::STAGE;
  constexpr int CPR = D / 8;
  const DmaPlan<D, NW> plan(wave, lane);
  // wait until at most one tile's DMA of this wave is still in flight
  auto wait_own_dma = [&]() {
    if constexpr (DmaPlan<D, NW>::NI * NW == DmaPlan<D, NW>::TOT)
      wait_vmcnt<DmaPlan<D, NW>::NI>();
    else
      wait_vmcnt_upto4(plan.count);
  };

  int q0 = 0, qlen = a.packed_q, ctx = a.max_ctx_len;
  if (a.packed_q == 0) {
    q0 = a.cu_q_lens[b];
    qlen = a.cu_q_lens[b + 1] - q0;
    ctx = a.ctx_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > a.max_ctx_len ? a.max_ctx_len : ctx);
  }
  const int t0 = tile * TQ;
  if (t0 >= qlen || (a.q_filter == kQMany && qlen == 1)) return;
  const int pos_base = ctx - qlen;
  const int t_last = min(t0 + TQ, qlen) - 1;
  const int kmax = max(0, a.causal ? min(ctx, pos_base + t_last + 1) : ctx);  // 0: rows left empty
  const int n_kt_all = (kmax + kKeys - 1) / kKeys;
  // this split's key tiles [kt_begin, n_kt), from the tile holding key_begin
  const int kt_first = a.key_begin / kKeys;
  const int per_split = max(0, (n_kt_all - kt_first + S - 1) / S);
  const int kt_begin = kt_first + split * per_split;
  const int n_kt = min(n_kt_all, kt_begin + per_split);
  const int n_pages = (ctx + kPage - 1) / kPage;
  const int first_pos = pos_base + t0;
  const int n_full = a.causal ? max(0, min((first_pos + 1) / kKeys, ctx / kKeys))
                              : ctx / kKeys;
  // the tile holding the context end, if that end is not on a page boundary
  const int tail_tile = (ctx % kPage) ? (ctx - 1) / kKeys : -1;

  const int r = wave * 32 + col;
  const int tt = t0 + r / G, hg = r % G;
  const bool row_ok = tt < qlen;
  const int qpos = pos_base + tt;
  const int key_lim = a.causal ? min(qpos, ctx - 1) : ctx - 1;
  const int64_t qrow = static_cast<int64_t>(q0 + (row_ok ? tt : 0)) * Hq + g * G + hg;

  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.bt_stride;
  // 64 consecutive pages in lane vectors, refreshed every 32 tiles: each
  // lane holds its page's (page, KV head) byte offset in the pools and the
  // bytes of its K rows | V^T page << 16 to move (0 for an absent page), so a
  // tile's DMA arguments are register reads, not memory loads and products.
  constexpr int PAGE_BYTES = kPage * D * 2;
  int pg_chunk = -1;
  uint32_t po_lo = 0, po_hi = 0, pnb = 0;
  auto dma = [&](int t, uint32_t stage) {
    const int c = (2 * t) >> 6;  // a tile's two pages share a chunk
    if (c != pg_chunk) {         // uniform; at most once per 32 tiles
      pg_chunk = c;
      const int p = 64 * c + lane;
      const int32_t id = p < n_pages ? bt[p] : -1;
      const bool ok = id >= 0 && id < a.num_blocks;
      const uint64_t o = ok ? (static_cast<uint64_t>(id) * Hkv + g) * PAGE_BYTES : 0;
      const int nv = min(kPage, max(0, ctx - p * kPage));
      po_lo = static_cast<uint32_t>(o);
      po_hi = static_cast<uint32_t>(o >> 32);
      pnb = ok ? static_cast<uint32_t>(nv * D * 2) | (nv > 0 ? uint32_t(PAGE_BYTES) << 16 : 0u) : 0u;
      // consume the load here, so its wait stays inside this rare branch
      asm volatile("" ::"v"(po_lo), "v"(po_hi), "v"(pnb));
    }
    uint64_t off[2];
    int knb[2], vnb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = (2 * t + j) & 63;
      off[j] = (static_cast<uint64_t>(__builtin_amdgcn_readlane(po_hi, q)) << 32) |
               static_cast<uint32_t>(__builtin_amdgcn_readlane(po_lo, q));
      const uint32_t nb = __builtin_amdgcn_readlane(pnb, q);
      knb[j] = static_cast<int>(nb & 0xffffu);
      vnb[j] = static_cast<int>(nb >> 16);
    }
    dma_tile<D, NW>(a, off, knb, vnb, stage, plan);
  };
  const uint32_t lds0 = lds_address(sm.buf);
  if (kt_begin < n_kt) {  // uniform; an empty split moves nothing
    dma(kt_begin, lds0);
    dma(kt_begin + 1, lds0 + STAGE);
  }

  bf16x8 qf[D / 16];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + half * 8);
      qf[ks] = row_ok ? v : bf16x8{};
    }
  }
  const float sc = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f, mu = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  wait_own_dma();  // tile 0 landed (tile 1 may still be in flight)
  __syncthreads();

  // stage of tile kt and of tile kt + 2 (three stages in rotation)
  int st_cur = 0, st_pre = 2;
  for (int kt = kt_begin; kt < n_kt; ++kt) {
    char* stg = sm.buf + st_cur * STAGE;
    if (kt == tail_tile) {
      // zero V^T slots of tokens at or past the context end in this stage
      uint16_t* vt = reinterpret_cast<uint16_t*>(stg + DmaSmem<D>::KB);
      for (int e = tid; e < 2 * D * kPage; e += 64 * NW) {
        const int pg = e / (D * kPage), rem = e % (D * kPage);
        const int d = rem / kPage, k = rem % kPage;
        if (kt * kKeys + pg * kPage + k >= ctx) {
          const int chunk = (k >> 3) ^ ((d >> 3) & 1);
          vt[pg * D * kPage + d * kPage + chunk * 8 + (k & 7)] = 0;
        }
      }
      __syncthreads();
    }
    // DMA tile kt+2 into the stage tile kt-1 used (all waves are past it)
    if (kt + 2 < n_kt)
      dma(kt + 2, lds0 + st_pre * STAGE);
    st_cur = st_cur == 2 ? 0 : st_cur + 1;
    st_pre = st_pre == 2 ? 0 : st_pre + 1;

    // S^T = K . Q^T
    // Lane col feeds key krow = col with bits 2 and 3 swapped as row col of
    // the MFMA, so that value i of a lane of half h is key
    // 16(i/8) + 8h + 4((i/4)%2) + i%4: each lane then holds 8 consecutive keys
    // per 16-key step, already the order of P.V's B operand (no lane swaps).
    const char* kbase = stg + krow * (D * 2);
    float sv[16];
    auto scores = [&]() {
      bf16x8 kf[D / 16];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int logical = 2 * ks + half;
        kf[ks] = *reinterpret_cast<const bf16x8*>(kbase + ((logical ^ (krow % CPR)) * 16));
      }
      f32x16 s = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[i] = s[i];
      // one uniform branch for both masks: keys past the row's last visible key,
      // and keys before key_begin (key_begin % 32 == 16: the first tile's first page)
      if (kt >= n_full || kt * kKeys < a.key_begin) {
        const int lim = key_lim - kt * kKeys - 8 * half;
        const int lo = a.key_begin - kt * kKeys - 8 * half;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = 16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3);
          sv[i] = off <= lim && off >= lo ? sv[i] : -INFINITY;
        }
      }
    };
    // weights against the running max mu, summed in four independent chains
    auto weights = [&]() {
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[i] = fast_exp2(__builtin_fmaf(sv[i], sc, -mu));
      float ps[4] = {sv[0], sv[1], sv[2], sv[3]};
#pragma unroll
      for (int i = 4; i < 16; ++i) ps[i & 3] += sv[i];
      return (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };
    // the tile's row max (both lane halves), in exponent units
    auto tile_max = [&]() {
      // IEEE maximum: no operand canonicalisation (no NaN can arise here)
      auto mx = [](float x, float y) { return __builtin_elementwise_maximum(x, y); };
      float mt = mx(mx(sv[0], sv[1]), sv[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mt = mx(mx(mt, sv[i]), sv[i + 1]);
      mt = mx(mt, sv[15]);
      return maxm_xor32(mt) * sc;
    };
    auto rescale = [&](float mt_s) {
      const float m_new = fmaxf(m, mt_s);
      const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
      m = m_new;
      mu = m == -INFINITY ? 0.f : m;
    };
    scores();
    float lt;
    if constexpr (D == 128) {
      // The running max is lazy and the tile's own max is not taken unless
      // needed: while every weight stays small against the stale max (this
      // lane's 16 weights sum to at most 2^8, so each is at most 2^8), the
      // sum and the accumulator are exact against it.  Otherwise (a row's
      // first visible keys, a max that grew, an overflow) the tile is redone
      // from the K tile still in LDS with the true max, and O and l rescaled.
      lt = weights();
      if (__any(!(lt <= 256.f) || m == -INFINITY)) {
        asm volatile("" ::: "memory");  // re-read K: no registers held across
        scores();
        rescale(tile_max());
        lt = weights();
      }
    } else {
      // d = 64: the max first (re-reading K would hold registers that keep
      // this kernel under 128 VGPRs, 4 waves per SIMD); rescale when a row's
      // max grows by more than 2^8
      const float mt_s = tile_max();
      if (__any(mt_s > m + 8.f)) rescale(mt_s);
      lt = weights();
    }
    l += lt;

    // O^T += V^T . P^T, page c = keys 16c..16c+15 of the tile
    const char* vbase = stg + DmaSmem<D>::KB;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // this lane holds keys 16c + 8*half + {0..7}, the B operand's order
      const bf16x8 pf = __builtin_bit_cast(
          bf16x8, u32x4{pack_bf16x2(sv[8 * c + 0], sv[8 * c + 1]), pack_bf16x2(sv[8 * c + 2], sv[8 * c + 3]),
                        pack_bf16x2(sv[8 * c + 4], sv[8 * c + 5]), pack_bf16x2(sv[8 * c + 6], sv[8 * c + 7])});
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = db * 32 + col;
        const int ep = half ^ ((d >> 3) & 1);
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vbase + c * (D * kPage * 2) + d * 32 + ep * 16);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[db], 0, 0, 0);
      }
    }
    // tile kt+1 must have landed before the barrier; tile kt+2 may still fly
    if (kt + 2 < n_kt) wait_own_dma(); else wait_vmcnt<0>();
    __syncthreads();
  }

  wait_vmcnt<0>();  // no DMA of this workgroup outlives it
  l = sum_xor32(l);
  if (!row_ok) return;
  write_rows<D>(a, acc, m, l, qrow, split, half);
}

// fp32 pools: one wave per (query row, query head), 64 keys per step (see
// f32_attend).
template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(AttnArgs a) {
  __shared__ float qs[4][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave, h = blockIdx.y, b = blockIdx.z;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv, g = h / G;
  const int q0 = a.cu_q_lens[b];
  const int qlen = a.cu_q_lens[b + 1] - q0;
  if (i >= qlen) return;
  int ctx = a.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx_len ? a.max_ctx_len : ctx);
  const int pos = ctx - qlen + i;
  const int t_end = a.causal ? min(ctx, pos + 1) : ctx;
  constexpr int NPL = D / 64;
  const int64_t row = static_cast<int64_t>(q0 + i) * Hq + h;
  const float* qp = static_cast<const float*>(a.q) + row * D;
  float o[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    qs[wave][lane + 64 * j] = qp[lane + 64 * j];
    o[j] = 0.f;
  }
  // the row is written and read by this wave only (LDS operations of a wave
  // complete in order)
  __builtin_amdgcn_wave_barrier();
  float m = -INFINITY, l = 0.f;
  f32_attend<D>(a, a.block_table + static_cast<int64_t>(b) * a.bt_stride, g, qs[wave], 0,
                max(t_end, 0), lane, o, m, l);
  const bool empty = !(l > 0.f);
  float* op = static_cast<float*>(a.o) + row * D;
#pragma unroll
  for (int j = 0; j < NPL; ++j) op[lane + 64 * j] = empty ? 0.f : o[j] / l;
  if (lane == 0 && a.lse) a.lse[row] = empty ? -INFINITY : (m + __log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// fp8 pools with every product on the fp8 MFMA (v_mfma_scale_f32_32x32x64_
// f8f6f4, E4M3 operands): FlashAttention-3's FP8 forward (the survey page,
// FlashAttention-3 section: low precision with block quantisation) fitted to
// the paged cache's per-page scales.
//   Q: each query row x is split in two E4M3 parts with one row scale
//      sq = amax/448: hi = E4M3(x/sq) and lo = E4M3((x/sq - hi) * 16); the
//      lo product enters the same accumulator through the instruction's block
//      scale 2^-4, so S carries Q to about 2^-8 relative (one E4M3 part alone
//      moves S by up to 2^-4 relative, which shifts the weights of rows that
//      see few keys).  K: the pool's codes; S = Q.Kc * sk(page).
//   P: the online softmax's weights (<= 4: the running max moves once a tile's
//      max passes it by 2 in log2 units) times their key's V page scale over
//      the largest V page scale of the workgroup's keys, times 112, rounded to
//      E4M3; the factor enters as log2 in the exponent, next to the K page
//      scale, so one FMA and one exp2 give each code's input.  O accumulates
//      Pc . Vc and is multiplied back by sv_max / 112 at the end.  O is divided
//      by the sum of the rounded weights it was built from (per page, from one
//      more MFMA of a page-selector operand with the P codes), so it is the
//      weighted mean of V under weights each within 2^-4 relative of the exact
//      ones (normal E4M3 codes); the logsumexp uses the sum of the unrounded
//      weights.
// Tiles of 64 keys (four pages; one 64-deep k-step for P.V).  K and V codes
// move by buffer loads straight into LDS, three stages of 16 KiB (d = 128):
//   K [64 keys][D/16 chunks of 16 B], chunk c of key i at c ^ fp8_ksw<D>(i);
//   V per page [D][16 keys], as in the pool.
// An operand lane of group g (lane / 32) holds k = 32g .. 32g+31 of each
// 64-deep k-step in A and B alike (any common order contracts the same).
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int D>
struct Fp8Smem {
  static constexpr int KB = 64 * D;          // K codes of a tile
  static constexpr int VB = 4 * kPage * D;   // V codes of a tile
  static constexpr int STAGE = KB + VB;
  char buf[3 * STAGE];
};

__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// the same with B's block scale 2^-4 (E8M0 123)
__device__ __forceinline__ f32x16 mfma_fp8_b16th(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 123);
}

// Chunk swizzle of K row `key` (0..63) of an fp8 tile: chunk c sits at
// c ^ fp8_ksw<D>(key).  The score MFMA's lanes 0..15 read keys 0-3, 32-35,
// 4-7, 36-39 (and so on), so keys of one bank row (same key % (128/D)) among
// them get distinct swizzles: bits 1-2 and 5 of the key for d = 128, bits 2
// and 5 for d = 64.
template <int D>
__device__ __forceinline__ int fp8_ksw(int key) {
  if constexpr (D == 128)
    return ((key >> 1) & 3) | (((key >> 5) & 1) << 2);
  else
    return ((key >> 2) & 1) | (((key >> 5) & 1) << 1);
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_fp8mma_kernel(AttnArgs a, int n_tiles) {
  __shared__ Fp8Smem<D> sm;
  constexpr int KT = 64;             // keys per tile
  constexpr int CK = D / 16;         // 16-byte chunks per K row
  constexpr int NI = D / 32;         // buffer loads per wave per tile (16 KiB / 1 KiB / 4)
  constexpr int STAGE = Fp8Smem<D>::STAGE;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
  // die-aware task order, as in the bf16 kernel
  const int S = a.num_splits;
  const int n_bg = gridDim.x, n_y = gridDim.y;
  const int lin = blockIdx.y * n_bg + blockIdx.x;
  int bg = blockIdx.x, y = blockIdx.y;
  if (n_bg % 8 == 0) {
    const int P = n_bg / 8, GP = pair_group(P);
    const int j = lin / 8, per_group = GP * n_y;
    const int grp = j / per_group, i = j % per_group;
    bg = (lin % 8) * P + grp * GP + i % GP;
    y = i / GP;
  }
  const int b = bg / Hkv, g = bg % Hkv;
  const int tile = n_tiles - 1 - y / S, split = y % S;
  const int TQ = 128 / G;

  // The prologue's memory reads overlap instead of chaining: the block ids of
  // pages 0..127 load with the sequence lengths, the first tiles' DMA goes
  // out as soon as they arrive, and Q and the page scales load beside it.
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.bt_stride;
  const int32_t id_raw0 = lane < a.bt_stride ? bt[lane] : -1;
  const int32_t id_raw1 = 64 + lane < a.bt_stride ? bt[64 + lane] : -1;
  const int q0 = a.cu_q_lens[b];
  const int qlen = a.cu_q_lens[b + 1] - q0;
  int ctx = a.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx_len ? a.max_ctx_len : ctx);
  const int t0 = tile * TQ;
  if (t0 >= qlen || (a.q_filter == kQMany && qlen == 1)) return;
  const int pos_base = ctx - qlen;
  const int t_last = min(t0 + TQ, qlen) - 1;
  const int kmax = max(0, a.causal ? min(ctx, pos_base + t_last + 1) : ctx);  // 0: rows left empty
  const int n_kt_all = (kmax + KT - 1) / KT;
  const int per_split = (n_kt_all + S - 1) / S;
  const int kt_begin = split * per_split;
  const int n_kt = min(n_kt_all, kt_begin + per_split);
  const int n_pages = (ctx + kPage - 1) / kPage;
  const int first_pos = pos_base + t0;
  const int n_full = a.causal ? max(0, min((first_pos + 1) / KT, ctx / KT)) : ctx / KT;
  const int tail_tile = (ctx % kPage) ? (ctx - 1) / KT : -1;

  const int r = wave * 32 + col;
  const int tt = t0 + r / G, hg = r % G;
  const bool row_ok = tt < qlen;
  const int qpos = pos_base + tt;
  const int key_lim = a.causal ? min(qpos, ctx - 1) : ctx - 1;
  const int64_t qrow = static_cast<int64_t>(q0 + (row_ok ? tt : 0)) * Hq + g * G + hg;

  // Q's raw bf16 row parts: this lane holds features 64ks + 32*half .. +31
  u32x4 raw[D / 64][4];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow * D;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        raw[ks][c] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 64 * ks + 32 * half + 8 * c)
                            : u32x4{0, 0, 0, 0};
  }

  // Lane vectors of 64 pages (16 tiles), read out per tile with readlane: the
  // DMA side keeps the page ids two tiles ahead; the compute side keeps its
  // own ids, K scales, and log2 and inverse of the P code factors.
  auto valid_id = [&](int p, int32_t id) -> int32_t {
    return p < n_pages && id >= 0 && id < a.num_blocks ? id : -1;
  };
  const int32_t id0 = valid_id(lane, id_raw0), id1 = valid_id(64 + lane, id_raw1);
  auto page_id = [&](int p) -> int32_t {
    if (p < 64) return id0;
    if (p < 128) return id1;  // p = 64 + lane
    return valid_id(p, p < n_pages ? bt[p] : -1);
  };
  int d_chunk = -1;
  int32_t d_idv = -1;
  auto page_at = [&](int t, int j) -> int32_t {  // DMA side
    const int p = 4 * t + j;
    if ((p >> 6) != d_chunk) {
      d_chunk = p >> 6;
      d_idv = page_id(64 * d_chunk + lane);
      asm volatile("" ::"v"(d_idv));
    }
    return __builtin_amdgcn_readlane(d_idv, p & 63);
  };
  int c_chunk = -1;
  int32_t idv = -1;
  float ksv = 0.f, lvsv = -INFINITY, ivsv = 0.f;
  float p_scale = 1.f;
  auto load_chunk = [&](int c) {  // compute side
    c_chunk = c;
    const int32_t id = page_id(64 * c + lane);
    const bool ok = id >= 0;
    const float vs = ok ? p_scale * a.v_scale[id] : 1.f;
    idv = id;
    ksv = ok ? a.k_scale[id] : 1.f;
    lvsv = ok ? __builtin_amdgcn_logf(vs) : -INFINITY;
    ivsv = ok ? __builtin_amdgcn_rcpf(vs) : 0.f;
    asm volatile("" ::"v"(idv), "v"(ksv), "v"(lvsv), "v"(ivsv));
  };
  // this wave's loads of a tile: all of page 4t + wave, D/64 loads of its K
  // rows, then D/64 of its V (64 lanes x 16 B each)
  constexpr int LP = D / 64;
  uint32_t kvo[LP], vvo[LP];
#pragma unroll
  for (int h = 0; h < LP; ++h) {
    const int m = h * 64 + lane, kip = m / CK, pos = m % CK;
    kvo[h] = static_cast<uint32_t>(kip * D + (pos ^ fp8_ksw<D>(kPage * wave + kip)) * 16);
    vvo[h] = static_cast<uint32_t>(h * 1024 + lane * 16);
  }
  const uint32_t lds0 = lds_address(sm.buf);
  auto dma_tile = [&](int t, uint32_t stage) {
    const int32_t id = page_at(t, wave);
    const int nv = min(kPage, max(0, ctx - (4 * t + wave) * kPage));
    const int64_t chunk = (static_cast<int64_t>(id < 0 ? 0 : id) * Hkv + g) * (kPage * D);
    const int32_t knb = id < 0 ? 0 : nv * D;
    const int32_t vnb = id < 0 || nv == 0 ? 0 : kPage * D;
    const uint32_t dst = stage + wave * (kPage * D);
#pragma unroll
    for (int h = 0; h < LP; ++h)
      dma16(static_cast<const char*>(a.k) + chunk, knb, kvo[h], dst + h * 1024);
#pragma unroll
    for (int h = 0; h < LP; ++h)
      dma16(static_cast<const char*>(a.v) + chunk, vnb, vvo[h], dst + Fp8Smem<D>::KB + h * 1024);
  };
  if (kt_begin < n_kt) {
    dma_tile(kt_begin, lds0);
    dma_tile(kt_begin + 1, lds0 + STAGE);
  }

  // largest V page scale among this workgroup's keys (the P.V reference)
  float sv_max = 0.f;
  {
    const int p0 = kt_begin * (KT / kPage), p1 = min(n_pages, n_kt * (KT / kPage));
    const int32_t ids[2] = {id0, id1};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int p = 64 * h + lane;
      if (p >= p0 && p < p1 && ids[h] >= 0) sv_max = fmaxf(sv_max, a.v_scale[ids[h]]);
    }
    for (int p = max(p0, 128) + lane; p < p1; p += 64) {
      const int32_t id = valid_id(p, bt[p]);
      if (id >= 0) sv_max = fmaxf(sv_max, a.v_scale[id]);
    }
    sv_max = wave_max(sv_max);
    if (!(sv_max > 0.f)) sv_max = 1.f;
  }
  p_scale = 112.f / sv_max;  // weights <= 4 reach codes <= 448
  if (kt_begin < n_kt) load_chunk((4 * kt_begin) >> 6);

  // Q row split in two E4M3 parts: this lane holds features 64ks + 32*half .. +31
  i32x8 qc[D / 64], ql[D / 64];
  float sq;
  {
    float amax = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          amax = fmaxf(amax, fmaxf(fabsf(__builtin_bit_cast(float, raw[ks][c][k] << 16)),
                                   fabsf(__builtin_bit_cast(float, raw[ks][c][k] & 0xffff0000u))));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    sq = amax > 0.f ? amax / 448.f : 1.f;
    const float inv = amax > 0.f ? 448.f / amax : 1.f;
    auto cl = [](float x) { return fminf(fmaxf(x, -448.f), 448.f); };
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t w0 = raw[ks][c][2 * k], w1 = raw[ks][c][2 * k + 1];
          const float x0 = cl(__builtin_bit_cast(float, w0 << 16) * inv);
          const float x1 = cl(__builtin_bit_cast(float, w0 & 0xffff0000u) * inv);
          const float x2 = cl(__builtin_bit_cast(float, w1 << 16) * inv);
          const float x3 = cl(__builtin_bit_cast(float, w1 & 0xffff0000u) * inv);
          const uint32_t h = fp8x4(x0, x1, x2, x3);
          const auto d01 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(h), false);
          const auto d23 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(h), true);
          qc[ks][2 * c + k] = static_cast<int>(h);
          ql[ks][2 * c + k] = static_cast<int>(fp8x4((x0 - d01[0]) * 16.f, (x1 - d01[1]) * 16.f,
                                                     (x2 - d23[0]) * 16.f, (x3 - d23[1]) * 16.f));
        }
  }
  const float sc = a.scale * kLog2e * sq;
  // page selector: row r < 4 of this A operand is 1.0 (E4M3 0x38) on the keys
  // of page r and zero elsewhere, so selector . P^T gives each page's sum of
  // rounded weights; a lane of group g holds keys 32g .. 32g+31 (pages 2g, 2g+1)
  i32x8 sel;
  {
    const int w0 = col == 2 * half ? 0x38383838 : 0, w1 = col == 2 * half + 1 ? 0x38383838 : 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      sel[k] = w0;
      sel[4 + k] = w1;
    }
  }
  float m = -INFINITY, lq = 0.f, mu = 0.f;  // lq: sum of the rounded weights
  // Rows that see fewer than 64 keys see them all in key tile 0, where P is
  // rounded in two E4M3 parts (the second through the block scale 2^-4): one
  // part alone moves such a row by up to 1/15 of its V spread; rows that see
  // more average the rounding down.
  const bool short_rows = (a.causal ? first_pos + 1 : ctx) < 64;
  // Q's second E4M3 part (through the block scale 2^-4) only where some row
  // sees fewer than 256 keys: Q's rounding moves a score by up to 2^-4 of
  // its size, the same for every key of the row, and only many keys average
  // its effect on O down (simulated worst |dO| on the test shapes, one part:
  // 0.052 at 64-127 keys, 0.035 at 128-255, 0.031 at 256-511, 0.030 beyond).
  const bool q_two = (a.causal ? first_pos + 1 : ctx) < 256;
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  wait_vmcnt<NI>();  // tile kt_begin landed (kt_begin + 1 may still fly)
  __syncthreads();

  int st_cur = 0, st_pre = 2;
  for (int kt = kt_begin; kt < n_kt; ++kt) {
    char* stg = sm.buf + st_cur * STAGE;
    if (kt == tail_tile) {
      // zero V codes of slots at or past the context end (they may be NaN codes)
      uint32_t* vw = reinterpret_cast<uint32_t*>(stg + Fp8Smem<D>::KB);
      for (int e = tid; e < 4 * D * 4; e += 256) {
        const int pg = e / (4 * D), kw = e % 4;
        const int key0 = kt * KT + pg * kPage + 4 * kw;
        uint32_t w = vw[e];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (key0 + k >= ctx) w &= ~(0xffu << (8 * k));
        vw[e] = w;
      }
      __syncthreads();
    }
    if (kt + 2 < n_kt) dma_tile(kt + 2, lds0 + st_pre * STAGE);
    st_cur = st_cur == 2 ? 0 : st_cur + 1;
    st_pre = st_pre == 2 ? 0 : st_pre + 1;

    // per page: score factor, log2 of the P code factor and its inverse
    // (pages without keys: weight 0 through a -inf exponent offset)
    // (an absent page: factor 1, and -inf added to its max and exponents)
    float fac[4], lvs[4], ivs[4], madd[4];
    if (((4 * kt) >> 6) != c_chunk) load_chunk((4 * kt) >> 6);  // a tile's 4 pages share a chunk
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pj = (4 * kt + j) & 63;
      const float ks = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ksv), pj));
      lvs[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lvsv), pj));
      ivs[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ivsv), pj));
      fac[j] = sc * ks;
      madd[j] = lvs[j] == -INFINITY ? -INFINITY : 0.f;
    }
    // this lane's scores of block beta all lie on page 2*half + beta
    float fb[2], lb[2], mb[2];
#pragma unroll
    for (int beta = 0; beta < 2; ++beta) {
      fb[beta] = half ? fac[2 + beta] : fac[beta];
      lb[beta] = half ? lvs[2 + beta] : lvs[beta];
      mb[beta] = half ? madd[2 + beta] : madd[beta];
    }

    // S^T = K . Q^T (Q's second part where the rows need it).  MFMA beta's row
    // col is key 32*((col/4)%2) + 16*beta + 4*(col/8) + col%4, so value v of a
    // lane of half h is key 32h + 16*beta + 4*(v/4) + v%4: a lane half holds
    // the 32 keys that its half of P.V's B operand takes, in byte order (no
    // swaps).
    f32x16 sacc[2] = {};
    const int8_t* kb = reinterpret_cast<const int8_t*>(stg);
    auto scores = [&](auto two) {
#pragma unroll
      for (int ks = 0; ks < D / 64; ++ks) {
#pragma unroll
        for (int beta = 0; beta < 2; ++beta) {  // the two blocks' chains interleaved
          const int key = 32 * ((col >> 2) & 1) + 16 * beta + 4 * (col >> 3) + (col & 3);
          const int c0 = 4 * ks + 2 * half;
          const u32x4 lo = *reinterpret_cast<const u32x4*>(kb + (key * CK + (c0 ^ fp8_ksw<D>(key))) * 16);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(kb + (key * CK + ((c0 + 1) ^ fp8_ksw<D>(key))) * 16);
          i32x8 kaa;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            kaa[k] = static_cast<int>(lo[k]);
            kaa[4 + k] = static_cast<int>(hi[k]);
          }
          sacc[beta] = mfma_fp8(kaa, qc[ks], sacc[beta]);
          if constexpr (decltype(two)::value) sacc[beta] = mfma_fp8_b16th(kaa, ql[ks], sacc[beta]);
        }
      }
    };
    if (q_two)
      scores(std::true_type{});
    else
      scores(std::false_type{});
    // value i = 16*beta + v is key 32*half + 16*beta + 4*(v/4) + v%4
    float sv[32];
#pragma unroll
    for (int beta = 0; beta < 2; ++beta)
#pragma unroll
      for (int v = 0; v < 16; ++v) sv[16 * beta + v] = sacc[beta][v];
    if (kt >= n_full) {
      const int lim = key_lim - kt * KT - 32 * half;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int off = 16 * (i >> 4) + 4 * ((i & 15) >> 2) + (i & 3);
        sv[i] = off <= lim ? sv[i] : -INFINITY;
      }
    }
    // row max over the tile: per block raw maxima times the (positive) factors
    // (IEEE maximum: no operand canonicalisation, and no NaN can arise here)
    auto mx = [](float x, float y) { return __builtin_elementwise_maximum(x, y); };
    float mt = -INFINITY;
#pragma unroll
    for (int beta = 0; beta < 2; ++beta) {
      const float* w = sv + 16 * beta;
      float pm = mx(mx(w[0], w[1]), w[2]);
#pragma unroll
      for (int k = 3; k < 15; k += 2) pm = mx(mx(pm, w[k]), w[k + 1]);
      pm = mx(pm, w[15]);
      mt = mx(mt, __builtin_fmaf(pm, fb[beta], mb[beta]));
    }
    mt = maxm_xor32(mt);
    // lazy rescale with headroom 2^2: every weight stays <= 4
    if (__any(mt > m + 2.f)) {
      const float m_new = fmaxf(m, mt);
      const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - m_new);
      lq *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
      m = m_new;
      mu = m == -INFINITY ? 0.f : m;
    }
    // weights times their page's code factor, straight from the exponent
    const float off_b[2] = {lb[0] - mu, lb[1] - mu};
#pragma unroll
    for (int i = 0; i < 32; ++i) sv[i] = fast_exp2(__builtin_fmaf(sv[i], fb[i >> 4], off_b[i >> 4]));

    // P^T codes as the B operand: group g takes keys 32g .. 32g+31, byte t
    // key 32g + t, which is this lane's value t
    i32x8 pb;
#pragma unroll
    for (int w = 0; w < 8; ++w)
      pb[w] = static_cast<int>(fp8x4(sv[4 * w], sv[4 * w + 1], sv[4 * w + 2], sv[4 * w + 3]));
    // O^T += V^T . P^T: V codes of pages 2g, 2g+1 for feature d
    const int8_t* vb = reinterpret_cast<const int8_t*>(stg + Fp8Smem<D>::KB);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + col;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(vb + (2 * half) * (kPage * D) + d * kPage);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(vb + (2 * half + 1) * (kPage * D) + d * kPage);
      i32x8 va;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        va[k] = static_cast<int>(lo[k]);
        va[4 + k] = static_cast<int>(hi[k]);
      }
      acc[db] = mfma_fp8(va, pb, acc[db]);
    }
    // rounded weights: rows 0..3 (values 0..3 of group 0's lanes) are the page
    // sums of the codes; group 1's lanes hold rows 4..7, which are zero
    f32x16 qs = mfma_fp8(sel, pb, f32x16{});
    if (kt == 0 && short_rows) {  // uniform: P's second E4M3 part, 16 x the remainder
      i32x8 pl;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const uint32_t h = static_cast<uint32_t>(pb[w]);
        const auto d01 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(h), false);
        const auto d23 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(h), true);
        pl[w] = static_cast<int>(fp8x4(16.f * (sv[4 * w] - d01[0]), 16.f * (sv[4 * w + 1] - d01[1]),
                                       16.f * (sv[4 * w + 2] - d23[0]), 16.f * (sv[4 * w + 3] - d23[1])));
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = db * 32 + col;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(vb + (2 * half) * (kPage * D) + d * kPage);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(vb + (2 * half + 1) * (kPage * D) + d * kPage);
        i32x8 va;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          va[k] = static_cast<int>(lo[k]);
          va[4 + k] = static_cast<int>(hi[k]);
        }
        acc[db] = mfma_fp8_b16th(va, pl, acc[db]);
      }
      qs = mfma_fp8_b16th(sel, pl, qs);
    }
    lq += (qs[0] * ivs[0] + qs[1] * ivs[1]) + (qs[2] * ivs[2] + qs[3] * ivs[3]);
    if (kt + 2 < n_kt) wait_vmcnt<NI>(); else wait_vmcnt<0>();
    __syncthreads();
  }

  wait_vmcnt<0>();
  lq = sum_xor32(lq);
  if (!row_ok) return;
  // acc holds codes: times sv_max / 112 it is sum(w V); write_rows divides by
  // the rounded weights' sum, which also gives the logsumexp
  const float back = sv_max * (1.f / 112.f);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] *= back;
  write_rows<D>(a, acc, m, lq, qrow, split, half);
}

// Merge of the key splits of every query row: the logsumexp-weighted sum of
// its S normalised partial rows (one wave per (sequence, token, head); empty
// splits carry lse = -inf and weight 0).
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int Hq = a.num_q_heads, S = a.num_splits;
  // kQOne: one row per sequence, partial row b (the packed rows of the
  // q_len = 1 sequences), written to the sequence's token.
  const int64_t per_seq = static_cast<int64_t>(a.q_filter == kQOne ? 1 : a.max_q_len) * Hq;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (r >= per_seq * a.num_seqs) return;
  const int b = static_cast<int>(r / per_seq);
  const int i = static_cast<int>((r % per_seq) / Hq), h = static_cast<int>(r % Hq);
  const int q0 = a.cu_q_lens[b], qlen = a.cu_q_lens[b + 1] - q0;
  if (i >= qlen) return;
  if ((a.q_filter == kQOne && qlen != 1) || (a.q_filter == kQMany && qlen == 1)) return;
  const int64_t out_row = static_cast<int64_t>(q0 + i) * Hq + h;  // token row of o and lse
  // the row of the partials: the token's, or the sequence's under kQOne
  const int64_t row = a.q_filter == kQOne ? static_cast<int64_t>(b) * Hq + h : out_row;
  const int64_t stride = a.part_rows * Hq;  // partial rows per split
  if (row >= stride) return;
  // lane s holds split s's logsumexp and weight (64 splits at a time)
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, a.ws_lse[s * stride + row]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float Mu = M == -INFINITY ? 0.f : M;
  constexpr int NPL = D / 64;
  float acc[NPL] = {};
  float W = 0.f;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int s = s0 + lane;
    const float lt = s < S ? a.ws_lse[s * stride + row] : -INFINITY;
    const float w = lt == -INFINITY ? 0.f : fast_exp2((lt - Mu) * kLog2e);
    W += w;
    const int n = min(64, S - s0);
    const float* op = a.ws_o + (s0 * stride + row) * D + lane;
    const int wbits = __builtin_bit_cast(int, w);
    int k = 0;
    for (; k + 8 <= n; k += 8) {  // 8 splits' loads in flight at once
      float x[8][NPL];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < NPL; ++j) x[u][j] = op[(k + u) * stride * D + 64 * j];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wbits, k + u));
#pragma unroll
        for (int j = 0; j < NPL; ++j) acc[j] += wk * x[u][j];
      }
    }
    for (; k < n; ++k) {
      const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wbits, k));
#pragma unroll
      for (int j = 0; j < NPL; ++j) acc[j] += wk * op[k * stride * D + 64 * j];
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) W += __shfl_xor(W, o);
  const bool empty = !(W > 0.f);
  const float inv = empty ? 0.f : 1.f / W;
#pragma unroll
  for (int j = 0; j < NPL; ++j)
    static_cast<uint16_t*>(a.o)[out_row * D + lane + 64 * j] = to_bf16_bits(acc[j] * inv);
  if (lane == 0 && a.lse) a.lse[out_row] = empty ? -INFINITY : M + __logf(W);
}

// The query rows of the sequences with q_len_b = 1, one per sequence:
// qd[b] = q[cu_q_lens[b]] for those sequences, zeros for the others (all
// heads, bf16).  One workgroup per sequence, 16 bytes per lane.
__global__ __launch_bounds__(256) void gather_q1_rows_kernel(const u32x4* __restrict__ q,
                                                             const int32_t* __restrict__ cu,
                                                             int row16, u32x4* __restrict__ qd) {
  const int b = blockIdx.x;
  const int q0 = cu[b];
  const bool one = cu[b + 1] - q0 == 1;
  u32x4* dst = qd + static_cast<int64_t>(b) * row16;
  if (one) {
    const u32x4* src = q + static_cast<int64_t>(q0) * row16;
    for (int i = threadIdx.x; i < row16; i += 256) dst[i] = src[i];
  } else {
    for (int i = threadIdx.x; i < row16; i += 256) dst[i] = u32x4{0, 0, 0, 0};
  }
}

// One pass of the bf16 or fp8 kernel over a's sequences (or its packed
// queries) and key range, num_splits splits.
template <int D>
hipError_t launch_pass(const AttnArgs& a, hipStream_t st) {
  const int G = a.num_q_heads / a.num_kv_heads;
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 4
#endif
  constexpr int NW = PA_PREFILL_WAVES;
  const int TQ = (a.kv_dtype == PA_BF16 ? 32 * NW : kRows) / G;
  const int n_q = a.packed_q > 0 ? a.packed_q : a.max_q_len;
  const int n_tiles = (n_q + TQ - 1) / TQ;
  const int n_seq = a.packed_q > 0 ? 1 : a.num_seqs;
  const dim3 grid(n_seq * a.num_kv_heads, n_tiles * a.num_splits);
  if (a.fp8_mma) {
    const int tq = 128 / G, nt = (n_q + tq - 1) / tq;
    prefill_fp8mma_kernel<D><<<dim3(n_seq * a.num_kv_heads, nt * a.num_splits), 256, 0, st>>>(a, nt);
  } else if (a.kv_dtype == PA_FP8_E4M3) {
    prefill_kernel<D, true><<<grid, 256, 0, st>>>(a, n_tiles);
  } else {
    prefill_dma_kernel<D, NW><<<grid, 64 * NW, 0, st>>>(a, n_tiles);
  }
  return hipGetLastError();
}

// Merge of the S = a.num_splits partials of every query row into o and lse.
template <int D>
hipError_t launch_merge(const AttnArgs& a, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * (a.q_filter == kQOne ? 1 : a.max_q_len) *
                       a.num_q_heads;
  prefill_merge_kernel<D><<<static_cast<unsigned>((rows + 3) / 4), 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_d(const AttnArgs& a, hipStream_t st) {
  if (a.kv_dtype == PA_F32) {
    const dim3 grid((a.max_q_len + 3) / 4, a.num_q_heads, a.num_seqs);
    prefill_f32_kernel<D><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  hipError_t e = launch_pass<D>(a, st);
  if (e != hipSuccess || a.ws_o == nullptr) return e;
  return launch_merge<D>(a, st);
}

// Shared prefix, packed: the first prefix_len keys (whole pages, the same
// physical blocks for every sequence) are attended once by the q_len = 1 rows
// of all sequences packed into one virtual sequence of B rows (row b is
// sequence b's query; zeros for the other sequences, whose partials are never
// read), with no mask since every query lies past the prefix, into partials
// 0..s_prefix-1; each of those rows' own keys from prefix_len on go through
// the decode split pass into partials s_prefix..s_prefix+s_suffix-1; the
// merge combines them into the rows' tokens.  Rows with q_len > 1 take the
// ordinary pass over all their keys (their work is the same packed or not).
template <int D>
hipError_t launch_shared_prefix_d(const AttnArgs& a, const SharedLaunch& L, hipStream_t st) {
  const bool mixed = a.max_q_len > 1;
  hipError_t e;
  const void* q1 = a.q;
  if (mixed) {
    AttnArgs c = a;
    c.q_filter = kQMany;
    c.num_splits = L.s_plain;
    c.split_base = 0;
    c.ws_o = L.s_plain > 1 ? L.ws_o2 : nullptr;
    c.ws_lse = L.s_plain > 1 ? L.ws_lse2 : nullptr;
    c.part_rows = static_cast<int64_t>(a.num_seqs) * a.max_q_len;
    e = launch_pass<D>(c, st);
    if (e != hipSuccess) return e;
    if (L.s_plain > 1) {
      e = launch_merge<D>(c, st);
      if (e != hipSuccess) return e;
    }
    gather_q1_rows_kernel<<<a.num_seqs, 256, 0, st>>>(
        static_cast<const u32x4*>(a.q), a.cu_q_lens, a.num_q_heads * D / 8,
        static_cast<u32x4*>(L.qd));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    q1 = L.qd;
  }
  AttnArgs p = a;
  p.q = q1;
  p.ws_o = L.ws_o;
  p.ws_lse = L.ws_lse;
  p.part_rows = a.num_seqs;
  p.q_filter = kQAll;
  p.packed_q = a.num_seqs;
  p.max_ctx_len = L.prefix_len;
  p.causal = 0;
  p.key_begin = 0;
  p.split_base = 0;
  p.num_splits = L.s_prefix;
  e = launch_pass<D>(p, st);
  if (e != hipSuccess) return e;
  AttnArgs s = a;
  s.q = q1;
  s.ws_o = L.ws_o;
  s.ws_lse = L.ws_lse;
  s.part_rows = a.num_seqs;
  s.q_filter = mixed ? kQOne : kQAll;
  s.packed_q = 0;
  s.key_begin = L.prefix_len;
  s.split_base = L.s_prefix;
  s.num_splits = L.s_suffix;
  e = launch_decode_split(s, st);
  if (e != hipSuccess) return e;
  AttnArgs m = a;
  m.ws_o = L.ws_o;
  m.ws_lse = L.ws_lse;
  m.part_rows = a.num_seqs;
  m.q_filter = kQOne;
  m.num_splits = L.s_prefix + L.s_suffix;
  return launch_merge<D>(m, st);
}

}  // namespace

hipError_t launch_prefill(const AttnArgs& a, hipStream_t st) {
  return a.head_dim == 64 ? launch_prefill_d<64>(a, st) : launch_prefill_d<128>(a, st);
}

hipError_t launch_prefill_shared_prefix(const AttnArgs& a, const SharedLaunch& L, hipStream_t st) {
  return a.head_dim == 64 ? launch_shared_prefix_d<64>(a, L, st)
                          : launch_shared_prefix_d<128>(a, L, st);
}

}  // namespace pa
