// Matrix-core variant of the paged decode wavefront (bf16 or FP8 caches,
// head dim 128, 4 to 16 query heads per KV head).
//
// What is computed is the same as the vector variant in decode_body.h
// (SourceAIX vLLM page §5.1.1, decode step: softmax over a sequence's
// context of the scaled q.K scores, weighted sum of V, tokens gathered
// through the block table).  Only the work inside a 16-token chunk differs:
//
//   scores  S[t][n] = K[t][:] . Q[n][:]   v_mfma_f32_16x16x32_bf16, four
//           instructions over the 128 dims; M = the chunk's 16 tokens,
//           N = 16 query columns of which the first G are the group's heads
//           (the rest hold zeros and are never stored)
//   output  O[n][d] += P[n][t] V[t][d]    v_mfma_f32_16x16x16_bf16, eight
//           instructions, one per dim d = 8c + e of each lane column c
//
// Lane l = 16 q4 + c.  The score tile leaves lane (q4, c) with the scores of
// tokens 4 q4 .. 4 q4 + 3 for column c, which is exactly the P operand
// layout of the output product, so probabilities never move between lanes.
// The K operand wants one token per lane column: lane (q4, c) loads token c
// of the chunk, 16 bytes of the dims of MFMA i (bf16: dims 32 i + 8 q4 ..,
// so one load instruction covers 64 contiguous bytes of every token; FP8:
// dims 32 q4 + 8 i .., one 32-byte run per lane).  The V operand wants four
// tokens of one dim per lane: lane (q4, c) loads tokens 4 q4 .. 4 q4 + 3,
// dims 8 c .. 8 c + 7 (a load instruction covers four whole head rows) and
// pairs the tokens of each dim with byte permutes.
//
// Softmax state: the lazily moved reference maximum m of column c is kept
// equal in the four lanes of the column (moved only by the wave-wide vote,
// from the column maximum); each lane sums its own probabilities and the
// four sums are added at the end of a segment.  Probabilities are rounded
// to bf16 for the product and the sum takes the rounded values, as in the
// vector variant.
#pragma once

#include "decode_body.h"

namespace pa {

typedef __bf16 mf_bf16x8 __attribute__((ext_vector_type(8)));
typedef short mf_i16x4 __attribute__((ext_vector_type(4)));
typedef float mf_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ mf_f32x4 mfma_16x16x32(const u32x4& a, const u32x4& b, mf_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8, a),
                                                 __builtin_bit_cast(mf_bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ mf_f32x4 mfma_16x16x16(uint2 a, uint2 b, mf_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mf_i16x4, a),
                                                   __builtin_bit_cast(mf_i16x4, b), c, 0, 0, 0);
}

// x of lane src (any lane of the wave)
__device__ __forceinline__ float lane_value(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

// Segment records of a shared item (see even_split_shared): kSegRow =
// group number | kSegShared | (rows of the group << kSegGroupShift).
// Staged table entries of a shared segment carry, above the block number,
// one bit per further row of the group whose own entry differs.
constexpr int kSegShared = 1 << 29;
constexpr int kSegGroupShift = 24;
constexpr int kEntryBits = 27;  // block numbers below 2^27; mismatch bits above
constexpr int kEntryBlock = (1 << kEntryBits) - 1;

template <bool BF16, int D, int G>
struct UseMfma {
  static constexpr bool value = BF16 && D == 128 && G >= 4 && G <= 16;
};

template <int G, bool FP8>
struct MfmaWave {
  static constexpr int D = 128, CHUNK = 16;
  static constexpr int KV = FP8 ? 2 : 4;    // 16-byte K pieces per lane per chunk
  static constexpr int KPH = FP8 ? 8 : 16;  // 16-byte pieces per K head row
  static constexpr int VPH = 16;            // V pieces (8 dims) per head row
  using VVec = typename std::conditional<FP8, uint2, u32x4>::type;
  struct Chunk {
    u32x4 k[KV];
    VVec v[4];
  };

  u32x4 qv[4];     // Q operand of score instruction i (zeros for columns >= G)
  mf_f32x4 o[8];   // O[heads 4 q4 + r][dim 8 c + e] in o[e][r]
  float m;         // reference max of column c (equal in the column's four lanes)
  float l;         // this lane's sum of probabilities of column c
  int lane, q4, c;
  bool hoist;
  int koff, voff[4];

  // 16-byte index (in bf16 units, 16 per head row) of the dims that score
  // instruction i takes from this lane
  __device__ __forceinline__ int kdim(int i) const { return FP8 ? 4 * q4 + i : 4 * i + q4; }

  // Offsets inside the slot rows that do not change from chunk to chunk
  // (the head position depends on the in-block position p only through
  // p & rot; see DecodeWave::prep for the condition).
  __device__ __forceinline__ void prep(int g, int rot, int log2b, int vrow) {
    const int B = 1 << log2b;
    hoist = B <= CHUNK || rot < CHUNK;
    koff = kv_head_pos(g, c & (B - 1), rot) * KPH + (FP8 ? 2 * q4 : q4);
#pragma unroll
    for (int j = 0; j < 4; ++j) voff[j] = j * vrow + kv_head_pos(g, (4 * q4 + j) & (B - 1), rot) * VPH + c;
  }

  // Chunk starting at token t0 of a segment whose staged block-table entry
  // for block b sits at tbl[tb + b] (mismatch bits above the block number).
  __device__ __forceinline__ void load(Chunk& ch, const u32x4* __restrict__ kc,
                                       const VVec* __restrict__ vc, const int32_t* tbl, int tb,
                                       int t0, int log2b, int bmask, int g, int rot, int64_t krow,
                                       int64_t vrow) const {
    const int bk = tbl[tb + ((t0 + c) >> log2b)] & kEntryBlock;
    const int bv = tbl[tb + ((t0 + 4 * q4) >> log2b)] & kEntryBlock;
    load_at(ch, kc, vc, bk, bv, t0, log2b, bmask, g, rot, krow, vrow);
  }

  // The same chunk from the blocks bk (this lane's K token) and bv (its V
  // tokens).
  __device__ __forceinline__ void load_at(Chunk& ch, const u32x4* __restrict__ kc,
                                          const VVec* __restrict__ vc, int bk, int bv, int t0,
                                          int log2b, int bmask, int g, int rot, int64_t krow,
                                          int64_t vrow) const {
    const int tk = t0 + c, tv = t0 + 4 * q4;
    const int64_t ks = (static_cast<int64_t>(bk) << log2b | (tk & bmask)) * krow;
    const int64_t vs = (static_cast<int64_t>(bv) << log2b | (tv & bmask)) * vrow;
    if (hoist) {
      const u32x4* kb = kc + ks + koff;
#pragma unroll
      for (int i = 0; i < KV; ++i) ch.k[i] = kb[FP8 ? i : 4 * i];
      const VVec* vb = vc + vs;
#pragma unroll
      for (int j = 0; j < 4; ++j) ch.v[j] = vb[voff[j]];
    } else {
      const u32x4* kb = kc + ks + kv_head_pos(g, tk & bmask, rot) * KPH + (FP8 ? 2 * q4 : q4);
#pragma unroll
      for (int i = 0; i < KV; ++i) ch.k[i] = kb[FP8 ? i : 4 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ch.v[j] = vc[vs + j * vrow + kv_head_pos(g, (tv + j) & bmask, rot) * VPH + c];
    }
  }

  __device__ __forceinline__ static u32x4 widen(uint2 w) {
    auto lo = [](uint32_t x) {
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
    };
    auto hi = [](uint32_t x) {
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
    };
    return u32x4{lo(w.x), hi(w.x), lo(w.y), hi(w.y)};
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }

  // Token np of the chunk (if any) takes nk / nv (bf16, this lane's pieces)
  // instead of what was loaded: the fused append's new token, always in a
  // masked chunk (np = -1: none).  With COLS, the query columns set in
  // colmask are dropped (their scores count as -inf).
  template <bool MASKED, bool COLS = false>
  __device__ __forceinline__ void compute(const Chunk& ch, int t0, int end, float scale_log2,
                                          int np, const u32x4 (&nk)[4], const u32x4& nv,
                                          int colmask = 0) {
    u32x4 kop[4], vv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (FP8) {
        const u32x4& w = ch.k[i >> 1];
        kop[i] = widen((i & 1) ? make_uint2(w.z, w.w) : make_uint2(w.x, w.y));
      } else {
        kop[i] = ch.k[i];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (FP8) vv[j] = widen(ch.v[j]);
      else vv[j] = ch.v[j];
    }
    const int tv = t0 + 4 * q4;
    if constexpr (MASKED) {
      if (t0 + c == np) {
#pragma unroll
        for (int i = 0; i < 4; ++i) kop[i] = nk[i];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (tv + j == np) vv[j] = nv;
    }

    mf_f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) sacc = mfma_16x16x32(kop[i], qv[i], sacc);

    float s[4];
    const bool col_off = COLS && ((colmask >> c) & 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = sacc[r] * scale_log2;
      if constexpr (COLS) {
        if (col_off) s[r] = -INFINITY;
      }
      if constexpr (MASKED) {
        if (tv + r >= end) {
          s[r] = -INFINITY;
          vv[r] = u32x4{0u, 0u, 0u, 0u};  // stale slots may hold NaN
        }
      }
    }
    const float cmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    if (__any(cmax > m + kTau)) {
      const float mn = fmaxf(m, rows_max<16>(cmax));
      const float alpha = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      l *= alpha;
      // output row r of this lane is column 4 q4 + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = lane_value(alpha, 4 * q4 + r);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e][r] *= a;
      }
    }
    const float mref = (m == -INFINITY) ? 0.f : m;
    const uint32_t p01 = pack_bf16(__builtin_amdgcn_exp2f(s[0] - mref), __builtin_amdgcn_exp2f(s[1] - mref));
    const uint32_t p23 = pack_bf16(__builtin_amdgcn_exp2f(s[2] - mref), __builtin_amdgcn_exp2f(s[3] - mref));
    l += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
    const uint2 pa = make_uint2(p01, p23);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint2 b0 = make_uint2(pair_lo(word(vv[0], w), word(vv[1], w)), pair_lo(word(vv[2], w), word(vv[3], w)));
      const uint2 b1 = make_uint2(pair_hi(word(vv[0], w), word(vv[1], w)), pair_hi(word(vv[2], w), word(vv[3], w)));
      o[2 * w] = mfma_16x16x16(pa, b0, o[2 * w]);
      o[2 * w + 1] = mfma_16x16x16(pa, b1, o[2 * w + 1]);
    }
  }
};

// ---- shared prefixes -------------------------------------------------------
//
// Segment records of a shared item: kSegQRow and kSegTable = the group's
// first row, kSegCtx = -1 (no fused append in a shared item).

__device__ __forceinline__ int lane_value_i(int x, int src) {
  return __builtin_amdgcn_ds_bpermute(src << 2, x);
}

// Balanced split with shared prefixes (DecodeArgs::share; at most 64 rows,
// row r on lane r).  Row r is a candidate when it and row r - 1 have tokens
// that may be shared (all but each row's last token) and their first
// block-table entries are equal (entry 0 is loaded with the length; a
// batch without such rows takes the plain split of those lengths); the
// tokens they share are then estimated from 15 more entries probed at the
// same positions in every row, equal steps over the longest candidate
// pair's common blocks (the run of equal probes from the start within the
// pair's own common blocks; the entries between probes are checked when
// the tables are staged).  A run of candidates
// after a row that is not one is cut into groups of up to 16 / G rows, and
// a group shares the least of its rows' estimates, rounded down to a
// chunk.  Costs, segments and plan entries then follow the items of the
// line: (shared item of a group, own item of its first row), own items of
// the other rows; everything else as in even_split.
template <int CHUNK, int G, class ZeroRow>
__device__ WaveWork even_split_shared(const DecodeArgs& a, int y, int block_size, int log2b,
                                      int32_t* lds, bool write_plan, ZeroRow&& zero_row,
                                      int32_t* xchg, int member, int group) {
  constexpr int M = kShareCols / G;  // rows per group
  const int lane = threadIdx.x & 63;
  const int r = lane;
  constexpr int Q = kPlanChunkCost, beta = kPlanRowCost;
  int qrow;
  const int64_t mbps = a.max_blocks_per_seq;
  const int rc = min(r, a.num_rows - 1);
  const int* trow = a.block_tables + static_cast<int64_t>(rc) * mbps;
  // the first entry is loaded with the length (both in flight at once)
  const int f0_raw = mbps > 0 ? trow[0] : -1;
  int ctx = plan_row(a, rc, block_size, qrow);
  if (r >= a.num_rows) ctx = -1;
  const int f0 = ctx > 0 ? f0_raw : -1;
  // a row's last token is never shared: in a fused append it is the step's
  // new token, and keeping the rule in plain decode too gives both calls
  // the same plan (and bit-identical outputs)
  const int tail = 1;
  const int ctx_prev = lane_value_i(ctx, max(r - 1, 0));  // all lanes take part
  const int f0_prev = lane_value_i(f0, max(r - 1, 0));
  const int ctx_p = r > 0 ? ctx_prev : -1;
  const int lim = min(ctx, ctx_p) - tail;  // tokens both rows may share
  const bool cand = r > 0 && ctx > 0 && ctx_p > 0 && lim >= CHUNK && f0 == f0_prev;
  const uint64_t cmask = __ballot(cand);
  PA_TL(const unsigned long long q1 = __builtin_amdgcn_s_memrealtime();)
  if (cmask == 0) {  // the plain split of the lengths already loaded
    const int ctx1[1] = {ctx}, qrow1[1] = {qrow};
    return split_rows<CHUNK, 1>(a, y, log2b, lds, write_plan, zero_row, ctx1, qrow1);
  }
  // 15 more entries at equal steps over the blocks the longest candidate
  // pair may share, at the same positions in every row: a row loads its own
  // (when it or the next row is a candidate) and takes its predecessor's by
  // a lane shuffle.  The run of equal entries from entry 0, over the pair's
  // common blocks, estimates the shared length.  The waves of a workgroup
  // (`group` of them, this one `member`) plan the same rows, so they share
  // the probes: wave w loads those with k mod group == w, and the equalities
  // meet in xchg (group x 64 words) after a barrier, which every wave of the
  // workgroup reaches here since they all see the same candidates.
  const int nbk = (wave_max(cand ? lim : 0) + block_size - 1) >> log2b;  // uniform
  const bool probe = cand || (r < 63 && ((cmask >> (r + 1)) & 1));
  const int nblk_own = ctx > 0 ? min((ctx + block_size - 1) >> log2b, static_cast<int>(mbps)) : 0;
  const int lim_b = (lim + block_size - 1) >> log2b;  // blocks holding the common tokens
  int er[15];
#pragma unroll
  for (int k = 0; k < 15; ++k) {
    const int pos = (k + 1) * (nbk - 1) / 15;
    er[k] = k % group == member && probe && pos < nblk_own ? trow[pos] : -1;
  }
  uint32_t eq = 0;  // bit k: probe k lies in the pair's common blocks and matches
#pragma unroll
  for (int k = 0; k < 15; ++k) {
    if (k % group != member) continue;  // uniform
    const int ep = lane_value_i(er[k], max(r - 1, 0));  // all lanes take part
    const int pos = (k + 1) * (nbk - 1) / 15;
    if (cand && pos < lim_b && er[k] == ep) eq |= 1u << k;
  }
  if (group > 1) {
    xchg[member * 64 + lane] = static_cast<int32_t>(eq);
    __syncthreads();
    eq = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (w < group) eq |= static_cast<uint32_t>(xchg[w * 64 + lane]);
  }
  int s_pair = 0;
  if (cand) {
    int lcp = 1;
    bool run = true;
#pragma unroll
    for (int k = 0; k < 15; ++k) {
      run = run && ((eq >> k) & 1) != 0;
      if (run) lcp = (k + 1) * (nbk - 1) / 15 + 1;
    }
    s_pair = min(lcp << log2b, lim);
  }
  PA_TL(asm volatile("" ::"v"(s_pair));
        const unsigned long long q2 = __builtin_amdgcn_s_memrealtime();)
  // run start: the last row at or before r that is not a candidate (row 0 never is)
  const uint64_t notc = ~cmask & (r == 63 ? ~0ull : ((2ull << r) - 1));
  const int run0 = 63 - __builtin_clzll(notc);
  const int L = r - (r - run0) % M;  // first row of r's group
  const uint64_t after = ~(cmask >> (L + 1 > 63 ? 63 : L + 1));
  const int more = L + 1 > 63 ? 0 : (after == 0 ? 64 : __builtin_ctzll(after));
  const int n = 1 + min(M - 1, more);  // rows of the group
  int smin = 0x7fffffff;
#pragma unroll
  for (int m = 1; m < M; ++m) {
    const int v = lane_value_i(s_pair, min(L + m, 63));
    if (m < n) smin = min(smin, v);
  }
  const int S = n >= 2 ? smin / CHUNK * CHUNK : 0;  // tokens of the shared item
  const bool grouped = S >= CHUNK;
  const int m_idx = r - L;
  const bool lead = grouped && m_idx == 0;
  const int gnum_l = wave_exclusive_scan(lead ? 1 : 0);
  const int gnum = lane_value_i(gnum_l, L);
  PA_TL(asm volatile("" ::"v"(gnum), "v"(S));
        const unsigned long long q3 = __builtin_amdgcn_s_memrealtime();)

  const int c_sh = lead ? S / CHUNK : 0;
  const int tok_pr = grouped ? S : 0;
  const int c_pr = ctx > tok_pr ? (ctx - tok_pr + CHUNK - 1) / CHUNK : 0;
  const int cost_sh = lead ? beta + Q * c_sh : 0;
  const int cost_pr = ctx < 0 ? 0 : ((grouped && c_pr == 0) ? 0 : beta + Q * c_pr);
  const int cost = cost_sh + cost_pr;
  const int pre = wave_exclusive_scan(cost);
  const int T = __builtin_amdgcn_readlane(pre + cost, 63);
  WaveWork ww{0, 0, 0};
  if (T == 0) return ww;
  int W = max((T + a.plan_max_cost - 1) / a.plan_max_cost, a.plan_share);
  W = min(min(W, a.max_partitions), max(1, T / Q));
  if (y >= W) return ww;
  const int lo = split_point(y, T, W), hi = split_point(y + 1, T, W);
  PA_TL(asm volatile("" ::"v"(lo), "v"(hi));
        const unsigned long long q4 = __builtin_amdgcn_s_memrealtime();)
  auto chunk_range = [&](int x0, int c, int& jl, int& jh) {
    jl = lo > x0 ? (lo - x0 + Q - 1) / Q : 0;
    jh = hi > x0 ? min(c, (hi - x0 + Q - 1) / Q) : 0;
  };
  const int p_sh = pre, p_pr = pre + cost_sh;
  const int x_sh = p_sh + beta, x_pr = p_pr + beta;
  // the wave holding an item's first unit writes its entries; an empty own
  // item at the very end of the line belongs to the last wave
  const bool own_here = (p_pr >= lo && p_pr < hi) || (p_pr == T && y == W - 1);
  if (ctx >= 0 && write_plan) {
    if (own_here) {
      int2 e = make_int2(0, 0);
      if (c_pr > 0) {
        const int yf = wave_of(x_pr, T, W), yl = wave_of(x_pr + Q * (c_pr - 1), T, W);
        e = make_int2(yf + r, yl - yf + 1);
      }
      *reinterpret_cast<int2*>(a.plan + 2 * r) = e;
      if (!grouped) *reinterpret_cast<int2*>(a.plan_sh + 2 * r) = make_int2(0, 0);
    }
    // shared item: its first row's entry for every row of the group
    if (lead && p_sh >= lo && p_sh < hi) {
      const int yf = wave_of(x_sh, T, W), yl = wave_of(x_sh + Q * (c_sh - 1), T, W);
      for (int m = 0; m < n; ++m)
        *reinterpret_cast<int2*>(a.plan_sh + 2 * (r + m)) =
            make_int2(yf + gnum, (yl - yf + 1) | (m << 16));
    }
  }
  if (ctx == 0 && own_here) zero_row(qrow);
  int jl_sh = 0, jh_sh = 0, jl_pr = 0, jh_pr = 0;
  if (lead) chunk_range(x_sh, c_sh, jl_sh, jh_sh);
  if (ctx > 0) chunk_range(x_pr, c_pr, jl_pr, jh_pr);
  const bool has_sh = jl_sh < jh_sh, has_pr = jl_pr < jh_pr;
  const int e_sh = has_sh ? seg_blocks<CHUNK>(jl_sh, jh_sh, log2b) : 0;
  // own-item chunks start at token tok_pr, a multiple of the chunk
  const int c0 = tok_pr / CHUNK;
  const int e_pr = has_pr ? seg_blocks<CHUNK>(c0 + jl_pr, c0 + jh_pr, log2b) : 0;
  const int lane_seg = (has_sh ? 1 : 0) + (has_pr ? 1 : 0);
  const int lane_e = e_sh + e_pr;
  const int seg_pre = wave_exclusive_scan(lane_seg);
  const int e_pre = wave_exclusive_scan(lane_e);
  ww.nseg = __builtin_amdgcn_readlane(seg_pre + lane_seg, 63);
  ww.E = __builtin_amdgcn_readlane(e_pre + lane_e, 63);
  // chunks of the items this range holds (jl > jh for an item outside it)
  ww.K = wave_sum((has_sh ? jh_sh - jl_sh : 0) + (has_pr ? jh_pr - jl_pr : 0));
  if (ww.nseg * kSegInts + ww.E > kDecodeLdsInts) {
    ww.nseg = ww.K = ww.E = 0;
    return ww;
  }
  PA_TL(ww.phase[0] = q1; ww.phase[1] = q2; ww.phase[2] = q3; ww.phase[3] = q4;)
  int sidx = seg_pre, eoff = e_pre;
  if (has_sh) {
    put_seg(lds, sidx, gnum | kSegShared | (n << kSegGroupShift), qrow, jl_sh * CHUNK,
            jh_sh * CHUNK, jh_sh - jl_sh, eoff, r, -1);
    ++sidx;
    eoff += e_sh;
  }
  if (has_pr) {
    const int final_flag = (!grouped && jl_pr == 0 && jh_pr == c_pr) ? kSegFinal : 0;
    put_seg(lds, sidx, r | final_flag, qrow, tok_pr + jl_pr * CHUNK,
            min(tok_pr + jh_pr * CHUNK, ctx), jh_pr - jl_pr, eoff, r, ctx);
  }
  return ww;
}

// stage_tables for a list that may hold shared segments: a shared
// segment's entry also gets, above the block number, bit m - 1 set when row
// m of the group has a different entry there.  Returns whether any entry
// of the wave has such a bit (wave-uniform).
__device__ __forceinline__ bool stage_tables_shared(const DecodeArgs& a, int32_t* lds,
                                                   const WaveWork& ww, int log2b,
                                                   int32_t num_blocks) {
  const int lane = threadIdx.x & 63;
  const int tb0 = ww.nseg * kSegInts;
  const int B = 1 << log2b;
  const int64_t mbps = a.max_blocks_per_seq;
  bool mism = false;
  for (int e0 = 0; e0 < ww.E; e0 += 256) {
    int val[4], bits[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * 64 + lane;
      val[u] = 0;
      bits[u] = 0;
      if (e < ww.E) {
        int lo = 0, hi = ww.nseg - 1;  // the last segment with eoff <= e
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (lds[mid * kSegInts + kSegEoff] <= e) lo = mid; else hi = mid - 1;
        }
        const int* d = lds + lo * kSegInts;
        const int bi = (d[kSegTok0] >> log2b) + (e - d[kSegEoff]);
        const int nblk = (d[kSegEnd] + B - 1) >> log2b;
        if (bi < nblk) {
          const int* t = a.block_tables + static_cast<int64_t>(d[kSegTable]) * mbps + bi;
          const int raw = t[0];
          if (d[kSegRow] & kSegShared) {
            const int n = (d[kSegRow] >> kSegGroupShift) & 31;
            for (int m = 1; m < n; ++m)
              if (t[m * mbps] != raw) bits[u] |= 1 << (m - 1);
          }
          val[u] = clampi(raw, 0, num_blocks - 1);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * 64 + lane;
      if (e < ww.E) lds[tb0 + e] = val[u] | (bits[u] << kEntryBits);
      mism = mism || bits[u] != 0;
    }
  }
  return __any(mism);
}

template <int G, bool FP8>
struct MfmaStages {
  static constexpr int value = FP8 ? 3 : 2;
};

// One decode wavefront on the matrix cores: KV head g and, with the
// balanced split, range y of the line, or partition y of row z (fixed
// split).  The plan, the segment list and the staged block tables are those
// of decode_partition_body (with shared prefixes, even_split_shared).
template <int G, bool FP8>
__device__ __forceinline__ void decode_mfma_body(const DecodeArgs& a, int g, int y, int z,
                                                 int32_t* lds, int32_t num_kv_heads,
                                                 int32_t num_blocks, int32_t log2b,
                                                 int32_t* xchg = nullptr, int member = 0,
                                                 int group = 1) {
  using W = MfmaWave<G, FP8>;
  constexpr int CHUNK = W::CHUNK, VPR = 16, D = 128;
  constexpr int M = kShareCols / G;  // rows of a shared group, at most
  static_assert(CHUNK == decode_chunk_tokens(2, D), "host and device chunk sizes differ");
  const int H = num_kv_heads * G;
  const int B = 1 << log2b;
  const int lane = threadIdx.x & 63;
  u32x4* out = static_cast<u32x4*>(a.out);

  PA_TL(const unsigned long long t_start = __builtin_amdgcn_s_memrealtime();)
  WaveWork ww;
  if (a.balanced) {
    auto zero_row = [&](int q_row) {  // this lane writes the G heads' zero rows
      u32x4* o = out + (static_cast<int64_t>(q_row) * H + g * G) * VPR;
      for (int v = 0; v < G * VPR; ++v) o[v] = u32x4{0u, 0u, 0u, 0u};
    };
    if constexpr (M >= 2) {
      if (a.share)
        ww = even_split_shared<CHUNK, G>(a, y, B, log2b, lds, g == 0, zero_row, xchg, member,
                                         group);
      else
        ww = even_split<CHUNK>(a, y, B, log2b, lds, g == 0, zero_row);
    } else {
      ww = even_split<CHUNK>(a, y, B, log2b, lds, g == 0, zero_row);
    }
  } else {
    const RowInfo ri = row_info(a, z, B);
    if (!ri.active) return;
    const int P = a.partition_size;
    const int nparts = (ri.ctx + P - 1) / P;
    if (ri.ctx == 0) {
      if (y == 0) {
        for (int v = lane; v < G * VPR; v += 64)
          out[(static_cast<int64_t>(ri.q_row) * H + g * G) * VPR + v] = u32x4{0u, 0u, 0u, 0u};
      }
      return;
    }
    if (y >= nparts) return;
    const int tok0 = y * P, end = min(tok0 + P, ri.ctx);
    const int n = (end - tok0 + CHUNK - 1) / CHUNK;
    if (lane == 0)
      put_seg(lds, 0, z | (nparts == 1 ? kSegFinal : 0), ri.q_row, tok0, end, n, 0, ri.table_row,
              ri.ctx);
    ww = WaveWork{1, n, seg_blocks<CHUNK>(tok0 / CHUNK, tok0 / CHUNK + n, log2b)};
  }
  ww.nseg = __builtin_amdgcn_readfirstlane(ww.nseg);
  ww.K = __builtin_amdgcn_readfirstlane(ww.K);
  ww.E = __builtin_amdgcn_readfirstlane(ww.E);
  PA_TL(const unsigned long long t_plan = __builtin_amdgcn_s_memrealtime();)
  if (ww.K <= 0 || ww.nseg <= 0) return;  // no segment record to read
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  auto seg = [&](int s, int f) { return __builtin_amdgcn_readfirstlane(lds[s * kSegInts + f]); };

  W w;
  w.lane = lane;
  w.q4 = lane >> 4;
  w.c = lane & 15;
  const int64_t krow = static_cast<int64_t>(num_kv_heads) * W::KPH;
  const int64_t vrow = static_cast<int64_t>(num_kv_heads) * W::VPH;
  w.prep(g, a.rot, log2b, static_cast<int>(vrow));
  const u32x4* qp = static_cast<const u32x4*>(a.q);
  // Query columns of a segment: head c of q row q_row (own item), or head
  // c mod G of row q_row + c / G (shared item, ncols = rows x G).  Columns
  // past ncols load a valid row and drop it.
  auto load_q = [&](int q_row, int ncols) {
    const int cc = min(w.c, ncols - 1);
    const u32x4* src = qp + (static_cast<int64_t>(q_row + cc / G) * H + g * G + cc % G) * VPR;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = src[w.kdim(i)];
      w.qv[i] = w.c < ncols ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto seg_cols = [&](int rf) {
    return (rf & kSegShared) ? ((rf >> kSegGroupShift) & 31) * G : G;
  };
  load_q(seg(0, kSegQRow), seg_cols(seg(0, kSegRow)));
  bool mism = false;
  if (a.share)
    mism = stage_tables_shared(a, lds, ww, log2b, num_blocks);
  else
    stage_tables(a, lds, ww, log2b, num_blocks);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  PA_TL(const unsigned long long t_stage = __builtin_amdgcn_s_memrealtime();)

  float scale_log2 = a.scale * kLog2e;
  float out_scale = 1.f;
  if constexpr (FP8) {
    scale_log2 *= a.k_scale[g];
    out_scale = a.v_scale[g];
  }
  using VVec = typename W::VVec;
  const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
  const VVec* vc = static_cast<const VVec*>(a.v_cache);
  const int rot = a.rot;
  const int bmask = B - 1;
  const int tb0 = ww.nseg * kSegInts;
  constexpr int S = MfmaStages<G, FP8>::value;

  for (int sg = 0; sg < ww.nseg; ++sg) {
    const int rf = seg(sg, kSegRow);
    const bool shared = (rf & kSegShared) != 0;
    const int zr = rf & ((1 << kSegGroupShift) - 1);  // row, or group number
    const int ncols = seg_cols(rf);
    const int q_row = seg(sg, kSegQRow);
    const int start = seg(sg, kSegTok0);
    const int end = seg(sg, kSegEnd);
    const int nchunks = seg(sg, kSegN);
    const int tb = tb0 + seg(sg, kSegEoff) - (start >> log2b);
    if (sg > 0) load_q(q_row, ncols);
    w.reset();

    // Fused append (see decode_partition_body): the segment that ends the
    // row attends the step's new token from registers and stores it.
    const bool row_end = a.new_slots != nullptr && end == seg(sg, kSegCtx);
    int slot_v = -1;
    u32x4 nk[4], nv{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) nk[i] = u32x4{0u, 0u, 0u, 0u};
    if (row_end) {
      slot_v = a.new_slots[zr + vgpr_zero()];
      const int64_t in = (static_cast<int64_t>(zr) * num_kv_heads + g) * VPR;
      const u32x4* nkp = static_cast<const u32x4*>(a.new_k) + in;
#pragma unroll
      for (int i = 0; i < 4; ++i) nk[i] = nkp[w.kdim(i)];
      nv = static_cast<const u32x4*>(a.new_v)[in + w.c];
    }

    // The chunk stream of the segment (the pipeline of S register buffers:
    // the loads of chunk c+S-1 are issued before chunk c is computed; loads
    // past the last chunk are clamped onto it; only the final S chunks are
    // computed with the length mask), with the fused append in its last
    // chunks.  COLS drops the query columns in colmask.
    auto stream = [&](auto cols_tag, int colmask) {
      constexpr bool COLS = decltype(cols_tag)::value;
      typename W::Chunk buf[S];
      const int last = nchunks - 1;
      auto load_chunk = [&](typename W::Chunk& ch, int ci) {
        ci = ci < last ? ci : last;
        w.load(ch, kc, vc, lds, tb, start + ci * CHUNK, log2b, bmask, g, rot, krow, vrow);
      };
#pragma unroll
      for (int s = 0; s < S - 1; ++s) load_chunk(buf[s], s);
      int c = 0;
      for (; c + S < nchunks; c += S) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
          load_chunk(buf[(s + S - 1) % S], c + s + S - 1);
          w.template compute<false, COLS>(buf[s], start + (c + s) * CHUNK, end, scale_log2, -1, nk,
                                          nv, colmask);
        }
      }
      load_chunk(buf[S - 1], c + S - 1);
      const int64_t slot = __builtin_amdgcn_readfirstlane(slot_v);
      const bool put = row_end && slot >= 0 && slot < (static_cast<int64_t>(num_blocks) << log2b);
      const int np = put ? end - 1 : -1;
      // what the cache receives: the bf16 rows, or their E4M3 codes (then the
      // attended values are the codes, widened)
      uint2 sk8[4], sv8 = make_uint2(0u, 0u);
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sk8[i] = quant_fp8x8(nk[i], a.k_scale[g]);
          nk[i] = W::widen(sk8[i]);
        }
        sv8 = quant_fp8x8(nv, a.v_scale[g]);
        nv = W::widen(sv8);
      }
#pragma unroll
      for (int s = 0; s < S; ++s)
        if (c + s < nchunks)
          w.template compute<true, COLS>(buf[s], start + (c + s) * CHUNK, end, scale_log2, np, nk,
                                         nv, colmask);
      if (put) {
        const int hp = kv_head_pos(g, static_cast<int>(slot) & bmask, rot);
        u32x4* kd = const_cast<u32x4*>(kc) + slot * krow + hp * W::KPH;
        VVec* vd = const_cast<VVec*>(vc) + slot * vrow + hp * W::VPH + w.c;
        if constexpr (FP8) {
          if (w.c == 0) {  // lane (q4, 0) holds dims 32 q4 .. 32 q4 + 31
            kd[2 * w.q4] = u32x4{sk8[0].x, sk8[0].y, sk8[1].x, sk8[1].y};
            kd[2 * w.q4 + 1] = u32x4{sk8[2].x, sk8[2].y, sk8[3].x, sk8[3].y};
          }
          if (w.q4 == 0) *vd = sv8;
        } else {
          if (w.c == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) kd[4 * i + w.q4] = nk[i];
          }
          if (w.q4 == 0) *vd = nv;
        }
      }
    };

    // A shared segment in which some row of the group has its own block
    // where the first row has another (found while staging) runs in passes:
    // the first row's blocks without those rows' columns, then, for each
    // such row, its own blocks (staged over the same entries) for its
    // columns alone.
    int diffs = 0;
    if (shared && mism) {
      const int e0 = tb0 + seg(sg, kSegEoff);
      const int nent = ((start + nchunks * CHUNK - 1) >> log2b) - (start >> log2b) + 1;
      int bits = 0;
      for (int e = lane; e < nent; e += 64) bits |= lds[e0 + e] >> kEntryBits;
#pragma unroll
      for (int b = 0; b < M - 1; ++b)
        if (__any((bits >> b) & 1)) diffs |= 1 << b;
    }
    if (diffs == 0) {
      stream(std::false_type{}, 0);
    } else {
    const int ne = ((start + nchunks * CHUNK - 1) >> log2b) - (start >> log2b) + 1;
#pragma unroll 1
    for (int pass = 0; pass < M; ++pass) {
      int colmask = 0;
      if (pass == 0) {
#pragma unroll
        for (int b = 0; b < M - 1; ++b)
          if ((diffs >> b) & 1) colmask |= ((1 << G) - 1) << ((b + 1) * G);
      } else {
        if (!((diffs >> (pass - 1)) & 1)) continue;
        colmask = 0xFFFF & ~(((1 << G) - 1) << (pass * G));
        const int* own = a.block_tables +
                         static_cast<int64_t>(seg(sg, kSegTable) + pass) * a.max_blocks_per_seq +
                         (start >> log2b);
        const int e0 = tb0 + seg(sg, kSegEoff);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        for (int e = lane; e < ne; e += 64) lds[e0 + e] = clampi(own[e], 0, num_blocks - 1);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      }
      stream(std::true_type{}, colmask);
    }
    }

    // column totals, then (m, sum) of this lane's output rows 4 q4 + r
    const float L = rows_sum<16>(w.l);
    float Mr[4], Lr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      Mr[r] = lane_value(w.m, 4 * w.q4 + r);
      Lr[r] = lane_value(L, 4 * w.q4 + r);
    }
    if (rf & kSegFinal) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * w.q4 + r;
        if (h >= G) continue;
        const float inv = out_scale / Lr[r];
        u32x4 res;
        res.x = pack_bf16(w.o[0][r] * inv, w.o[1][r] * inv);
        res.y = pack_bf16(w.o[2][r] * inv, w.o[3][r] * inv);
        res.z = pack_bf16(w.o[4][r] * inv, w.o[5][r] * inv);
        res.w = pack_bf16(w.o[6][r] * inv, w.o[7][r] * inv);
        out[(static_cast<int64_t>(q_row) * H + g * G + h) * VPR + w.c] = res;
      }
    } else {
      // partial of column col: own item, index (y + row) * H + g G + col (or
      // the fixed split's); shared item, ((y + group) H_kv + g) 16 + col
      float* po_base;
      float* pml_base;
      int64_t hstride;
      if (shared) {
        const int64_t base = ((static_cast<int64_t>(y) + zr) * num_kv_heads + g) * kShareCols;
        po_base = a.sh_o + base * D;
        pml_base = a.sh_ml + base * 2;
        hstride = 1;
      } else {
        const int64_t base = a.balanced ? (static_cast<int64_t>(y) + zr) * H + g * G
                                        : (static_cast<int64_t>(zr) * H + g * G) * a.max_partitions + y;
        hstride = a.balanced ? 1 : a.max_partitions;
        po_base = a.part_o + base * D;
        pml_base = a.part_ml + base * 2;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = 4 * w.q4 + r;
        if (col >= ncols) continue;
        float* po = po_base + col * hstride * D + 8 * w.c;
        *reinterpret_cast<float4*>(po) = make_float4(w.o[0][r] * out_scale, w.o[1][r] * out_scale,
                                                     w.o[2][r] * out_scale, w.o[3][r] * out_scale);
        *reinterpret_cast<float4*>(po + 4) = make_float4(w.o[4][r] * out_scale, w.o[5][r] * out_scale,
                                                         w.o[6][r] * out_scale, w.o[7][r] * out_scale);
        if (w.c == 0)
          *reinterpret_cast<float2*>(pml_base + col * hstride * 2) = make_float2(Mr[r], Lr[r]);
      }
    }
  }
  PA_TL(const int64_t trace_idx = static_cast<int64_t>(y) * num_kv_heads + g;
        if (a.trace && a.balanced && lane == 0 && trace_idx < kTraceDecodeWaves) {
    unsigned long long* t = a.trace + trace_idx * 10;
    t[0] = t_start;
    t[1] = t_plan;
    t[2] = t_stage;
    t[3] = __builtin_amdgcn_s_memrealtime();
    t[4] = __builtin_amdgcn_s_getreg((31 << 11) | 20) |
           (static_cast<unsigned long long>(__builtin_amdgcn_s_getreg((31 << 11) | 4)) << 32);
    t[5] = static_cast<unsigned long long>(ww.nseg) | (static_cast<unsigned long long>(ww.K) << 32);
    for (int i = 0; i < 4; ++i) t[6 + i] = ww.phase[i];
  })
}

}  // namespace pa
