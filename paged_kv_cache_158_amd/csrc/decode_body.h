// Device code of the split-K paged decode: geometry, the per-wave chunk
// loop, row mapping, the balanced-split plan and the body of one decode
// wavefront.  Included by decode.hip (the decode and merge kernels) and by
// varlen.hip (the fused varlen kernel).
#pragma once

#include <cfloat>
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace pa {

constexpr int kMaxTable = 1024;  // block-table entries a partition may span
constexpr float kTau = 8.0f;     // lazy-rescale threshold (log2 units)

template <bool BF16, int D>
struct Geo {
  static constexpr int ELEM = BF16 ? 2 : 4;
  static constexpr int EPV = 16 / ELEM;   // elements per 16-byte vector
  static constexpr int LPT = D / EPV;     // lanes per token row
  static constexpr int TPI = 64 / LPT;    // token rows per wave load
  static constexpr int J = 4;             // tokens per lane row per chunk
  static constexpr int CHUNK = TPI * J;   // tokens per chunk
  static constexpr int NST = ilog2(LPT);  // exchange stages inside a token row
  static constexpr int VPR = D * ELEM / 16;  // 16-byte vectors per head row (== LPT)
};

// Exchange partner of stage k inside a token row of width LPT: lane ^ mask.
// The masks have distinct leading bits, so they form a GF(2) basis of the
// lane index.
template <int LPT>
__host__ __device__ constexpr int stage_mask(int k) {
  if constexpr (LPT == 8) {
    constexpr int m[3] = {7, 2, 1};
    return m[k];
  } else if constexpr (LPT == 16) {
    constexpr int m[4] = {8, 7, 2, 1};
    return m[k];
  } else {
    constexpr int m[5] = {16, 8, 7, 2, 1};
    return m[k];
  }
}

// Head slot permutation: lane c keeps q of head (slot ^ head_mask(c)) in
// slot `slot`.  head_mask(c) collects the coordinates of c along the first
// g stage masks, so the stage-k partner always holds the complementary
// half of heads in the matching slots.
template <int LPT, int LOG2G>
__host__ __device__ constexpr int head_mask(int c) {
  int m = 0;
  for (int k = 0; k < ilog2(LPT); ++k) {
    const int mk = stage_mask<LPT>(k);
    const int lead = ilog2(mk);
    const int a = (c >> lead) & 1;
    c ^= a * mk;
    if (k < LOG2G) m |= a << (LOG2G - 1 - k);
  }
  return m;
}

template <int LPT, int LOG2G>
__host__ __device__ constexpr int rep_lane(int h) {
  for (int c = 0; c < LPT; ++c)
    if (head_mask<LPT, LOG2G>(c) == h) return c;
  return -1;
}

template <int LPT, int LOG2G, int K>
struct Reduce {
  template <int G, int J>
  __device__ __forceinline__ static void run(float (&sc)[G][J]) {
    if constexpr (K < ilog2(LPT)) {
      constexpr int X = stage_mask<LPT>(K);
      if constexpr (K < LOG2G) {
        constexpr int half = G >> (K + 1);
#pragma unroll
        for (int s = 0; s < half; ++s)
#pragma unroll
          for (int j = 0; j < J; ++j) sc[s][j] += xor_lane<X>(sc[s + half][j]);
      } else {
#pragma unroll
        for (int j = 0; j < J; ++j) sc[0][j] += xor_lane<X>(sc[0][j]);
      }
      Reduce<LPT, LOG2G, K + 1>::template run<G, J>(sc);
    }
  }
};

// All lanes of the group of width W receive the value of lane REP(h) of
// their group, for every head h.
template <int W, int LOG2G, int H, int G>
struct BcastHeads {
  template <int N>
  __device__ __forceinline__ static void run(const uint32_t (&src)[N], uint32_t (&dst)[G][N]) {
    if constexpr (H < G) {
      constexpr int rep = rep_lane<W, LOG2G>(H);
      static_assert(rep >= 0, "no lane holds this head");
#pragma unroll
      for (int n = 0; n < N; ++n) dst[H][n] = bcast_in_group<W, rep>(src[n]);
      BcastHeads<W, LOG2G, H + 1, G>::template run<N>(src, dst);
    }
  }
};

template <int W, int LOG2G, int H, int G>
struct BcastHeadsF {
  __device__ __forceinline__ static void run(float src, float (&dst)[G]) {
    if constexpr (H < G) {
      constexpr int rep = rep_lane<W, LOG2G>(H);
      dst[H] = bcast_in_group_f<W, rep>(src);
      BcastHeadsF<W, LOG2G, H + 1, G>::run(src, dst);
    }
  }
};

// Sum (or max) across the token rows of the wave: lanes c, c+LPT, c+2*LPT ...
template <int LPT>
__device__ __forceinline__ float rows_sum(float x) {
  if constexpr (LPT <= 8) x += xor_lane<8>(x);
  if constexpr (LPT <= 16) x += xor_lane<16>(x);
  if constexpr (LPT <= 32) x += xor_lane<32>(x);
  return x;
}
template <int LPT>
__device__ __forceinline__ float rows_max(float x) {
  if constexpr (LPT <= 8) x = fmaxf(x, xor_lane<8>(x));
  if constexpr (LPT <= 16) x = fmaxf(x, xor_lane<16>(x));
  if constexpr (LPT <= 32) x = fmaxf(x, xor_lane<32>(x));
  return x;
}

// Register buffers of the chunk pipeline (prefetch depth S-1).  Chosen so
// the wave keeps >= 2 chunks in flight while the accumulators of its G heads
// still fit the 256 architectural VGPRs.
#ifndef PA_DECODE_STAGES_SMALL_G
#define PA_DECODE_STAGES_SMALL_G 3
#endif
#ifndef PA_DECODE_STAGES_G8
#define PA_DECODE_STAGES_G8 2
#endif
template <bool BF16, int D, int G>
struct DecodeStages {
  static constexpr int value = G <= 4 ? PA_DECODE_STAGES_SMALL_G : (G == 8 ? PA_DECODE_STAGES_G8 : 2);
};

template <bool BF16, int D, int G>
struct DecodeWave {
  using Gm = Geo<BF16, D>;
  static constexpr int EPV = Gm::EPV, LPT = Gm::LPT, J = Gm::J, CHUNK = Gm::CHUNK;
  static constexpr int LOG2G = ilog2(G);
  static_assert((1 << LOG2G) == G, "group must be a power of two");
  static_assert(LOG2G <= Gm::NST, "group larger than the lanes of a token row");

  // per-lane state
  u32x4 qv[G];      // q slots (bf16 pairs, or fp32 bits)
  float o[G][EPV];  // unnormalised output of every head, this lane's dims
  float m;          // reference max of this lane's head and row (log2 units)
  float l;          // sum of probabilities of this lane's head and row
  int lane, row, col, hmask;

  struct Chunk {
    u32x4 k[J];
    u32x4 v[J];
  };

  __device__ __forceinline__ void load(Chunk& ch, const u32x4* __restrict__ kc,
                                       const u32x4* __restrict__ vc, const int32_t* tbl,
                                       int first_blk, int t0, int log2b, int bmask,
                                       int64_t head_off, int64_t row_stride) const {
    const int t = t0 + row * J;
    const int blk = tbl[(t >> log2b) - first_blk];
    const int64_t base = (static_cast<int64_t>(blk) << log2b | (t & bmask)) * row_stride + head_off;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      ch.k[j] = kc[base + j * row_stride];
      ch.v[j] = vc[base + j * row_stride];
    }
  }

  template <bool MASKED>
  __device__ __forceinline__ void compute(Chunk& ch, int t0, int end, float scale_log2) {
    // partial dot products for every (slot, token)
    float sc[G][J];
#pragma unroll
    for (int s = 0; s < G; ++s)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float acc = 0.f;
        if constexpr (BF16) {
          acc = dot2_bf16(qv[s].x, ch.k[j].x, acc);
          acc = dot2_bf16(qv[s].y, ch.k[j].y, acc);
          acc = dot2_bf16(qv[s].z, ch.k[j].z, acc);
          acc = dot2_bf16(qv[s].w, ch.k[j].w, acc);
        } else {
          acc = fmaf(__uint_as_float(qv[s].x), __uint_as_float(ch.k[j].x), acc);
          acc = fmaf(__uint_as_float(qv[s].y), __uint_as_float(ch.k[j].y), acc);
          acc = fmaf(__uint_as_float(qv[s].z), __uint_as_float(ch.k[j].z), acc);
          acc = fmaf(__uint_as_float(qv[s].w), __uint_as_float(ch.k[j].w), acc);
        }
        sc[s][j] = acc;
      }
    Reduce<LPT, LOG2G, 0>::template run<G, J>(sc);

    const int t = t0 + row * J;
    float s[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      s[j] = sc[0][j] * scale_log2;
      if constexpr (MASKED) {
        if (t + j >= end) {
          s[j] = -INFINITY;
          ch.v[j] = u32x4{0u, 0u, 0u, 0u};  // stale slots may hold NaN
        }
      }
    }
    float cmax = s[0];
#pragma unroll
    for (int j = 1; j < J; ++j) cmax = fmaxf(cmax, s[j]);

    if (__any(cmax > m + kTau)) {
      const float mn = fmaxf(m, cmax);
      const float alpha = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      l *= alpha;
      float a[G];
      BcastHeadsF<LPT, LOG2G, 0, G>::run(alpha, a);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPV; ++e) o[h][e] *= a[h];
    }
    const float mref = (m == -INFINITY) ? 0.f : m;

    if constexpr (BF16) {
      uint32_t pp[J / 2];
#pragma unroll
      for (int jp = 0; jp < J / 2; ++jp) {
        pp[jp] = pack_bf16(__builtin_amdgcn_exp2f(s[2 * jp] - mref), __builtin_amdgcn_exp2f(s[2 * jp + 1] - mref));
        l += bf16_lo(pp[jp]) + bf16_hi(pp[jp]);
      }
      uint32_t pb[G][J / 2];
      BcastHeads<LPT, LOG2G, 0, G>::template run<J / 2>(pp, pb);
#pragma unroll
      for (int jp = 0; jp < J / 2; ++jp) {
        const u32x4& v0 = ch.v[2 * jp];
        const u32x4& v1 = ch.v[2 * jp + 1];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a = pair_lo(word(v0, w), word(v1, w));
          const uint32_t b = pair_hi(word(v0, w), word(v1, w));
#pragma unroll
          for (int h = 0; h < G; ++h) {
            o[h][2 * w] = dot2_bf16(pb[h][jp], a, o[h][2 * w]);
            o[h][2 * w + 1] = dot2_bf16(pb[h][jp], b, o[h][2 * w + 1]);
          }
        }
      }
    } else {
      uint32_t pu[J];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const float p = __builtin_amdgcn_exp2f(s[j] - mref);
        l += p;
        pu[j] = __float_as_uint(p);
      }
      uint32_t pb[G][J];
      BcastHeads<LPT, LOG2G, 0, G>::template run<J>(pu, pb);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const float v0 = __uint_as_float(ch.v[j].x), v1 = __uint_as_float(ch.v[j].y);
        const float v2 = __uint_as_float(ch.v[j].z), v3 = __uint_as_float(ch.v[j].w);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = __uint_as_float(pb[h][j]);
          o[h][0] = fmaf(p, v0, o[h][0]);
          o[h][1] = fmaf(p, v1, o[h][1]);
          o[h][2] = fmaf(p, v2, o[h][2]);
          o[h][3] = fmaf(p, v3, o[h][3]);
        }
      }
    }
  }
};

// Which query/output row, block-table row and context length grid row z
// stands for (see DecodeArgs::mode); active is false for rows another
// kernel handles.
struct RowInfo {
  int q_row, table_row, ctx;
  bool active;
};

__device__ __forceinline__ RowInfo row_info(const DecodeArgs& a, int z, int block_size) {
  RowInfo r{z, z, 0, true};
  if (a.mode == kRowsDecode) {
    r.ctx = a.context_lens[z];
  } else if (a.mode == kRowsVarlenDecode) {
    const int q0 = a.query_start_loc[z], q1 = a.query_start_loc[z + 1];
    r.active = (q1 - q0) == 1;
    r.q_row = q0;
    r.ctx = a.context_lens[z];
  } else {
    // segment s with qsl[s] <= z < qsl[s+1]: binary search over the offsets
    int lo = 0, hi = a.num_seqs;  // invariant: qsl[lo] <= z < qsl[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.query_start_loc[mid] <= z) lo = mid; else hi = mid;
    }
    const int q0 = a.query_start_loc[lo], q1 = a.query_start_loc[lo + 1];
    r.table_row = lo;
    r.ctx = a.context_lens[lo] - (q1 - q0) + (z - q0) + 1;
  }
  r.ctx = clampi(r.ctx, 0, min(a.max_context_len, a.max_blocks_per_seq * block_size));
  return r;
}

// A wave's share of a balanced split (see DecodeArgs::balanced).
struct PlanEntry {
  RowInfo ri;
  int row, part, nparts, first_slot, c0, c1;
  bool valid;
};

// Wave-wide sum / max of an int: DPP steps inside each 16-lane row, then
// the four row results read out as scalars (no LDS traffic).
__device__ __forceinline__ int row_sum_i(int x) {
  x += static_cast<int>(dpp_u32<DPP_QUAD_XOR1>(x));
  x += static_cast<int>(dpp_u32<DPP_QUAD_XOR2>(x));
  x += static_cast<int>(dpp_u32<DPP_ROW_HALF_MIRROR>(x));
  x += static_cast<int>(dpp_u32<DPP_ROW_ROR8>(x));
  return x;
}

__device__ __forceinline__ int wave_sum(int x) {
  x = row_sum_i(x);
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
         __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

__device__ __forceinline__ int wave_max(int x) {
  x = max(x, static_cast<int>(dpp_u32<DPP_QUAD_XOR1>(x)));
  x = max(x, static_cast<int>(dpp_u32<DPP_QUAD_XOR2>(x)));
  x = max(x, static_cast<int>(dpp_u32<DPP_ROW_HALF_MIRROR>(x)));
  x = max(x, static_cast<int>(dpp_u32<DPP_ROW_ROR8>(x)));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

__device__ __forceinline__ float wave_sum_f(float x) {
  x += xor_lane<1>(x);
  x += xor_lane<2>(x);
  x += xor_lane<7>(x);
  x += xor_lane<8>(x);
  const auto rl = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l)); };
  return (rl(0) + rl(16)) + (rl(32) + rl(48));
}

__device__ __forceinline__ float wave_max_f(float x) {
  x = fmaxf(x, xor_lane<1>(x));
  x = fmaxf(x, xor_lane<2>(x));
  x = fmaxf(x, xor_lane<7>(x));
  x = fmaxf(x, xor_lane<8>(x));
  const auto rl = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l)); };
  return fmaxf(fmaxf(rl(0), rl(16)), fmaxf(rl(32), rl(48)));
}

// Exclusive prefix sum over the lanes: inclusive scans inside each 16-lane
// row with DPP row shifts (lanes shifted in from outside the row read 0),
// then the totals of the rows below added as scalars.
__device__ __forceinline__ int wave_exclusive_scan(int x) {
  int v = x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  const int below = (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
  return v + below - x;
}

__device__ __forceinline__ uint32_t div_ceil(uint32_t c, uint32_t t) { return (c + t - 1) / t; }

// Partitions a row of c chunks gets under a per-wave cap of t chunks.
__device__ __forceinline__ int row_parts(int c, bool active, int t) {
  return active ? max(1, static_cast<int>(div_ceil(c, t))) : 0;
}

template <int RPL>
__device__ __forceinline__ int plan_count(const int (&c)[RPL], const bool (&act)[RPL], int t) {
  int n = 0;
#pragma unroll
  for (int i = 0; i < RPL; ++i) n += row_parts(c[i], act[i], t);
  return wave_sum(n);
}

// Smallest per-wave cap t whose plan fits `slots` waves (cmax when none
// does).  Since ceil(c/t) < c/t + 1, a cap t fits as soon as total/t + rows
// <= slots, which bounds the search to a few steps.
template <int RPL>
__device__ int plan_cap(const int (&c)[RPL], const bool (&act)[RPL], int total, int rows,
                        int cmax, int slots) {
  int lo = max(1, static_cast<int>(div_ceil(total, slots)));
  int hi = cmax;
  if (slots > rows) hi = min(hi, max(lo, static_cast<int>(div_ceil(total, slots - rows))));
  if (lo >= hi) return min(lo, cmax);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (plan_count(c, act, mid) <= slots) hi = mid; else lo = mid + 1;
  }
  return hi;
}

// Context length and q row of row r for a plan (row modes kRowsDecode and
// kRowsVarlenDecode); -1 for a row the decode kernels skip.  r is in range.
__device__ __forceinline__ int plan_row(const DecodeArgs& a, int r, int block_size, int& q_row) {
  int ctx;
  if (a.mode == kRowsDecode) {
    q_row = r;
    ctx = a.context_lens[r];
  } else {
    const int q0 = a.query_start_loc[r], q1 = a.query_start_loc[r + 1];
    q_row = q0;
    ctx = (q1 - q0) == 1 ? a.context_lens[r] : -1;
  }
  return ctx < 0 ? -1 : clampi(ctx, 0, min(a.max_context_len, a.max_blocks_per_seq * block_size));
}

// Every wave evaluates the whole plan from the rows' lengths (a few loads
// per lane, served by L2 after the first waves) and picks the row and
// partition of work slot y.  Lane l owns rows l*RPL .. l*RPL+RPL-1, so slot
// order is row order.  The cap is the smallest one for which the rows fit
// one wave per SIMD (plan_share per KV head); when that cap is more than
// 2.5x the cap for two waves per SIMD, two waves per SIMD finish sooner
// despite sharing the SIMD unevenly, and that plan is used.
template <int CHUNK, int RPL>
__device__ PlanEntry plan_lookup(const DecodeArgs& a, int y, int block_size) {
  const int lane = threadIdx.x & 63;
  const int r0 = lane * RPL;
  int chunks[RPL], ctx[RPL], qrow[RPL];
  bool act[RPL];
  // loads first (row index clamped into range), masks after
#pragma unroll
  for (int i = 0; i < RPL; ++i) ctx[i] = plan_row(a, min(r0 + i, a.num_rows - 1), block_size, qrow[i]);
  int lane_chunks = 0, lane_max = 0, lane_rows = 0;
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    act[i] = r0 + i < a.num_rows && ctx[i] >= 0;
    chunks[i] = act[i] ? (ctx[i] + CHUNK - 1) / CHUNK : 0;
    lane_chunks += chunks[i];
    lane_max = max(lane_max, chunks[i]);
    lane_rows += act[i] ? 1 : 0;
  }
  const int total = wave_sum(lane_chunks);
  const int cmax = max(1, wave_max(lane_max));
  const int rows = wave_sum(lane_rows);
  const int s1 = a.plan_share, s2 = a.plan_share2;
  int t = plan_cap(chunks, act, total, rows, cmax, s1);
  // the two-per-SIMD cap is at least ceil(total / s2): search it only when
  // that bound leaves it able to win
  if (s2 > s1 && 2 * t > 5 * max(1, static_cast<int>(div_ceil(total, s2)))) {
    const int t2 = plan_cap(chunks, act, total, rows, cmax, s2);
    if (2 * t > 5 * t2) t = t2;
  }
  t = min(t, max(1, a.plan_max_tokens / CHUNK));  // block-table staging limit

  int n[RPL];
  int lane_n = 0;
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    n[i] = row_parts(chunks[i], act[i], t);
    lane_n += n[i];
  }
  int pre = wave_exclusive_scan(lane_n);
  int hit = -1, hit_pre = 0, hc = 0, hn = 0, hctx = 0, hq = 0;
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    if (y >= pre && y < pre + n[i]) {
      hit = i;
      hit_pre = pre;
      hc = chunks[i];
      hn = n[i];
      hctx = ctx[i];
      hq = qrow[i];
    }
    pre += n[i];
  }
  PlanEntry e{};
  const uint64_t mask = __ballot(hit >= 0);
  e.valid = mask != 0;
  if (!e.valid) return e;
  const int src = __builtin_ctzll(mask);
  e.row = __builtin_amdgcn_readlane(r0 + hit, src);
  e.first_slot = __builtin_amdgcn_readlane(hit_pre, src);
  e.nparts = __builtin_amdgcn_readlane(hn, src);
  const int c = __builtin_amdgcn_readlane(hc, src);
  e.ri.ctx = __builtin_amdgcn_readlane(hctx, src);
  e.ri.q_row = __builtin_amdgcn_readlane(hq, src);
  e.ri.table_row = e.row;
  e.ri.active = true;
  e.part = y - e.first_slot;
  // chunk range [floor(p c / n), floor((p+1) c / n)) with c = q n + r:
  // floor(p c / n) = p q + floor(p r / n), and p r < n^2 < 2^32
  const uint32_t q = static_cast<uint32_t>(c) / e.nparts, rem = static_cast<uint32_t>(c) % e.nparts;
  const uint32_t p = e.part;
  e.c0 = static_cast<int>(p * q + p * rem / e.nparts);
  e.c1 = static_cast<int>((p + 1) * q + (p + 1) * rem / e.nparts);
  return e;
}

template <int CHUNK>
__device__ __forceinline__ PlanEntry plan_lookup(const DecodeArgs& a, int y, int block_size) {
  if (a.num_rows <= 64) return plan_lookup<CHUNK, 1>(a, y, block_size);
  if (a.num_rows <= 256) return plan_lookup<CHUNK, 4>(a, y, block_size);
  return plan_lookup<CHUNK, kPlanMaxRows / 64>(a, y, block_size);
}

// The work of one decode wavefront: KV head g, work slot y (balanced split)
// or partition y of row z (fixed split).  tbl is this wave's block-table
// staging area in LDS (kMaxTable entries).  Used by the decode kernel (one
// wave per workgroup) and by the fused varlen kernel (eight independent
// waves per workgroup), so it synchronises only its own wave.
template <bool BF16, int D, int G>
__device__ __forceinline__ void decode_partition_body(const DecodeArgs& a, int g, int y, int z,
                                                      int32_t* tbl, int32_t num_kv_heads,
                                                      int32_t num_blocks, int32_t log2b) {
  using W = DecodeWave<BF16, D, G>;
  using Gm = Geo<BF16, D>;
  constexpr int EPV = Gm::EPV, LPT = Gm::LPT, CHUNK = Gm::CHUNK, VPR = Gm::VPR;
  const int H = num_kv_heads * G;
  const int B = 1 << log2b;
  const int lane = threadIdx.x & 63;

  // this wave's row, partition and token range [start, end)
  RowInfo ri;
  int zrow, part, nparts, start, end;
  int64_t part_base;  // workspace index of (this partition, query head g*G)
  if (a.balanced) {
    const PlanEntry pe = plan_lookup<CHUNK>(a, y, B);
    if (!pe.valid) return;
    ri = pe.ri;
    zrow = pe.row;
    part = pe.part;
    nparts = pe.nparts;
    start = pe.c0 * CHUNK;
    end = min(pe.c1 * CHUNK, ri.ctx);
    part_base = static_cast<int64_t>(y) * H + g * G;
    if (part == 0 && g == 0 && lane == 0)
      *reinterpret_cast<int2*>(a.plan + 2 * static_cast<int64_t>(zrow)) = make_int2(pe.first_slot, nparts);
  } else {
    part = y;
    zrow = z;
    ri = row_info(a, zrow, B);
    const int P = a.partition_size;
    nparts = (ri.ctx + P - 1) / P;
    start = part * P;
    end = min(start + P, ri.ctx);
    part_base = (static_cast<int64_t>(zrow) * H + g * G) * a.max_partitions + part;
  }
  if (!ri.active) return;
  const int seq = ri.q_row;  // q / out row
  const int ctx = ri.ctx;

  if (ctx == 0) {
    // nothing to attend: partition 0 writes a zero row for each head
    if (part == 0) {
      const int row = lane / LPT, col = lane % LPT;
      for (int h = row; h < G; h += Gm::TPI) {
        const int64_t off = (static_cast<int64_t>(seq) * H + g * G + h) * VPR + col;
        static_cast<u32x4*>(a.out)[off] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    return;
  }
  if (part >= nparts) return;

  // q loads first, so they are in flight together with the table loads
  W w;
  w.lane = lane;
  w.row = lane / LPT;
  w.col = lane % LPT;
  w.hmask = head_mask<LPT, ilog2(G)>(w.col);
  {
    const u32x4* qp = static_cast<const u32x4*>(a.q);
#pragma unroll
    for (int s = 0; s < G; ++s) {
      const int h = g * G + (s ^ w.hmask);
      w.qv[s] = qp[(static_cast<int64_t>(seq) * H + h) * VPR + w.col];
    }
  }

  const int nchunks = (end - start + CHUNK - 1) / CHUNK;
  const int first_blk = start >> log2b;
  const int last_blk = (start + nchunks * CHUNK - 1) >> log2b;
  const int nblk_ctx = (ctx + B - 1) >> log2b;
  const int32_t* trow = a.block_tables + static_cast<int64_t>(ri.table_row) * a.max_blocks_per_seq;
  for (int i = lane; i <= last_blk - first_blk; i += 64) {
    const int bi = first_blk + i;
    tbl[i] = bi < nblk_ctx ? clampi(trow[bi], 0, num_blocks - 1) : 0;
  }
  // the table is written and read by this wave only; LDS executes one
  // wave's accesses in order, so a compiler-level fence suffices
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPV; ++e) w.o[h][e] = 0.f;
  w.m = -INFINITY;
  w.l = 0.f;

  const float scale_log2 = a.scale * kLog2e;
  const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
  const u32x4* vc = static_cast<const u32x4*>(a.v_cache);
  const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * VPR;
  const int64_t head_off = static_cast<int64_t>(g) * VPR + w.col;
  const int bmask = B - 1;

  // Software pipeline over the partition's chunks with S register buffers:
  // the loads of chunk c+S-1 are issued before chunk c is computed, so up to
  // S-1 chunks (S-1 x 8 KiB for bf16 D=128) are in flight per wavefront.
  // Buffer indices are compile-time, so the ring stays in registers.  Loads
  // past the last chunk are clamped onto it instead of branched around: they
  // hit the L2 lines just fetched and keep the steady-state loop branch-free.
  // Only the final S chunks are computed with the length mask.
  constexpr int S = DecodeStages<BF16, D, G>::value;
  typename W::Chunk buf[S];
  const int last = nchunks - 1;
  auto load_chunk = [&](typename W::Chunk& ch, int ci) {
    ci = ci < last ? ci : last;
    w.load(ch, kc, vc, tbl, first_blk, start + ci * CHUNK, log2b, bmask, head_off, row_stride);
  };
#pragma unroll
  for (int s = 0; s < S - 1; ++s) load_chunk(buf[s], s);
  int c = 0;
  for (; c + S < nchunks; c += S) {  // chunks c .. c+S-1 are full
#pragma unroll
    for (int s = 0; s < S; ++s) {
      load_chunk(buf[(s + S - 1) % S], c + s + S - 1);
      w.template compute<false>(buf[s], start + (c + s) * CHUNK, end, scale_log2);
    }
  }
  // 1..S chunks remain; chunk c+s sits in buf[s]
  load_chunk(buf[S - 1], c + S - 1);
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (c + s < nchunks) w.template compute<true>(buf[s], start + (c + s) * CHUNK, end, scale_log2);

  // merge the token rows: per head, bring (m, l) of the head's lane to every
  // lane of the row, then combine rows with the usual max-rescale.
  constexpr int LOG2G = ilog2(G);
  float mh[G], lh[G];
  BcastHeadsF<LPT, LOG2G, 0, G>::run(w.m, mh);
  BcastHeadsF<LPT, LOG2G, 0, G>::run(w.l, lh);
  float L[G], M[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    M[h] = rows_max<LPT>(mh[h]);
    const float f = (mh[h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mh[h] - M[h]);
    L[h] = rows_sum<LPT>(f * lh[h]);
#pragma unroll
    for (int e = 0; e < EPV; ++e) w.o[h][e] = rows_sum<LPT>(f * w.o[h][e]);
  }

  // every row now holds the merged partition result; row r stores heads
  // h = r, r + TPI, ...
  const int row = w.row, col = w.col;
  if (nparts == 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (h % Gm::TPI != row) continue;
      const float inv = 1.f / L[h];
      const int64_t off = (static_cast<int64_t>(seq) * H + g * G + h) * VPR + col;
      u32x4 r;
      if constexpr (BF16) {
        r.x = pack_bf16(w.o[h][0] * inv, w.o[h][1] * inv);
        r.y = pack_bf16(w.o[h][2] * inv, w.o[h][3] * inv);
        r.z = pack_bf16(w.o[h][4] * inv, w.o[h][5] * inv);
        r.w = pack_bf16(w.o[h][6] * inv, w.o[h][7] * inv);
      } else {
        r.x = __float_as_uint(w.o[h][0] * inv);
        r.y = __float_as_uint(w.o[h][1] * inv);
        r.z = __float_as_uint(w.o[h][2] * inv);
        r.w = __float_as_uint(w.o[h][3] * inv);
      }
      static_cast<u32x4*>(a.out)[off] = r;
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (h % Gm::TPI != row) continue;
      const int64_t idx = part_base + (a.balanced ? h : static_cast<int64_t>(h) * a.max_partitions);
      float* po = a.part_o + idx * D + col * EPV;
#pragma unroll
      for (int e = 0; e < EPV; e += 4)
        *reinterpret_cast<float4*>(po + e) = make_float4(w.o[h][e], w.o[h][e + 1], w.o[h][e + 2], w.o[h][e + 3]);
      if (col == 0) *reinterpret_cast<float2*>(a.part_ml + idx * 2) = make_float2(M[h], L[h]);
    }
  }
}

}  // namespace pa
