// Device code of the split-K paged decode: geometry, the per-wave chunk
// loop, row mapping, the balanced-split plan and the body of one decode
// wavefront.  Included by decode.hip (the decode and merge kernels) and by
// varlen.hip (the fused varlen kernel).
#pragma once

#include <cfloat>
#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pa {

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
// FP8 chunks carry half the bytes of bf16 ones, so two more are kept in
// flight for the same bytes per wave.
template <bool BF16, int D, int G, bool FP8 = false>
struct DecodeStages {
  static constexpr int value = FP8 ? (G <= 4 ? PA_DECODE_STAGES_SMALL_G + 2 : (G == 8 ? 3 : 2))
                                   : (G <= 4 ? PA_DECODE_STAGES_SMALL_G : (G == 8 ? PA_DECODE_STAGES_G8 : 2));
};

// FP8 (E4M3 caches): the lane geometry of bf16 (each lane covers the same 8
// head dims of a token row) with 8-byte loads; the codes are converted to
// bf16 (exactly: every E4M3 value is a bf16 value) before the bf16 compute,
// and the per-KV-head scales are applied to the scores and the output.
template <bool BF16, int D, int G, bool FP8 = false, bool HOIST = true>
struct DecodeWave {
  using Gm = Geo<BF16, D>;
  static_assert(!FP8 || BF16, "FP8 caches use the bf16 lane geometry");
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

  using Vec = typename std::conditional<FP8, uint2, u32x4>::type;  // one lane's piece of a row
  static constexpr int VPH = FP8 ? D / 8 : Gm::VPR;  // Vec per head row
  struct Chunk {
    Vec k[J];
    Vec v[J];
  };

  // Offsets of this lane's J tokens inside their slot rows, when they are
  // the same for every chunk (hoist): token j of lane row `row` has in-block
  // position p = (t0 mod B) + row*J + j with t0 a multiple of CHUNK, so
  // kv_head_pos depends on p only through p & rot, which drops t0 whenever
  // B <= CHUNK (t0 mod B = 0) or rot < CHUNK (t0 mod B a multiple of
  // CHUNK, hence of rot + 1).  HOIST = false keeps the per-chunk
  // computation (and four registers) where a kernel is short of them.
  int hoff[J];
  bool hoist;
  __device__ __forceinline__ void prep(int g, int rot, int log2b, int row_stride) {
    const int B = 1 << log2b;
    hoist = HOIST && (B <= CHUNK || rot < CHUNK);
#pragma unroll
    for (int j = 0; j < J; ++j)
      hoff[j] = j * row_stride + kv_head_pos(g, (row * J + j) & (B - 1), rot) * VPH + col;
  }

  // Chunk starting at token t0 of a segment whose block-table entry for
  // block b sits at tbl[tb + b].
  // KV head g sits at head position kv_head_pos(g, p, rot) of the slot row
  // of in-block position p.
  // row_stride: Vec per slot row (num_kv_heads * VPH)
  __device__ __forceinline__ void load(Chunk& ch, const Vec* __restrict__ kc,
                                       const Vec* __restrict__ vc, const int32_t* tbl,
                                       int tb, int t0, int log2b, int bmask, int g, int rot,
                                       int64_t row_stride) const {
    const int t = t0 + row * J;
    const int blk = tbl[tb + (t >> log2b)];
    const int64_t slot = static_cast<int64_t>(blk) << log2b | (t & bmask);
    if (HOIST && hoist) {
      const Vec* kb = kc + slot * row_stride;
      const Vec* vb = vc + slot * row_stride;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        ch.k[j] = kb[hoff[j]];
        ch.v[j] = vb[hoff[j]];
      }
    } else {
      const int64_t base = slot * row_stride + col;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int64_t off = base + j * row_stride + kv_head_pos(g, (t + j) & bmask, rot) * VPH;
        ch.k[j] = kc[off];
        ch.v[j] = vc[off];
      }
    }
  }

  // 8 E4M3 codes -> 8 bf16, element order kept
  __device__ __forceinline__ static u32x4 widen(uint2 c) {
    auto lo = [](uint32_t w) {
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    };
    auto hi = [](uint32_t w) {
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    };
    return u32x4{lo(c.x), hi(c.x), lo(c.y), hi(c.y)};
  }

  // Token np of the chunk (if any) takes nk / nv instead of what was loaded:
  // the fused append's new token, which is in the last chunk of its row and
  // so always in a masked chunk (np = -1: none).
  template <bool MASKED>
  __device__ __forceinline__ void compute(Chunk& c8, int t0, int end, float scale_log2, int np,
                                          const u32x4& nk, const u32x4& nv) {
    if constexpr (FP8) {
      typename DecodeWave<BF16, D, G, false>::Chunk ch;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        ch.k[j] = widen(c8.k[j]);
        ch.v[j] = widen(c8.v[j]);
      }
      if constexpr (MASKED) substitute(ch.k, ch.v, t0, np, nk, nv);
      compute_rows<MASKED>(ch.k, ch.v, t0, end, scale_log2);
    } else {
      if constexpr (MASKED) substitute(c8.k, c8.v, t0, np, nk, nv);
      compute_rows<MASKED>(c8.k, c8.v, t0, end, scale_log2);
    }
  }

  __device__ __forceinline__ void substitute(u32x4 (&kk)[J], u32x4 (&vv)[J], int t0, int np,
                                             const u32x4& nk, const u32x4& nv) const {
    const int t = t0 + row * J;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (t + j == np) {
        kk[j] = nk;
        vv[j] = nv;
      }
    }
  }

  template <bool MASKED>
  __device__ __forceinline__ void compute_rows(const u32x4 (&kk)[J], u32x4 (&vv)[J], int t0, int end,
                                               float scale_log2) {
    // partial dot products for every (slot, token)
    float sc[G][J];
#pragma unroll
    for (int s = 0; s < G; ++s)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float acc = 0.f;
        if constexpr (BF16) {
          acc = dot2_bf16(qv[s].x, kk[j].x, acc);
          acc = dot2_bf16(qv[s].y, kk[j].y, acc);
          acc = dot2_bf16(qv[s].z, kk[j].z, acc);
          acc = dot2_bf16(qv[s].w, kk[j].w, acc);
        } else {
          acc = fmaf(__uint_as_float(qv[s].x), __uint_as_float(kk[j].x), acc);
          acc = fmaf(__uint_as_float(qv[s].y), __uint_as_float(kk[j].y), acc);
          acc = fmaf(__uint_as_float(qv[s].z), __uint_as_float(kk[j].z), acc);
          acc = fmaf(__uint_as_float(qv[s].w), __uint_as_float(kk[j].w), acc);
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
          vv[j] = u32x4{0u, 0u, 0u, 0u};  // stale slots may hold NaN
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
        const u32x4& v0 = vv[2 * jp];
        const u32x4& v1 = vv[2 * jp + 1];
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
        const float v0 = __uint_as_float(vv[j].x), v1 = __uint_as_float(vv[j].y);
        const float v2 = __uint_as_float(vv[j].z), v3 = __uint_as_float(vv[j].w);
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


// ---- wave work lists ------------------------------------------------------
//
// A decode wave works through a list of row segments kept at the start of
// its LDS area, kSegInts ints each, followed by the block-table entries of
// all of them (the entries of segment s start at table_start + eoff).
enum : int {
  kSegRow = 0,    // work row, | kSegFinal when the segment is the whole row
  kSegQRow = 1,   // q / out row
  kSegTok0 = 2,   // first token (a multiple of the chunk)
  kSegEnd = 3,    // one past the last token
  kSegN = 4,      // chunks
  kSegEoff = 5,   // first table entry, relative to the table start
  kSegTable = 6,  // block-table row
  kSegCtx = 7,    // the row's context length
};
constexpr int kSegFinal = 1 << 30;

struct WaveWork {
  int nseg;  // segments
  int K;     // chunks over all segments
  int E;     // table entries over all segments
  // plan phase stamps (timeline build)
  PA_TL(unsigned long long phase[4] = {0, 0, 0, 0};)
};

__device__ __forceinline__ void put_seg(int32_t* lds, int s, int row_flags, int q_row, int tok0,
                                        int end, int n, int eoff, int table_row, int ctx) {
  int4* d = reinterpret_cast<int4*>(lds + s * kSegInts);
  d[0] = make_int4(row_flags, q_row, tok0, end);
  d[1] = make_int4(n, eoff, table_row, ctx);
}

// floor(y T / W) in 32-bit arithmetic: with T = q W + r, y T / W = y q +
// y r / W, where y q <= T < 2^30 and y r < W^2 < 2^32.
__device__ __forceinline__ int split_point(uint32_t y, uint32_t T, uint32_t W) {
  const uint32_t q = T / W, r = T % W;
  return static_cast<int>(y * q + (y * r) / W);
}

// The wave whose range holds cost unit x: the largest y with
// floor(y T / W) <= x, i.e. y = ceil((x + 1) W / T) - 1.
__device__ __forceinline__ int wave_of(int x, int T, int W) {
  return static_cast<int>((static_cast<uint64_t>(x + 1) * W - 1) / static_cast<uint64_t>(T));
}

// Table entries of chunks [c0, c1) of a row: blocks of tokens
// [c0 * CHUNK, c1 * CHUNK).
template <int CHUNK>
__device__ __forceinline__ int seg_blocks(int c0, int c1, int log2b) {
  return ((c1 * CHUNK - 1) >> log2b) - ((c0 * CHUNK) >> log2b) + 1;
}

// Balanced split (DecodeArgs::balanced): wave y's segments.  Every wave
// evaluates the whole line from the rows' lengths (RPL rows per lane: rows
// lane * RPL + i, length ctx[i], -1 for no row, q/out row qrow[i]), writes
// its segments to lds, and, as owner of a row's first unit, the row's plan
// entry (when write_plan) and, for an empty context, calls zero_row(q_row).
template <int CHUNK, int RPL, class ZeroRow>
__device__ WaveWork split_rows(const DecodeArgs& a, int y, int log2b, int32_t* lds,
                               bool write_plan, ZeroRow&& zero_row, const int (&ctx)[RPL],
                               const int (&qrow)[RPL]) {
  const int lane = threadIdx.x & 63;
  const int r0 = lane * RPL;
  constexpr int Q = kPlanChunkCost, beta = kPlanRowCost;
  int cost[RPL];
  PA_TL(const unsigned long long p1 = __builtin_amdgcn_s_memrealtime();)
  int lane_cost = 0;
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    cost[i] = ctx[i] >= 0 ? beta + Q * ((ctx[i] + CHUNK - 1) / CHUNK) : 0;
    lane_cost += cost[i];
  }
  const int pre = wave_exclusive_scan(lane_cost);
  const int T = __builtin_amdgcn_readlane(pre + lane_cost, 63);
  PA_TL(const unsigned long long p2 = __builtin_amdgcn_s_memrealtime();)
  WaveWork ww{0, 0, 0};
  if (T == 0) return ww;
  // W: enough waves to keep every range within plan_max_cost, at least
  // plan_share, at most the launch's waves, and few enough that every range
  // spans >= Q units: then every wave between the first and the last of a
  // row holds a chunk of it, so a row's segments sit on consecutive waves
  int W = max((T + a.plan_max_cost - 1) / a.plan_max_cost, a.plan_share);
  W = min(min(W, a.max_partitions), max(1, T / Q));
  if (y >= W) return ww;
  const int lo = split_point(y, T, W), hi = split_point(y + 1, T, W);
  PA_TL(asm volatile("" ::"v"(lo), "v"(hi));
        const unsigned long long p3 = __builtin_amdgcn_s_memrealtime();)

  int seg_lo[RPL], seg_hi[RPL];
  int lane_seg = 0, lane_k = 0, lane_e = 0;
  int p = pre;  // first unit of row r0 + i
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    seg_lo[i] = seg_hi[i] = 0;
    if (ctx[i] >= 0) {
      const int c = (ctx[i] + CHUNK - 1) / CHUNK;
      const int x0 = p + beta;  // first unit of chunk 0
      if (p >= lo && p < hi) {
        if (c == 0) zero_row(qrow[i]);
        if (write_plan) {
          int2 e = make_int2(0, 0);
          if (c > 0) {
            const int yf = wave_of(x0, T, W), yl = wave_of(x0 + Q * (c - 1), T, W);
            e = make_int2(yf + r0 + i, yl - yf + 1);
          }
          *reinterpret_cast<int2*>(a.plan + 2 * static_cast<int64_t>(r0 + i)) = e;
          if (a.share)  // a plan that found no shared prefix
            *reinterpret_cast<int2*>(a.plan_sh + 2 * static_cast<int64_t>(r0 + i)) = make_int2(0, 0);
        }
      }
      // chunks whose first unit x0 + Q j lies in [lo, hi)
      const int jl = lo > x0 ? (lo - x0 + Q - 1) / Q : 0;
      const int jh = hi > x0 ? min(c, (hi - x0 + Q - 1) / Q) : 0;
      if (jl < jh) {
        seg_lo[i] = jl;
        seg_hi[i] = jh;
        ++lane_seg;
        lane_k += jh - jl;
        lane_e += seg_blocks<CHUNK>(jl, jh, log2b);
      }
    }
    p += cost[i];
  }
  const int seg_pre = wave_exclusive_scan(lane_seg);
  const int e_pre = wave_exclusive_scan(lane_e);
  ww.nseg = __builtin_amdgcn_readlane(seg_pre + lane_seg, 63);
  ww.E = __builtin_amdgcn_readlane(e_pre + lane_e, 63);
  ww.K = wave_sum(lane_k);
  // the split bounds every range by plan_max_cost units, which keeps the
  // list and its table inside the LDS area; checked again here so that an
  // inconsistent argument block can never write past it
  if (ww.nseg * kSegInts + ww.E > kDecodeLdsInts) {
    ww.nseg = ww.K = ww.E = 0;
    return ww;
  }
  PA_TL(ww.phase[0] = p1; ww.phase[1] = p2; ww.phase[2] = p3;
        ww.phase[3] = __builtin_amdgcn_s_memrealtime();)
  int sidx = seg_pre, eoff = e_pre;
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    if (seg_lo[i] < seg_hi[i]) {
      const int c = (ctx[i] + CHUNK - 1) / CHUNK;
      const int final_flag = (seg_lo[i] == 0 && seg_hi[i] == c) ? kSegFinal : 0;
      put_seg(lds, sidx, (r0 + i) | final_flag, qrow[i], seg_lo[i] * CHUNK,
              min(seg_hi[i] * CHUNK, ctx[i]), seg_hi[i] - seg_lo[i], eoff, r0 + i, ctx[i]);
      ++sidx;
      eoff += seg_blocks<CHUNK>(seg_lo[i], seg_hi[i], log2b);
    }
  }
  return ww;
}

// The balanced split of the rows' lengths as they stand in memory (a few
// loads served by L2 after the first waves).
template <int CHUNK, int RPL, class ZeroRow>
__device__ WaveWork even_split(const DecodeArgs& a, int y, int block_size, int log2b,
                               int32_t* lds, bool write_plan, ZeroRow&& zero_row) {
  const int r0 = (threadIdx.x & 63) * RPL;
  int ctx[RPL], qrow[RPL];
  // loads first (row index clamped into range), masks after
#pragma unroll
  for (int i = 0; i < RPL; ++i) ctx[i] = plan_row(a, min(r0 + i, a.num_rows - 1), block_size, qrow[i]);
#pragma unroll
  for (int i = 0; i < RPL; ++i)
    if (r0 + i >= a.num_rows) ctx[i] = -1;
  return split_rows<CHUNK, RPL>(a, y, log2b, lds, write_plan, zero_row, ctx, qrow);
}

template <int CHUNK, class ZeroRow>
__device__ __forceinline__ WaveWork even_split(const DecodeArgs& a, int y, int block_size, int log2b,
                                               int32_t* lds, bool write_plan, ZeroRow&& zero_row) {
  if (a.num_rows <= 64) return even_split<CHUNK, 1>(a, y, block_size, log2b, lds, write_plan, zero_row);
  if (a.num_rows <= 256) return even_split<CHUNK, 4>(a, y, block_size, log2b, lds, write_plan, zero_row);
  return even_split<CHUNK, kPlanMaxRows / 64>(a, y, block_size, log2b, lds, write_plan, zero_row);
}

// Copies the block-table entries of all segments into LDS after the list,
// lanes over entries (4 loads in flight per lane), each lane finding its
// entry's segment by binary search over the list.  Entries past a
// segment's context read 0; the others are clamped into [0, num_blocks).
__device__ __forceinline__ void stage_tables(const DecodeArgs& a, int32_t* lds, const WaveWork& ww,
                                             int log2b, int32_t num_blocks) {
  const int lane = threadIdx.x & 63;
  const int tb0 = ww.nseg * kSegInts;
  const int B = 1 << log2b;
  for (int e0 = 0; e0 < ww.E; e0 += 256) {
    int val[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * 64 + lane;
      val[u] = 0;
      if (e < ww.E) {
        int lo = 0, hi = ww.nseg - 1;  // the last segment with eoff <= e
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (lds[mid * kSegInts + kSegEoff] <= e) lo = mid; else hi = mid - 1;
        }
        const int* d = lds + lo * kSegInts;
        const int bi = (d[kSegTok0] >> log2b) + (e - d[kSegEoff]);
        const int nblk = (d[kSegEnd] + B - 1) >> log2b;
        if (bi < nblk)
          val[u] = clampi(a.block_tables[static_cast<int64_t>(d[kSegTable]) * a.max_blocks_per_seq + bi],
                          0, num_blocks - 1);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * 64 + lane;
      if (e < ww.E) lds[tb0 + e] = val[u];
    }
  }
}

// The work of one decode wavefront: KV head g and, with the balanced split,
// range y of the line (every wave of the launch), or partition y of row z
// (fixed split).  lds is this wave's kDecodeLdsInts area.  Used by the
// decode kernel (one wave per workgroup) and by the fused varlen kernel
// (four independent waves per workgroup), so it synchronises only its own
// wave.
template <bool BF16, int D, int G, bool FP8 = false, bool HOIST = true>
__device__ __forceinline__ void decode_partition_body(const DecodeArgs& a, int g, int y, int z,
                                                      int32_t* lds, int32_t num_kv_heads,
                                                      int32_t num_blocks, int32_t log2b) {
  using W = DecodeWave<BF16, D, G, FP8, HOIST>;
  using Gm = Geo<BF16, D>;
  constexpr int EPV = Gm::EPV, LPT = Gm::LPT, CHUNK = Gm::CHUNK, VPR = Gm::VPR;
  static_assert(CHUNK == decode_chunk_tokens(Gm::ELEM, D), "host and device chunk sizes differ");
  const int H = num_kv_heads * G;
  const int B = 1 << log2b;
  const int lane = threadIdx.x & 63;
  u32x4* out = static_cast<u32x4*>(a.out);

  WaveWork ww;
  if (a.balanced) {
    auto zero_row = [&](int q_row) {  // this lane writes the G heads' zero rows
      u32x4* o = out + (static_cast<int64_t>(q_row) * H + g * G) * VPR;
      for (int v = 0; v < G * VPR; ++v) o[v] = u32x4{0u, 0u, 0u, 0u};
    };
    ww = even_split<CHUNK>(a, y, B, log2b, lds, g == 0, zero_row);
  } else {
    const RowInfo ri = row_info(a, z, B);
    if (!ri.active) return;
    const int P = a.partition_size;
    const int nparts = (ri.ctx + P - 1) / P;
    if (ri.ctx == 0) {
      // nothing to attend: partition 0 writes a zero row for each head
      if (y == 0) {
        const int row = lane / LPT, col = lane % LPT;
        for (int h = row; h < G; h += Gm::TPI)
          out[(static_cast<int64_t>(ri.q_row) * H + g * G + h) * VPR + col] = u32x4{0u, 0u, 0u, 0u};
      }
      return;
    }
    if (y >= nparts) return;
    const int tok0 = y * P, end = min(tok0 + P, ri.ctx);
    const int n = (end - tok0 + CHUNK - 1) / CHUNK;
    if (lane == 0)
      put_seg(lds, 0, z | (nparts == 1 ? kSegFinal : 0), ri.q_row, tok0, end, n, 0, ri.table_row,
              ri.ctx);
    // P is a multiple of 64, so tok0 is a multiple of the chunk
    ww = WaveWork{1, n, seg_blocks<CHUNK>(tok0 / CHUNK, tok0 / CHUNK + n, log2b)};
  }
  // wave-uniform from here on (the fixed split derives them from loads the
  // compiler cannot prove uniform); keeps the loop control scalar
  ww.nseg = __builtin_amdgcn_readfirstlane(ww.nseg);
  ww.K = __builtin_amdgcn_readfirstlane(ww.K);
  ww.E = __builtin_amdgcn_readfirstlane(ww.E);
  if (ww.K == 0) return;
  // the list is written and read by this wave only; LDS executes one
  // wave's accesses in order, so a compiler-level fence suffices
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  auto seg = [&](int s, int f) { return __builtin_amdgcn_readfirstlane(lds[s * kSegInts + f]); };

  W w;
  w.lane = lane;
  w.row = lane / LPT;
  w.col = lane % LPT;
  w.hmask = head_mask<LPT, ilog2(G)>(w.col);
  w.prep(g, a.rot, log2b, num_kv_heads * W::VPH);
  const u32x4* qp = static_cast<const u32x4*>(a.q);
  auto load_q = [&](int q_row) {
#pragma unroll
    for (int s = 0; s < G; ++s) {
      const int h = g * G + (s ^ w.hmask);
      w.qv[s] = qp[(static_cast<int64_t>(q_row) * H + h) * VPR + w.col];
    }
  };
  // q of the first segment is in flight with the table loads
  load_q(seg(0, kSegQRow));
  stage_tables(a, lds, ww, log2b, num_blocks);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // FP8: scores take the K scale, outputs the V scale of this KV head
  float scale_log2 = a.scale * kLog2e;
  float out_scale = 1.f;
  if constexpr (FP8) {
    scale_log2 *= a.k_scale[g];
    out_scale = a.v_scale[g];
  }
  using Vec = typename W::Vec;
  const Vec* kc = static_cast<const Vec*>(a.k_cache);
  const Vec* vc = static_cast<const Vec*>(a.v_cache);
  const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * W::VPH;
  const int rot = a.rot;
  const int bmask = B - 1;
  const int tb0 = ww.nseg * kSegInts;
  constexpr int LOG2G = ilog2(G);
  constexpr int S = DecodeStages<BF16, D, G, FP8>::value;

  for (int sg = 0; sg < ww.nseg; ++sg) {
    const int rf = seg(sg, kSegRow);
    const int zr = rf & (kSegFinal - 1);
    const int q_row = seg(sg, kSegQRow);
    const int start = seg(sg, kSegTok0);
    const int end = seg(sg, kSegEnd);
    const int nchunks = seg(sg, kSegN);
    const int tb = tb0 + seg(sg, kSegEoff) - (start >> log2b);
    if (sg > 0) load_q(q_row);  // in flight with the segment's first chunks
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPV; ++e) w.o[h][e] = 0.f;
    w.m = -INFINITY;
    w.l = 0.f;

    // Software pipeline over the segment's chunks with S register buffers:
    // the loads of chunk c+S-1 are issued before chunk c is computed, so up
    // to S-1 chunks (S-1 x 8 KiB for bf16 D=128) are in flight per
    // wavefront.  Buffer indices are compile-time, so the ring stays in
    // registers.  Loads past the last chunk are clamped onto it instead of
    // branched around: they hit the L2 lines just fetched and keep the
    // steady-state loop branch-free.  Only the final S chunks are computed
    // with the length mask.  The ring drains at the end of a segment; the
    // split charges a row switch for that.
    // Fused append: the segment that ends the row holds the step's new token
    // (position ctx - 1, input row zr).  Its K/V for this KV head is attended
    // from registers and stored through new_slots[zr] after the segment, so
    // no wave of the launch reads that slot from memory (the block a token
    // is appended to belongs to its row alone).  Skipped, like a cache write,
    // for a slot out of range; then the cache is read as it is.  The loads
    // go out before the segment's first chunks and are consumed only in its
    // last ones, so they never hold up the stream.
    const bool row_end = a.new_slots != nullptr && end == seg(sg, kSegCtx);
    int slot_v = -1;
    u32x4 nk{0u, 0u, 0u, 0u}, nv{0u, 0u, 0u, 0u};
    if (row_end) {
      slot_v = a.new_slots[zr + vgpr_zero()];
      const int64_t in = (static_cast<int64_t>(zr) * num_kv_heads + g) * VPR + w.col;
      nk = static_cast<const u32x4*>(a.new_k)[in];
      nv = static_cast<const u32x4*>(a.new_v)[in];
    }

    typename W::Chunk buf[S];
    const int last = nchunks - 1;
    auto load_chunk = [&](typename W::Chunk& ch, int ci) {
      ci = ci < last ? ci : last;
      w.load(ch, kc, vc, lds, tb, start + ci * CHUNK, log2b, bmask, g, rot, row_stride);
    };
#pragma unroll
    for (int s = 0; s < S - 1; ++s) load_chunk(buf[s], s);
    int c = 0;
    for (; c + S < nchunks; c += S) {  // chunks c .. c+S-1 are full
#pragma unroll
      for (int s = 0; s < S; ++s) {
        load_chunk(buf[(s + S - 1) % S], c + s + S - 1);
        w.template compute<false>(buf[s], start + (c + s) * CHUNK, end, scale_log2, -1, nk, nv);
      }
    }
    // 1..S chunks remain; chunk c+s sits in buf[s]
    load_chunk(buf[S - 1], c + S - 1);
    const int64_t slot = __builtin_amdgcn_readfirstlane(slot_v);
    const bool put = row_end && slot >= 0 && slot < (static_cast<int64_t>(num_blocks) << log2b);
    const int np = put ? end - 1 : -1;
    Vec sk, sv;  // what the cache receives
    if constexpr (FP8) {
      sk = quant_fp8x8(nk, a.k_scale[g]);
      sv = quant_fp8x8(nv, a.v_scale[g]);
      nk = W::widen(sk);
      nv = W::widen(sv);
    } else {
      sk = nk;
      sv = nv;
    }
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (c + s < nchunks)
        w.template compute<true>(buf[s], start + (c + s) * CHUNK, end, scale_log2, np, nk, nv);
    if (put && w.row == 0) {  // the first token row's lanes cover the head row
      const int64_t dst =
          slot * row_stride + kv_head_pos(g, static_cast<int>(slot) & bmask, rot) * W::VPH + w.col;
      const_cast<Vec*>(kc)[dst] = sk;
      const_cast<Vec*>(vc)[dst] = sv;
    }

    // merge the token rows: per head, bring (m, l) of the head's lane to
    // every lane of the row, then combine rows with the usual max-rescale
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

    // every row now holds the merged result; row r stores heads r, r + TPI, ...
    const int row = w.row, col = w.col;
    if (rf & kSegFinal) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (h % Gm::TPI != row) continue;
        const float inv = out_scale / L[h];
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
        out[(static_cast<int64_t>(q_row) * H + g * G + h) * VPR + col] = r;
      }
    } else {
      // partial index of head g*G + h: balanced (y + row) * H + g*G + h,
      // fixed (row * H + g*G + h) * max_partitions + y
      const int64_t base = a.balanced ? (static_cast<int64_t>(y) + zr) * H + g * G
                                      : (static_cast<int64_t>(zr) * H + g * G) * a.max_partitions + y;
      const int64_t hstride = a.balanced ? 1 : a.max_partitions;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (h % Gm::TPI != row) continue;
        const int64_t idx = base + h * hstride;
        float* po = a.part_o + idx * D + col * EPV;
#pragma unroll
        for (int e = 0; e < EPV; e += 4)
          *reinterpret_cast<float4*>(po + e) =
              make_float4(w.o[h][e] * out_scale, w.o[h][e + 1] * out_scale, w.o[h][e + 2] * out_scale,
                          w.o[h][e + 3] * out_scale);
        if (col == 0) *reinterpret_cast<float2*>(a.part_ml + idx * 2) = make_float2(M[h], L[h]);
      }
    }
  }
}

}  // namespace pa
