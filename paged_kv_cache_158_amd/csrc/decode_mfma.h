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

  __device__ __forceinline__ void load(Chunk& ch, const u32x4* __restrict__ kc,
                                       const VVec* __restrict__ vc, const int32_t* tbl, int tb,
                                       int t0, int log2b, int bmask, int g, int rot, int64_t krow,
                                       int64_t vrow) const {
    const int tk = t0 + c, tv = t0 + 4 * q4;
    const int bk = tbl[tb + (tk >> log2b)];
    const int bv = tbl[tb + (tv >> log2b)];
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
  // masked chunk (np = -1: none).
  template <bool MASKED>
  __device__ __forceinline__ void compute(const Chunk& ch, int t0, int end, float scale_log2,
                                          int np, const u32x4 (&nk)[4], const u32x4& nv) {
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
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = sacc[r] * scale_log2;
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

template <int G, bool FP8>
struct MfmaStages {
  static constexpr int value = FP8 ? 5 : 2;
};

// One decode wavefront on the matrix cores: KV head g and, with the
// balanced split, range y of the line, or partition y of row z (fixed
// split).  The plan, the segment list and the staged block tables are those
// of decode_partition_body; see there.
template <int G, bool FP8>
__device__ __forceinline__ void decode_mfma_body(const DecodeArgs& a, int g, int y, int z,
                                                 int32_t* lds, int32_t num_kv_heads,
                                                 int32_t num_blocks, int32_t log2b) {
  using W = MfmaWave<G, FP8>;
  constexpr int CHUNK = W::CHUNK, VPR = 16, D = 128;
  static_assert(CHUNK == decode_chunk_tokens(2, D), "host and device chunk sizes differ");
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
  if (ww.K == 0) return;
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
  const int hc = min(w.c, G - 1);  // columns past the group load a valid row and drop it
  auto load_q = [&](int q_row) {
    const u32x4* src = qp + (static_cast<int64_t>(q_row) * H + g * G + hc) * VPR;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = src[w.kdim(i)];
      w.qv[i] = w.c < G ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  load_q(seg(0, kSegQRow));
  stage_tables(a, lds, ww, log2b, num_blocks);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

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
    const int zr = rf & (kSegFinal - 1);
    const int q_row = seg(sg, kSegQRow);
    const int start = seg(sg, kSegTok0);
    const int end = seg(sg, kSegEnd);
    const int nchunks = seg(sg, kSegN);
    const int tb = tb0 + seg(sg, kSegEoff) - (start >> log2b);
    if (sg > 0) load_q(q_row);
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
        w.template compute<false>(buf[s], start + (c + s) * CHUNK, end, scale_log2, -1, nk, nv);
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
        w.template compute<true>(buf[s], start + (c + s) * CHUNK, end, scale_log2, np, nk, nv);
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
      const int64_t base = a.balanced ? (static_cast<int64_t>(y) + zr) * H + g * G
                                      : (static_cast<int64_t>(zr) * H + g * G) * a.max_partitions + y;
      const int64_t hstride = a.balanced ? 1 : a.max_partitions;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * w.q4 + r;
        if (h >= G) continue;
        const int64_t idx = base + h * hstride;
        float* po = a.part_o + idx * D + 8 * w.c;
        *reinterpret_cast<float4*>(po) = make_float4(w.o[0][r] * out_scale, w.o[1][r] * out_scale,
                                                     w.o[2][r] * out_scale, w.o[3][r] * out_scale);
        *reinterpret_cast<float4*>(po + 4) = make_float4(w.o[4][r] * out_scale, w.o[5][r] * out_scale,
                                                         w.o[6][r] * out_scale, w.o[7][r] * out_scale);
        if (w.c == 0) *reinterpret_cast<float2*>(a.part_ml + idx * 2) = make_float2(Mr[r], Lr[r]);
      }
    }
  }
}

}  // namespace pa
