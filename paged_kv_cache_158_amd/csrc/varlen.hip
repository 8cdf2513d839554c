// Chunked-prefill attention over the paged cache with bf16 MFMA (gfx950).
//
// What is computed (CSDN "vLLM 0.10.0 flow" page §3.2 chunked prefill and
// §3.5 attention metadata; dn008 overview §2.1 causal mask): segment s of a
// varlen batch owns query rows [query_start_loc[s], query_start_loc[s+1]).
// With q_len rows and L = seq_lens[s] tokens in total, the row at index i of
// the segment is the token at position P + i, P = L - q_len, and attends to
// keys 0 .. P + i of the sequence, whose K/V live in the paged cache behind
// block_tables[s].  This kernel handles segments with q_len >= 2; one-row
// (decode) segments go through the split-K decode kernels.
//
// Tiling.  A workgroup of 4 wavefronts owns (q-block, KV head g, segment s).
// Each wavefront owns 16 MFMA columns = (query row, query head) pairs of the
// G heads that share KV head g (16/G rows x G heads), so every K/V tile it
// reads from LDS serves all G heads.  Keys advance in tiles of 64 (four
// 16-token blocks at B = 16), gathered through the block table into LDS: K
// row-major [key][d], V transposed [d][key].
//
// Scores are computed transposed, S^T = K Q^T (keys on the MFMA M axis,
// query columns on N) with v_mfma_f32_16x16x32_bf16.  Its fp32 result
// leaves lane l holding keys 4*(l/16)+i of column l%16 — exactly the 8 key
// slots that lane must supply as the bf16 B operand of O^T += V^T P^T when a
// 32-key MFMA step takes keys {4a..4a+3} from one 16-key M-tile and
// {16+4a..16+4a+3} from the next (a = l/16).  The V^T A operand reads the
// same key order from LDS, so P never moves between lanes.  Online softmax
// per column in base 2 with a lazily moved reference max, as in decode.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kKT = 64;             // keys per tile
constexpr int kThreads = 256;       // 4 wavefronts
constexpr float kTauV = 8.0f;       // lazy-rescale threshold (log2 units)

__device__ __forceinline__ f32x4_t mfma16(const u32x4& a, const u32x4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int D>
struct Tile {
  static constexpr int KPITCH = D + 8;        // K tile row pitch (bf16): 16 B pad
  static constexpr int VPITCH = kKT + 4;      // V^T tile row pitch (bf16): 8 B pad
  static constexpr int VPR = D / 8;           // 16-byte vectors per K/V row
  static constexpr int NVEC = kKT * VPR / kThreads;  // vectors per thread per tile
  static constexpr int KSTEPS = D / 32;       // QK MFMA k-steps
  static constexpr int DMT = D / 16;          // PV M-tiles (head dims)
};

}  // namespace

template <int D, int G>
__global__ void __launch_bounds__(kThreads)
varlen_prefill_kernel(const VarlenArgs a, int32_t num_kv_heads, int32_t num_blocks,
                      int32_t log2b) {
  using T = Tile<D>;
  constexpr int RPW = 16 / G;           // query rows per wavefront
  constexpr int ROWS = 4 * RPW;         // query rows per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t ks[kKT * T::KPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t vts[D * T::VPITCH];

  const int qb = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;
  const int H = num_kv_heads * G;
  const int B = 1 << log2b;
  const int q0 = a.query_start_loc[s];
  const int qlen = a.query_start_loc[s + 1] - q0;
  if (qlen < 2 || qb * ROWS >= qlen) return;
  int L = a.seq_lens[s];
  L = clampi(L, 0, min(a.max_seq_len, a.max_blocks_per_seq * B));
  const int prior = max(L - qlen, 0);
  L = prior + qlen;  // keys a row may see never pass its own position
  const int nblk = min((L + B - 1) >> log2b, a.max_blocks_per_seq);
  const int32_t* trow = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;  // MFMA column = (row, head) pair
  const int grp = lane >> 4;  // lane group: key slots 4*grp .. 4*grp+3 of each 16-key M-tile

  // this lane's query column
  const int rr = col / G, hh = col % G;
  const int qrow = qb * ROWS + wave * RPW + rr;  // row within the segment
  const bool col_valid = qrow < qlen;
  const int qrow_c = min(qrow, qlen - 1);
  const int pos = prior + qrow_c;                // last key this column sees
  const int head = g * G + hh;

  // wave / workgroup key extents
  const int wave_first = min(qb * ROWS + wave * RPW, qlen - 1);
  const int wave_last = min(qb * ROWS + wave * RPW + RPW - 1, qlen - 1);
  const int pos_lo = prior + wave_first;
  const int pos_hi = prior + wave_last;
  const int wg_last = min(qb * ROWS + ROWS - 1, qlen - 1);
  const int ntiles = (prior + wg_last + 1 + kKT - 1) / kKT;

  // Q^T as the MFMA B operand: column col, head dims ks*32 + 8*grp .. +7
  u32x4 qv[T::KSTEPS];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(q0 + qrow_c) * H + head) * D);
#pragma unroll
    for (int k = 0; k < T::KSTEPS; ++k) qv[k] = qp[k * 4 + grp];
  }

  f32x4_t oacc[T::DMT];
#pragma unroll
  for (int i = 0; i < T::DMT; ++i) oacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // reference max of this column (log2 units)
  float lsum = 0.f;     // this lane's share of the column's probability sum
  const float scale_log2 = a.scale * kLog2e;

  // staging: thread tid moves vectors v = tid + kThreads*i of the tile
  const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
  const u32x4* vc = static_cast<const u32x4*>(a.v_cache);
  const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * T::VPR;  // vectors per slot
  u32x4 kreg[T::NVEC], vreg[T::NVEC];
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < T::NVEC; ++i) {
      const int v = tid + kThreads * i;
      const int key = t * kKT + v / T::VPR;
      const int cc = v % T::VPR;
      if (key < L) {
        const int bi = min(key >> log2b, nblk - 1);
        const int blk = clampi(trow[bi], 0, num_blocks - 1);
        const int64_t off = ((static_cast<int64_t>(blk) << log2b) + (key & (B - 1))) * row_stride +
                            static_cast<int64_t>(g) * T::VPR + cc;
        kreg[i] = kc[off];
        vreg[i] = vc[off];
      } else {
        // past the sequence: zeros (stale slots may hold NaN)
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < T::NVEC; ++i) {
      const int v = tid + kThreads * i;
      const int kk = v / T::VPR;
      const int cc = v % T::VPR;
      *reinterpret_cast<u32x4*>(&ks[kk * T::KPITCH + cc * 8]) = kreg[i];
      const uint32_t vw[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vts[(cc * 8 + 2 * e) * T::VPITCH + kk] = static_cast<uint16_t>(vw[e] & 0xffffu);
        vts[(cc * 8 + 2 * e + 1) * T::VPITCH + kk] = static_cast<uint16_t>(vw[e] >> 16);
      }
    }
  };

  fetch(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // every wave is done reading the previous tile
    stage();
    __syncthreads();
    if (t + 1 < ntiles) fetch(t + 1);

    const int tile0 = t * kKT;
    if (tile0 > pos_hi) continue;  // no column of this wave sees these keys
    const bool need_mask = tile0 + kKT - 1 > pos_lo;

    // S^T tile: 4 M-tiles of 16 keys x this wave's 16 columns
    f32x4_t sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sacc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < T::KSTEPS; ++k) {
        const u32x4 av =
            *reinterpret_cast<const u32x4*>(&ks[(mt * 16 + col) * T::KPITCH + k * 32 + grp * 8]);
        sacc[mt] = mfma16(av, qv[k], sacc[mt]);
      }
    }
    float sv[4][4];
    float cmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = sacc[mt][i] * scale_log2;
        if (need_mask && tile0 + mt * 16 + grp * 4 + i > pos) x = -INFINITY;
        sv[mt][i] = x;
        cmax = fmaxf(cmax, x);
      }
    cmax = fmaxf(cmax, xor_lane<16>(cmax));
    cmax = fmaxf(cmax, xor_lane<32>(cmax));
    if (__any(cmax > m + kTauV)) {
      const float mn = fmaxf(m, cmax);
      const float alpha = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < T::DMT; ++i) oacc[i] *= alpha;
    }
    const float mref = (m == -INFINITY) ? 0.f : m;
    // probabilities as the bf16 B operand of two 32-key PV steps
    u32x4 pb[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      uint32_t w[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int mt = 2 * k2 + h2;
        w[2 * h2] = pack_bf16(__builtin_amdgcn_exp2f(sv[mt][0] - mref),
                              __builtin_amdgcn_exp2f(sv[mt][1] - mref));
        w[2 * h2 + 1] = pack_bf16(__builtin_amdgcn_exp2f(sv[mt][2] - mref),
                                  __builtin_amdgcn_exp2f(sv[mt][3] - mref));
        lsum += bf16_lo(w[2 * h2]) + bf16_hi(w[2 * h2]) + bf16_lo(w[2 * h2 + 1]) +
                bf16_hi(w[2 * h2 + 1]);
      }
      pb[k2] = u32x4{w[0], w[1], w[2], w[3]};
    }
    // O^T += V^T P^T: A operand = V^T rows (head dims), keys in the same slot order
#pragma unroll
    for (int dm = 0; dm < T::DMT; ++dm) {
      const uint16_t* vrow = &vts[(dm * 16 + col) * T::VPITCH];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + k2 * 32 + grp * 4);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + k2 * 32 + 16 + grp * 4);
        oacc[dm] = mfma16(u32x4{lo.x, lo.y, hi.x, hi.y}, pb[k2], oacc[dm]);
      }
    }
  }

  // column sums across the 4 lane groups, normalise, store valid columns
  lsum += xor_lane<16>(lsum);
  lsum += xor_lane<32>(lsum);
  if (!col_valid) return;
  const float inv = 1.f / lsum;
  uint16_t* op = static_cast<uint16_t*>(a.out) +
                 (static_cast<int64_t>(q0 + qrow) * H + head) * D + grp * 4;
#pragma unroll
  for (int dm = 0; dm < T::DMT; ++dm) {
    const uint2 w = {pack_bf16(oacc[dm][0] * inv, oacc[dm][1] * inv),
                     pack_bf16(oacc[dm][2] * inv, oacc[dm][3] * inv)};
    *reinterpret_cast<uint2*>(op + dm * 16) = w;
  }
}

bool varlen_prefill_supported(const pa_cache_dims& d) {
  if (d.dtype != PA_DTYPE_BF16) return false;
  if (d.head_dim != 64 && d.head_dim != 128) return false;
  const int G = d.num_heads / d.num_kv_heads;
  return G == 1 || G == 2 || G == 4 || G == 8 || G == 16;
}

template <int D, int G>
static hipError_t launch_prefill_t(const VarlenArgs& a, const pa_cache_dims& d, hipStream_t st) {
  constexpr int ROWS = 4 * (16 / G);
  const dim3 grid((a.max_query_len + ROWS - 1) / ROWS, d.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((varlen_prefill_kernel<D, G>), grid, dim3(kThreads), 0, st, a,
                     d.num_kv_heads, d.num_blocks, ilog2(d.block_size));
  return hipGetLastError();
}

template <int D>
static hipError_t prefill_group(const VarlenArgs& a, const pa_cache_dims& d, hipStream_t st) {
  switch (d.num_heads / d.num_kv_heads) {
    case 1: return launch_prefill_t<D, 1>(a, d, st);
    case 2: return launch_prefill_t<D, 2>(a, d, st);
    case 4: return launch_prefill_t<D, 4>(a, d, st);
    case 8: return launch_prefill_t<D, 8>(a, d, st);
    case 16: return launch_prefill_t<D, 16>(a, d, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_varlen_prefill(const VarlenArgs& a, const pa_cache_dims& d, hipStream_t stream) {
  if (!varlen_prefill_supported(d)) return hipErrorInvalidValue;
  if (a.max_query_len < 2 || a.num_seqs == 0) return hipSuccess;
  return d.head_dim == 128 ? prefill_group<128>(a, d, stream) : prefill_group<64>(a, d, stream);
}

}  // namespace pa
