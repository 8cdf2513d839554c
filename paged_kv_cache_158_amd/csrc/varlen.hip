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
// A wavefront owns NT x 16 MFMA columns = (query row, query head) pairs of
// the G heads that share KV head g (head fastest), so each K/V element read
// from LDS feeds NT MFMAs: with NT = 4 a wave does 128 MFMAs per 64-key tile
// against 32 KiB of LDS reads, which keeps LDS below half its bandwidth.
// Keys advance in tiles of 64, gathered through the block table: every
// thread fetches its 16-byte pieces of the next tile into registers while
// the current one is computed, then writes them into the other half of a
// double-buffered LDS ring.  K and V tiles stay row-major ([key][d]); the
// 16-byte chunks of each row are XOR-swizzled by the row so that the MFMA
// operand reads are free of bank conflicts.
//
// Scores are computed transposed, S^T = K Q^T (keys on the MFMA M axis,
// query columns on N) with v_mfma_f32_16x16x32_bf16.  Its fp32 result
// leaves lane l holding keys 4*(l/16)+i of column l%16 — exactly the 8 key
// slots that lane supplies as the bf16 B operand of O^T += V^T P^T when a
// 32-key step takes keys {4a..4a+3} from one 16-key M-tile and
// {16+4a..16+4a+3} from the next (a = l/16), so P never moves between lanes.
// The V^T A operand comes out of the row-major V tile with the LDS transpose
// read ds_read_b64_tr_b16: each lane of a 16-lane group points at 4
// consecutive head dims of one key row, and lane i receives dim i of four
// consecutive keys.  Online softmax per column in base 2 with a lazily moved
// reference maximum, as in decode.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kKT = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 wavefronts
constexpr float kTauV = 8.0f;  // lazy-rescale threshold (log2 units)

__device__ __forceinline__ f32x4_t mfma16(const u32x4& a, const u32x4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 8 bytes of LDS transposed across each 16-lane group (see the header).
__device__ __forceinline__ uint2 lds_read_tr(const uint16_t* p) {
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4_t __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(uint2, r);
}

template <int D>
struct Tile {
  static constexpr int NCH = D / 8;                  // 16-byte chunks per K/V row
  static constexpr int NVEC = kKT * NCH / kThreads;  // chunks per thread per tile
  static constexpr int KSTEPS = D / 32;              // QK MFMA k-steps
  static constexpr int DMT = D / 16;                 // PV M-tiles (head dims)
  static constexpr int ELEMS = kKT * D;              // bf16 per K (or V) tile
  // chunk swizzles: the 16 rows read together by a K operand load hit 16
  // distinct chunk positions; the V transpose read of 16 rows x 32 bytes
  // spreads over two conflict-free passes
  __device__ static int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  __device__ static int swz_v(int row) { return D == 128 ? ((row & 7) << 1) : (((row >> 1) & 3) << 1); }
};

}  // namespace

#ifndef PA_PREFILL_NT
#define PA_PREFILL_NT 2
#endif
template <int D, int G>
struct PrefillCfg {
  static constexpr int NT = PA_PREFILL_NT < G ? PA_PREFILL_NT : G;  // 16-column N-tiles per wavefront
  static constexpr int COLS = NT * 16;             // columns per wavefront
  static constexpr int RPW = COLS / G;             // query rows per wavefront
  static constexpr int ROWS = 4 * RPW;             // query rows per workgroup
};

template <int D, int G>
__global__ void __launch_bounds__(kThreads)
varlen_prefill_kernel(const VarlenArgs a, int32_t num_kv_heads, int32_t num_blocks,
                      int32_t log2b) {
  using T = Tile<D>;
  using C = PrefillCfg<D, G>;
  constexpr int NT = C::NT, RPW = C::RPW, ROWS = C::ROWS;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][T::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][T::ELEMS];

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
  const int col16 = lane & 15;  // column within an N-tile
  const int grp = lane >> 4;    // lane group: key slots 4*grp .. 4*grp+3 of each 16-key M-tile

  // this lane's NT query columns: column c = nt*16 + col16 -> (row c/G, head c%G)
  int pos[NT];
  bool col_valid[NT];
  int qrow_v[NT], head_v[NT];
  const int row0 = qb * ROWS + wave * RPW;  // first query row of this wave
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = nt * 16 + col16;
    const int qrow = row0 + c / G;
    col_valid[nt] = qrow < qlen;
    qrow_v[nt] = min(qrow, qlen - 1);
    pos[nt] = prior + qrow_v[nt];
    head_v[nt] = g * G + c % G;
  }
  const int pos_lo = prior + min(row0, qlen - 1);
  const int pos_hi = prior + min(row0 + RPW - 1, qlen - 1);
  const int wg_last = min(qb * ROWS + ROWS - 1, qlen - 1);
  const int ntiles = (prior + wg_last + 1 + kKT - 1) / kKT;

  // Q^T as the MFMA B operand: column (nt, col16), head dims k*32 + 8*grp .. +7
  u32x4 qv[NT][T::KSTEPS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(q0 + qrow_v[nt]) * H + head_v[nt]) * D);
#pragma unroll
    for (int k = 0; k < T::KSTEPS; ++k) qv[nt][k] = qp[k * 4 + grp];
  }

  f32x4_t oacc[T::DMT][NT];
#pragma unroll
  for (int i = 0; i < T::DMT; ++i)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) oacc[i][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[NT], lsum[NT];  // per column: reference max (log2 units), this lane's share of the sum
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -INFINITY;
    lsum[nt] = 0.f;
  }
  const float scale_log2 = a.scale * kLog2e;

  // staging: thread tid moves chunks v = tid + kThreads*i of each tile
  const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
  const u32x4* vc = static_cast<const u32x4*>(a.v_cache);
  const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * T::NCH;  // chunks per slot
  u32x4 kreg[T::NVEC], vreg[T::NVEC];
  // Block-table entries are loaded a full tile ahead of the K/V loads that
  // use them, so no iteration waits on a table load followed by a dependent
  // K/V load.
  int blk[T::NVEC];
  auto fetch_table = [&](int t) {
#pragma unroll
    for (int i = 0; i < T::NVEC; ++i) {
      const int key = t * kKT + (tid + kThreads * i) / T::NCH;
      const int bi = max(min(key >> log2b, nblk - 1), 0);
      blk[i] = key < L ? clampi(trow[bi], 0, num_blocks - 1) : 0;
    }
  };
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < T::NVEC; ++i) {
      const int v = tid + kThreads * i;
      const int key = t * kKT + v / T::NCH;
      const int cc = v % T::NCH;
      if (key < L) {
        const int64_t off = ((static_cast<int64_t>(blk[i]) << log2b) + (key & (B - 1))) * row_stride +
                            static_cast<int64_t>(g) * T::NCH + cc;
        kreg[i] = kc[off];
        vreg[i] = vc[off];
      } else {
        // past the sequence: zeros (stale slots may hold NaN)
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < T::NVEC; ++i) {
      const int v = tid + kThreads * i;
      const int kk = v / T::NCH;
      const int cc = v % T::NCH;
      *reinterpret_cast<u32x4*>(&ks[buf][kk * D + ((cc ^ T::swz_k(kk)) << 3)]) = kreg[i];
      *reinterpret_cast<u32x4*>(&vs[buf][kk * D + ((cc ^ T::swz_v(kk)) << 3)]) = vreg[i];
    }
  };

  fetch_table(0);
  fetch(0);
  fetch_table(1);
  stage(0);
  if (ntiles > 1) fetch(1);
  fetch_table(2);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int tile0 = t * kKT;
    if (tile0 <= pos_hi) {  // some column of this wave sees keys of this tile
      const bool need_mask = tile0 + kKT - 1 > pos_lo;
      const uint16_t* kt = ks[buf];
      const uint16_t* vt = vs[buf];
      // the 64-key tile in two 32-key halves: S^T for 2 M-tiles x NT N-tiles,
      // online softmax, then one 32-key PV step (keeps the live registers low;
      // not unrolled, so the two halves' operand loads are not hoisted together)
#pragma unroll 1
      for (int k2 = 0; k2 < 2; ++k2) {
        f32x4_t sacc[2][NT];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int mt = 2 * k2 + h2;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) sacc[h2][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          const int krow = mt * 16 + col16;
#pragma unroll
          for (int k = 0; k < T::KSTEPS; ++k) {
            const u32x4 av = *reinterpret_cast<const u32x4*>(
                &kt[krow * D + (((k * 4 + grp) ^ T::swz_k(krow)) << 3)]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) sacc[h2][nt] = mfma16(av, qv[nt][k], sacc[h2][nt]);
          }
        }
        u32x4 pb[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float sv[2][4];
          float cmax = -INFINITY;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float x = sacc[h2][nt][i] * scale_log2;
              if (need_mask && tile0 + (2 * k2 + h2) * 16 + grp * 4 + i > pos[nt]) x = -INFINITY;
              sv[h2][i] = x;
              cmax = fmaxf(cmax, x);
            }
          cmax = fmaxf(cmax, xor_lane<16>(cmax));
          cmax = fmaxf(cmax, xor_lane<32>(cmax));
          if (__any(cmax > m[nt] + kTauV)) {
            const float mn = fmaxf(m[nt], cmax);
            const float alpha = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m[nt] - mn);
            m[nt] = mn;
            lsum[nt] *= alpha;
#pragma unroll
            for (int i = 0; i < T::DMT; ++i) oacc[i][nt] *= alpha;
          }
          const float mref = (m[nt] == -INFINITY) ? 0.f : m[nt];
          uint32_t w[4];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            w[2 * h2] = pack_bf16(__builtin_amdgcn_exp2f(sv[h2][0] - mref),
                                  __builtin_amdgcn_exp2f(sv[h2][1] - mref));
            w[2 * h2 + 1] = pack_bf16(__builtin_amdgcn_exp2f(sv[h2][2] - mref),
                                      __builtin_amdgcn_exp2f(sv[h2][3] - mref));
            lsum[nt] += bf16_lo(w[2 * h2]) + bf16_hi(w[2 * h2]) + bf16_lo(w[2 * h2 + 1]) +
                        bf16_hi(w[2 * h2 + 1]);
          }
          pb[nt] = u32x4{w[0], w[1], w[2], w[3]};
        }
        // O^T += V^T P^T: the A operand (head dims x key slots) by transpose reads
#pragma unroll
        for (int dm = 0; dm < T::DMT; ++dm) {
          const int d0 = dm * 16 + 4 * (col16 & 3);  // this lane's 4-dim piece
          uint2 part[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int key = k2 * 32 + h * 16 + grp * 4 + (col16 >> 2);
            const int chunk = d0 >> 3;
            part[h] = lds_read_tr(&vt[key * D + ((chunk ^ T::swz_v(key)) << 3) + (d0 & 7)]);
          }
          const u32x4 av = u32x4{part[0].x, part[0].y, part[1].x, part[1].y};
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) oacc[dm][nt] = mfma16(av, pb[nt], oacc[dm][nt]);
        }
      }
    }
    if (t + 1 < ntiles) stage(buf ^ 1);  // regs hold tile t+1; that buffer was freed by the last barrier
    if (t + 2 < ntiles) fetch(t + 2);    // its table entries arrived during this tile
    fetch_table(t + 3);
    __syncthreads();
  }

  // column sums across the 4 lane groups, normalise, store valid columns
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = lsum[nt];
    l += xor_lane<16>(l);
    l += xor_lane<32>(l);
    if (!col_valid[nt]) continue;
    const float inv = 1.f / l;
    uint16_t* op = static_cast<uint16_t*>(a.out) +
                   (static_cast<int64_t>(q0 + qrow_v[nt]) * H + head_v[nt]) * D + grp * 4;
#pragma unroll
    for (int dm = 0; dm < T::DMT; ++dm) {
      const uint2 w = {pack_bf16(oacc[dm][nt][0] * inv, oacc[dm][nt][1] * inv),
                       pack_bf16(oacc[dm][nt][2] * inv, oacc[dm][nt][3] * inv)};
      *reinterpret_cast<uint2*>(op + dm * 16) = w;
    }
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
  constexpr int ROWS = PrefillCfg<D, G>::ROWS;
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
