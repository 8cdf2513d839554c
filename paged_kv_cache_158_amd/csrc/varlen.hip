// Chunked-prefill attention over the paged cache with bf16 MFMA (gfx950).
//
// What is computed (CSDN "vLLM 0.10.0 flow" page §3.2 chunked prefill and
// §3.5 attention metadata; dn008 overview §2.1 causal mask): segment s of a
// varlen batch owns query rows [query_start_loc[s], query_start_loc[s+1]).
// With q_len rows and L = seq_lens[s] tokens in total, the row at index i of
// the segment is the token at position P + i, P = L - q_len, and attends to
// keys 0 .. P + i of the sequence, whose K/V live in the paged cache behind
// block_tables[s].  This kernel handles segments with q_len >= 2; one-row
// (decode) segments go through the split-K decode kernels.  Caches are bf16
// or FP8 (E4M3 codes with per-KV-head scales: code tiles in LDS, each MFMA
// operand widened to bf16 in registers as it is read, exactly).
//
// Tiling.  A workgroup of 4 wavefronts owns (query block, KV head g,
// segment s); two workgroups share a CU (two waves per SIMD, so one wave's
// matrix work can overlap the other's softmax), and being independent they
// do not wait on each other's tile barriers.  Every wavefront reads the
// whole K and V tile from LDS (32 KiB per 64 keys at D = 128): one 1 KiB
// operand per 32x32x16 MFMA, so at full matrix rate the four SIMDs would
// ask LDS for ~128 bytes per clock, about what it delivers (~120 for
// 16-byte reads, ~90 for 8-byte ones), and a tile is bound by the
// latency of its read -> MFMA -> softmax -> MFMA chain unless these
// overlap; wider wavefronts that reuse each operand for more columns need
// more registers than two waves per SIMD allow, and one wave per SIMD
// measured slower.  A wavefront owns 32 MFMA columns =
// (query row, query head) pairs of the G heads that share KV head g, head
// fastest.  Keys advance in tiles of 64, gathered through the block table
// straight into the other half of a double-buffered LDS ring
// (global_load_lds, no staging registers) while the current tile is
// computed; block-table entries are loaded a tile before the K/V loads
// that use them.  K and V tiles stay row-major ([key][d]); the 16-byte
// chunks of each row are XOR-swizzled by the row so that the operand reads
// below are free of bank conflicts.
//
// Scores are computed transposed, S^T = K Q^T (32 keys on the MFMA M axis,
// 32 query columns on N) with v_mfma_f32_32x32x16_bf16.  Its fp32 result
// leaves lane l holding keys 8j + 4(l/32) + r (j, r = 0..3) of column l%32;
// registers 8t..8t+7 (keys 16t + 4(l/32) + {0..3} and 16t + 8 + 4(l/32) +
// {0..3}) are exactly what that lane supplies as the bf16 B operand of the
// 16-key step t of O^T += V^T P^T when the step's k index e maps to those
// keys in that order, so probabilities never move between lanes.  The V^T A
// operand of the same step comes from the row-major V tile with two LDS
// transpose reads (ds_read_b64_tr_b16): each lane of a 16-lane group points
// at 4 consecutive head dims of one key row, and lane i receives dim i of
// four consecutive keys.  A column's 32 keys of a block sit in lanes l and
// l ^ 32, so its maximum and sum need one v_permlane32_swap.  Online softmax
// in base 2 with a lazily moved reference maximum, as in decode.
#include <cmath>

#include "decode_body.h"
#include "decode_mfma.h"
#include "varlen.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kKT = 64;        // keys per tile
constexpr int kWaves = 4;      // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = 32;      // MFMA columns per wavefront
constexpr float kTauV = 8.0f;  // lazy-rescale threshold (log2 units)

__device__ __forceinline__ f32x16_t mfma32(const u32x4& a, const u32x4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 8 bytes of LDS transposed across each 16-lane group (see the header).
__device__ __forceinline__ uint2 lds_read_tr(const uint16_t* p) {
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4_t __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(uint2, r);
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes
// land at lds + 16 i (lds is the same for every lane of the wave).
__device__ __forceinline__ void lds_dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds), 16, 0, 0);
}

// x of lane l ^ 32 (v_permlane32_swap exchanges the upper half of its first
// operand with the lower half of its second).
__device__ __forceinline__ float partner32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(threadIdx.x & 32 ? r[0] : r[1]);
}

template <int D>
struct Tile {
  static constexpr int NCH = D / 8;                  // 16-byte chunks per K/V row
  static constexpr int NVEC = kKT * NCH / kThreads;  // chunks per thread per tile (K, and V)
  static constexpr int KSTEPS = D / 16;              // QK MFMA k-steps
  static constexpr int DMT = D / 32;                 // PV M-tiles (head dims)
  static constexpr int ELEMS = kKT * D;              // bf16 per K (or V) tile
  static constexpr int NCH8 = D / 16;                // 16-byte chunks per FP8 row
  static constexpr int NVEC8 = kKT * NCH8 / kThreads;  // FP8 chunks per thread per tile
  // K operand reads: 8 consecutive rows read the same chunk; V transpose
  // reads: 4 consecutive rows read two adjacent chunks
  __device__ static int swz_k(int row) { return row & 7; }
  __device__ static int swz_v(int row) { return (row & 3) << 1; }
  // FP8 code tiles (D bytes per row, NCH8 16-byte chunks): the 8-byte K
  // reads of 16 consecutive rows and the 8-byte transpose reads of rows
  // {0..3, 8..11} + 4h then fall in distinct 16-byte bank groups
  __device__ static int swz8(int row) { return (row >> 1) & (NCH8 - 1); }
};

// 8 bytes of LDS transposed across each 16-lane group: lane i receives
// byte i % 8 of source lanes 2j + i / 8, j = 0..7, in j order.
__device__ __forceinline__ uint2 lds_read_tr8(const uint8_t* p) {
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  const i32x2_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (i32x2_t __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(uint2, r);
}

// Codes 0, 1 (lo) or 2, 3 (hi) of a word of E4M3 codes as a bf16 pair
// (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ uint32_t fp8_lo(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8_hi(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
__device__ __forceinline__ u32x4 fp8x8_bf16(uint2 c) {
  return u32x4{fp8_lo(c.x), fp8_hi(c.x), fp8_lo(c.y), fp8_hi(c.y)};
}

}  // namespace

template <int G>
struct PrefillCfg {
  static constexpr int RPW = kCols / G;     // query rows per wavefront
  static constexpr int ROWS = kWaves * RPW;  // query rows per workgroup
};

// Where a prefill workgroup's results go: final rows of `out` (part_o ==
// nullptr), or, for one key-range piece of a split unit, the unnormalised
// output and (max, sum) of each of its columns at workspace column
// col0 + c, c = wave * 32 + column (see PrefillSplit).
struct PrefillDest {
  float* part_o;   // [columns][D]
  float* part_ml;  // [columns][2]: max (log2 units, scale included), sum
  int64_t col0;
};

// The work of one prefill workgroup: key tiles [t_begin, t_end) (clamped to
// the unit's tiles) of query block qb of segment s, KV head g.  lds0 and
// lds1 are two distinct __shared__ arrays of at least 2 * 64 * D bf16 each,
// the two halves of a double-buffered ring, each a K tile followed by a V
// tile (bf16, or E4M3 codes for FP8 caches).  The tile being filled and the
// tile being read then always lie in
// different arrays, which the compiler's LDS alias analysis can tell apart,
// so it does not make the tile's LDS reads wait for the fill in flight.
template <int D, int G, bool FP8 = false>
__device__ __forceinline__ void prefill_body(const VarlenArgs& a, int qb, int g, int s,
                                             uint16_t* lds0, uint16_t* lds1,
                                             int32_t num_kv_heads, int32_t num_blocks,
                                             int32_t log2b, int t_begin, int t_end,
                                             const PrefillDest dst) {
  using T = Tile<D>;
  constexpr int RPW = PrefillCfg<G>::RPW, ROWS = PrefillCfg<G>::ROWS;
  PA_TL(const unsigned long long t_start = __builtin_amdgcn_s_memrealtime();)
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
  const int n = lane & 31;  // this lane's column
  const int h = lane >> 5;  // lane half: key offset 4h inside every 8 keys

  // column n -> (row n / G, head n % G) of this wave's rows
  const int row0 = qb * ROWS + wave * RPW;
  const int qrow = row0 + n / G;
  const bool col_valid = qrow < qlen;
  const int qrow_c = min(qrow, qlen - 1);
  const int pos = prior + qrow_c;
  const int head = g * G + n % G;
  const int pos_lo = prior + min(row0, qlen - 1);
  const int pos_hi = prior + min(row0 + RPW - 1, qlen - 1);
  const int wg_last = min(qb * ROWS + ROWS - 1, qlen - 1);
  const int ntiles = min((prior + wg_last + 1 + kKT - 1) / kKT, t_end);
  if (t_begin >= ntiles) return;

  // Q^T as the B operand: column n, head dims 16k + 8h .. 16k + 8h + 7
  u32x4 qv[T::KSTEPS];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(q0 + qrow_c) * H + head) * D);
#pragma unroll
    for (int k = 0; k < T::KSTEPS; ++k) qv[k] = qp[2 * k + h];
  }

  f32x16_t oacc[T::DMT];
#pragma unroll
  for (int i = 0; i < T::DMT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  float m = -INFINITY;  // reference maximum (log2 units) of this lane's column
  float lsum = 0.f;     // this lane's share of the column's sum
  float scale_log2 = a.scale * kLog2e;
  float out_scale = 1.f;
  if constexpr (FP8) {  // scores take the K scale, outputs the V scale of this KV head
    scale_log2 *= a.k_scale[g];
    out_scale = a.v_scale[g];
  }

  // Tile loads go straight from global memory into LDS (global_load_lds,
  // 16 bytes per lane): instruction i of wave w fills LDS chunks
  // (i * kWaves + w) * 64 + lane, i.e. chunk v = tid + kThreads * i, which
  // is position cpos = v % NCH of tile row kk = v / NCH.  The XOR swizzle of
  // the row's chunks is applied on the source side: that lane fetches chunk
  // cpos ^ swz(kk) of the key's row.  Keys past the sequence read the last
  // key's row instead (finite data: their probabilities are exactly 0, and
  // a stale slot may hold NaN, which 0 * NaN would carry into the output).
  const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
  const u32x4* vc = static_cast<const u32x4*>(a.v_cache);
  const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * T::NCH;  // chunks per slot
  const int rot = a.rot;
  int blk[T::NVEC];
  auto fetch_table = [&](int t) {
#pragma unroll
    for (int i = 0; i < T::NVEC; ++i) {
      const int key = min(t * kKT + (tid + kThreads * i) / T::NCH, L - 1);
      const int bi = max(min(key >> log2b, nblk - 1), 0);
      blk[i] = clampi(trow[bi], 0, num_blocks - 1);
    }
  };
  // a block's bytes fit 32 bits, so a chunk's byte offset is the block's
  // base (one 32 x 32 -> 64-bit multiply-add) plus a 32-bit offset in it
  const uint32_t blk_bytes = static_cast<uint32_t>(B * row_stride * 16);
  const uint32_t slot_bytes = static_cast<uint32_t>(row_stride * 16);
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // LDS destinations in scalars
  // tile t into the ring half kv (K tile, then V tile)
  auto load_tile = [&](int t, uint16_t* kv) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < T::NVEC; ++i) {
      const int v = tid + kThreads * i;
      const int kk = v / T::NCH;
      const int cpos = v % T::NCH;
      const int key = min(t * kKT + kk, L - 1);
      const int p = key & (B - 1);
      const uint32_t in_blk = p * slot_bytes + kv_head_pos(g, p, rot) * (T::NCH * 16);
      const uint64_t off = static_cast<uint64_t>(static_cast<uint32_t>(blk[i])) * blk_bytes + in_blk;
      const int base = (i * kWaves + wave_s) * 64 * 8;  // first bf16 of this wave's 64 chunks
      lds_dma16(reinterpret_cast<const char*>(kc) + off + ((cpos ^ T::swz_k(kk)) << 4), kv + base);
      lds_dma16(reinterpret_cast<const char*>(vc) + off + ((cpos ^ T::swz_v(kk)) << 4),
                kv + T::ELEMS + base);
    }
  };

  // One 64-key tile: S^T of both 32-key blocks, one lazy-rescale check for
  // the tile, then the probabilities and O^T += V^T P^T.  `masked` applies
  // the causal mask (only tiles that reach past this wave's first position
  // need it); apart from that branch and the rare rescale the body is
  // straight-line code, so the scheduler can overlap one block's exp2 work
  // with the other block's MFMAs.
  auto tile_body = [&](const void* ktile, const void* vtile, int tile0, bool masked)
                       __attribute__((always_inline)) {
    const uint16_t* kt = static_cast<const uint16_t*>(ktile);
    const uint16_t* vt = static_cast<const uint16_t*>(vtile);
    const uint8_t* kt8 = static_cast<const uint8_t*>(ktile);
    const uint8_t* vt8 = static_cast<const uint8_t*>(vtile);
    f32x16_t sacc[2];
    u32x4 kop[2][T::KSTEPS];
    // operands read in the order the MFMAs below consume them, so the first
    // MFMA waits for one read rather than for all of them; FP8 codes (8 per
    // lane: dims 16k + 8h .. +7 of the key row) are widened in registers
#pragma unroll
    for (int k = 0; k < T::KSTEPS; ++k)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int krow = kb * 32 + n;
        if constexpr (FP8)
          kop[kb][k] = fp8x8_bf16(*reinterpret_cast<const uint2*>(
              &kt8[krow * D + ((k ^ T::swz8(krow)) << 4) + 8 * h]));
        else
          kop[kb][k] = *reinterpret_cast<const u32x4*>(&kt[krow * D + (((2 * k + h) ^ T::swz_k(krow)) << 3)]);
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
    // the two blocks' accumulation chains alternate, so consecutive MFMAs
    // are independent
#pragma unroll
    for (int k = 0; k < T::KSTEPS; ++k)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma32(kop[kb][k], qv[k], sacc[kb]);
    // schedule: half the operand reads up front, then each MFMA pair followed
    // by the next two reads (reads stay in flight under the MFMAs, within
    // the registers two waves per SIMD leave)
    __builtin_amdgcn_sched_group_barrier(0x100, T::KSTEPS, 0);
#pragma unroll
    for (int i = 0; i < T::KSTEPS / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, T::KSTEPS, 0);
    // register i of block kb holds key tile0 + 32kb + 8(i/4) + 4h + i%4
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (tile0 + 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3) > pos) sacc[kb][i] = -INFINITY;
    }
    // maximum of raw scores (the scale is positive); v_maximum3 needs no
    // NaN canonicalisation of the MFMA results
    float rmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2)
        rmax = __builtin_elementwise_maximum(rmax, __builtin_elementwise_maximum(sacc[kb][i], sacc[kb][i + 1]));
    rmax = __builtin_elementwise_maximum(rmax, partner32(rmax));
    const float cmax = rmax * scale_log2;
    if (__any(cmax > m + kTauV)) {
      const float mn = fmaxf(m, cmax);
      const float alpha = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < T::DMT; ++i) oacc[i] *= alpha;
    }
    const float nmref = (m == -INFINITY) ? 0.f : -m;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // probabilities as bf16 B operands of the block's two 16-key steps
      u32x4 pb[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w[q] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * st + 2 * q], scale_log2, nmref)),
                           __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * st + 2 * q + 1], scale_log2, nmref)));
          lsum = dot2_bf16(w[q], 0x3F803F80u, lsum);  // + both rounded probabilities
        }
        pb[st] = u32x4{w[0], w[1], w[2], w[3]};
      }
      // O^T += V^T P^T
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u32x4 vop[T::DMT];
        if constexpr (FP8) {
          // one 8-bit transpose read per operand: source lane 2j + p of a
          // 16-lane group points at 8 dims (half p of the group's 16) of
          // the key holding k index j, so lane i receives dim 8p + i % 8 of
          // the 8 keys in k order
          const int j = (lane & 15) >> 1, p = lane & 1;
          const int key = kb * 32 + 16 * st + 4 * h + (j & 3) + 8 * (j >> 2);
#pragma unroll
          for (int dm = 0; dm < T::DMT; ++dm) {
            const int chunk = 2 * dm + ((lane >> 4) & 1);
            vop[dm] = fp8x8_bf16(lds_read_tr8(&vt8[key * D + ((chunk ^ T::swz8(key)) << 4) + 8 * p]));
          }
        } else {
          const int key = kb * 32 + 16 * st + 4 * h + ((lane & 15) >> 2);
#pragma unroll
          for (int dm = 0; dm < T::DMT; ++dm) {
            const int d0 = dm * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // this lane's 4-dim piece
            const int chunk = d0 >> 3;
            const uint2 lo = lds_read_tr(&vt[key * D + ((chunk ^ T::swz_v(key)) << 3) + (d0 & 7)]);
            const uint2 hi = lds_read_tr(&vt[(key + 8) * D + ((chunk ^ T::swz_v(key + 8)) << 3) + (d0 & 7)]);
            vop[dm] = u32x4{lo.x, lo.y, hi.x, hi.y};
          }
        }
#pragma unroll
        for (int dm = 0; dm < T::DMT; ++dm) oacc[dm] = mfma32(vop[dm], pb[st], oacc[dm]);
      }
    }
    // schedule of each block: the first step's V reads, then its MFMAs each
    // followed by the next step's reads for one operand, then the next
    // step's MFMAs
    constexpr int RPO = FP8 ? 1 : 2;  // LDS reads per V operand
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      __builtin_amdgcn_sched_group_barrier(0x100, RPO * T::DMT, 1);
#pragma unroll
      for (int dm = 0; dm < T::DMT; ++dm) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, RPO, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, T::DMT, 1);
    }
  };

  auto run_tile = [&](int t, const void* kt, const void* vt) __attribute__((always_inline)) {
    const int tile0 = t * kKT;
    if (tile0 <= pos_hi)  // some column of this wave sees keys of this tile
      tile_body(kt, vt, tile0, tile0 + kKT - 1 > pos_lo);
  };

  if constexpr (!FP8) {
    fetch_table(t_begin);
    load_tile(t_begin, lds0);
    fetch_table(t_begin + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // tile t+1 streams into the other half (freed by the last barrier) while
    // tile t is computed; its table entries arrived during tile t-1.  The
    // loop is unrolled by two so that every access names its half.
    auto step = [&](int t, uint16_t* cur, uint16_t* nxt) __attribute__((always_inline)) {
      if (t + 1 < ntiles) load_tile(t + 1, nxt);
      fetch_table(t + 2);
      run_tile(t, cur, cur + T::ELEMS);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's part of tile t+1 is in LDS
      __syncthreads();
    };
    for (int t = t_begin; t < ntiles; t += 2) {
      step(t, lds0, lds1);
      if (t + 1 < ntiles) step(t + 1, lds1, lds0);
    }
  } else {
    // FP8 caches: each tile's E4M3 codes (D bytes per key row, K rows then
    // V rows, 16-byte chunks swizzled by swz8 on the source side) stream
    // into the ring halves as the bf16 tiles do, and the MFMA operands are
    // read straight from the codes and widened in registers (see the tile
    // body); the KV head's scales are folded into the score scale and the
    // output.
    const uint8_t* kc8 = static_cast<const uint8_t*>(a.k_cache);
    const uint8_t* vc8 = static_cast<const uint8_t*>(a.v_cache);
    const int64_t row_bytes = static_cast<int64_t>(num_kv_heads) * D;
    const uint32_t row_bytes32 = static_cast<uint32_t>(row_bytes);
    const uint32_t blk_bytes8 = static_cast<uint32_t>(B * row_bytes);  // fits 32 bits
    int blk8[T::NVEC8];
    auto fetch_table8 = [&](int t) {
#pragma unroll
      for (int i = 0; i < T::NVEC8; ++i) {
        const int key = min(t * kKT + (tid + kThreads * i) / T::NCH8, L - 1);
        const int bi = max(min(key >> log2b, nblk - 1), 0);
        blk8[i] = clampi(trow[bi], 0, num_blocks - 1);
      }
    };
    // tile t into the ring half kv (K codes, then V codes)
    auto load_tile8 = [&](int t, uint16_t* kv) __attribute__((always_inline)) {
      uint8_t* sk = reinterpret_cast<uint8_t*>(kv);
      uint8_t* sv = sk + kKT * D;
#pragma unroll
      for (int i = 0; i < T::NVEC8; ++i) {
        const int v = tid + kThreads * i;
        const int kk = v / T::NCH8;
        const int cpos = v % T::NCH8;
        const int key = min(t * kKT + kk, L - 1);
        const int p = key & (B - 1);
        const uint64_t off = static_cast<uint64_t>(static_cast<uint32_t>(blk8[i])) * blk_bytes8 +
                             (p * row_bytes32 + kv_head_pos(g, p, rot) * D + ((cpos ^ T::swz8(kk)) << 4));
        const int base = (i * kWaves + wave_s) * 64 * 16;  // this wave's 64 chunks
        lds_dma16(kc8 + off, sk + base);
        lds_dma16(vc8 + off, sv + base);
      }
    };
    fetch_table8(t_begin);
    load_tile8(t_begin, lds0);
    fetch_table8(t_begin + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    auto step8 = [&](int t, uint16_t* cur, uint16_t* nxt) __attribute__((always_inline)) {
      if (t + 1 < ntiles) load_tile8(t + 1, nxt);
      fetch_table8(t + 2);
      const uint8_t* c8 = reinterpret_cast<const uint8_t*>(cur);
      run_tile(t, c8, c8 + kKT * D);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's part of tile t+1 is in LDS
      __syncthreads();
    };
    for (int t = t_begin; t < ntiles; t += 2) {
      step8(t, lds0, lds1);
      if (t + 1 < ntiles) step8(t + 1, lds1, lds0);
    }
  }

  PA_TL(const int64_t trace_wg = blockIdx.x + static_cast<int64_t>(gridDim.x) *
                                     (blockIdx.y + static_cast<int64_t>(gridDim.y) * blockIdx.z);
        if (a.trace && threadIdx.x == 0 && trace_wg < kTraceVarlenWgs) {
          unsigned long long* t = a.trace + trace_wg * 4;
          t[0] = t_start;
          t[1] = __builtin_amdgcn_s_memrealtime();
          t[2] = static_cast<unsigned long long>(ntiles - t_begin) |
                 (static_cast<unsigned long long>(qb) << 16) |
                 (static_cast<unsigned long long>(s) << 32) |
                 (static_cast<unsigned long long>(g) << 48) | (1ull << 62);
          t[3] = __builtin_amdgcn_s_getreg((31 << 11) | 20) |
                 (static_cast<unsigned long long>(__builtin_amdgcn_s_getreg((31 << 11) | 4)) << 32);
        })
  // column sums over both lane halves, normalise, store a valid column:
  // register i of M-tile dm holds dim 32 dm + 8(i/4) + 4h + i%4
  lsum += partner32(lsum);
  if (!col_valid) return;
  if (dst.part_o != nullptr) {
    // a piece of a split unit: unnormalised output (V scale applied) and
    // (max, sum) of the column
    const int64_t col = dst.col0 + wave * kCols + n;
    float* po = dst.part_o + col * D;
#pragma unroll
    for (int dm = 0; dm < T::DMT; ++dm)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(po + dm * 32 + 8 * j + 4 * h) =
            make_float4(oacc[dm][4 * j] * out_scale, oacc[dm][4 * j + 1] * out_scale,
                        oacc[dm][4 * j + 2] * out_scale, oacc[dm][4 * j + 3] * out_scale);
    if (h == 0) *reinterpret_cast<float2*>(dst.part_ml + col * 2) = make_float2(m, lsum);
    return;
  }
  const float inv = out_scale / lsum;
  uint16_t* op = static_cast<uint16_t*>(a.out) + (static_cast<int64_t>(q0 + qrow_c) * H + head) * D;
#pragma unroll
  for (int dm = 0; dm < T::DMT; ++dm)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint2 w = {pack_bf16(oacc[dm][4 * j] * inv, oacc[dm][4 * j + 1] * inv),
                       pack_bf16(oacc[dm][4 * j + 2] * inv, oacc[dm][4 * j + 3] * inv)};
      *reinterpret_cast<uint2*>(op + dm * 32 + 8 * j + 4 * h) = w;
    }
}

template <int D, int G, bool FP8>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
varlen_prefill_kernel(const VarlenArgs a, int32_t num_kv_heads, int32_t num_blocks,
                      int32_t log2b) {
  __shared__ __attribute__((aligned(16))) uint16_t lds0[2 * Tile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t lds1[2 * Tile<D>::ELEMS];
  prefill_body<D, G, FP8>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds0, lds1, num_kv_heads,
                          num_blocks, log2b, 0, INT32_MAX, PrefillDest{nullptr, nullptr, 0});
}

// Prefill units and pieces of a varlen batch.  Segment s with q_len >= 2
// has ceil(q_len / ROWS) units (query blocks), taken from the last (the
// most keys) to the first; unit qb needs tiles(s, qb) key tiles.  When the
// units of a KV head fill less than half of its `budget` workgroup slots
// (the workgroups that run on the chip at once, e.g. one long-context chunk
// of 512 rows: 16 units for 64 slots), each unit is cut into
// n = clamp(floor(tiles * budget / T), 1, tiles / kMinPieceTiles) key-range
// pieces (T = all units' tiles), piece p covering tiles
// [floor(p tiles / n), floor((p+1) tiles / n)); the pieces then number at
// most `budget` and all run at once, each writing (max, sum, output)
// partials that prefill_merge_kernel combines.  Otherwise every unit is
// one piece and writes its rows directly.  Pieces are numbered in segment
// order, units from the last query block, pieces in key order.  Lane l owns
// segments l*RPL .. l*RPL+RPL-1.
constexpr int kMinPieceTiles = 4;

// Keys before a segment's first query row, as prefill_body counts them.
__device__ __forceinline__ int segment_prior(const VarlenArgs& a, int s, int qlen, int block_size) {
  const int L = clampi(a.seq_lens[s], 0, min(a.max_seq_len, a.max_blocks_per_seq * block_size));
  return max(L - qlen, 0);
}

__device__ __forceinline__ int unit_tiles(int prior, int qlen, int qb, int rows) {
  return (prior + min(qb * rows + rows, qlen) + kKT - 1) / kKT;
}

struct PrefillPiece {
  int s, qb;   // unit
  int p, n;    // piece p of the unit's n
  int t0, t1;  // key tiles [t0, t1)
  int first;   // index of the unit's piece 0
  bool valid;
};

template <int ROWS, int RPL>
struct PrefillSplit {
  int qlen[RPL], prior[RPL], units[RPL], pieces[RPL];
  int unit_pre, piece_pre;
  int total_units, total_pieces, tiles_all, budget;
  bool split;

  __device__ int pieces_of(int t) const {
    if (!split) return 1;
    const int64_t n = static_cast<int64_t>(t) * budget / tiles_all;
    return static_cast<int>(max<int64_t>(1, min<int64_t>(n, t / kMinPieceTiles)));
  }

  __device__ void init(const VarlenArgs& a, int slots, int bsize) {
    const int lane = threadIdx.x & 63;
    budget = slots;
    // all loads first, then the arithmetic
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int r = min(lane * RPL + i, a.num_seqs - 1);
      const int q = a.query_start_loc[r + 1] - a.query_start_loc[r];
      qlen[i] = q;
      prior[i] = segment_prior(a, r, q, bsize);
    }
    int lane_tiles = 0, lane_units = 0;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      units[i] = (lane * RPL + i < a.num_seqs && qlen[i] >= 2) ? (qlen[i] + ROWS - 1) / ROWS : 0;
      for (int qb = 0; qb < units[i]; ++qb) lane_tiles += unit_tiles(prior[i], qlen[i], qb, ROWS);
      lane_units += units[i];
    }
    total_units = wave_sum(lane_units);
    unit_pre = wave_exclusive_scan(lane_units);
    tiles_all = wave_sum(lane_tiles);
    // within the host's bound the pieces number at most budget + units,
    // which is what the workspace holds
    split = budget > 0 && 2 * total_units <= budget && tiles_all > 0 &&
            total_units <= a.unit_bound;
    int lane_pieces = 0;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      pieces[i] = 0;
      if (split) {
        for (int qb = 0; qb < units[i]; ++qb)
          pieces[i] += pieces_of(unit_tiles(prior[i], qlen[i], qb, ROWS));
      } else {
        pieces[i] = units[i];
      }
      lane_pieces += pieces[i];
    }
    total_pieces = wave_sum(lane_pieces);
    piece_pre = wave_exclusive_scan(lane_pieces);
  }

  // The segment holding index x of a per-segment count (pieces or units),
  // x's offset in it and the segment's first index (wave-uniform).
  __device__ int locate(int x, bool by_pieces, int& off, int& base) const {
    const int lane = threadIdx.x & 63;
    int hit = -1, hpre = 0;
    int pre = by_pieces ? piece_pre : unit_pre;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int c = by_pieces ? pieces[i] : units[i];
      if (x >= pre && x < pre + c) {
        hit = i;
        hpre = pre;
      }
      pre += c;
    }
    const uint64_t mask = __ballot(hit >= 0);
    if (!mask) return -1;
    const int src = __builtin_ctzll(mask);
    base = __builtin_amdgcn_readlane(hpre, src);
    off = x - base;
    return __builtin_amdgcn_readlane(lane * RPL + hit, src);
  }

  // (q_len, prior) of segment seg (wave-uniform), from its owner lane
  __device__ void segment(int seg, int& q, int& pr) const {
    const int owner = seg / RPL, k = seg - owner * RPL;
    int qv = 0, pv = 0;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int qi = __shfl(qlen[i], owner), pi = __shfl(prior[i], owner);
      if (i == k) {
        qv = qi;
        pv = pi;
      }
    }
    q = __builtin_amdgcn_readfirstlane(qv);
    pr = __builtin_amdgcn_readfirstlane(pv);
  }

  __device__ PrefillPiece piece(int pi) const {
    PrefillPiece r{0, 0, 0, 1, 0, 0, 0, false};
    if (pi >= total_pieces) return r;
    int off = 0, base = 0;
    const int seg = locate(pi, true, off, base);
    if (seg < 0) return r;
    int q, pr;
    segment(seg, q, pr);
    const int nu = (q + ROWS - 1) / ROWS;
    int acc = 0;
    for (int qb = nu - 1; qb >= 0; --qb) {
      const int t = unit_tiles(pr, q, qb, ROWS);
      const int n = pieces_of(t);
      if (off < acc + n) {
        r.s = seg;
        r.qb = qb;
        r.p = off - acc;
        r.n = n;
        r.t0 = static_cast<int>(static_cast<int64_t>(r.p) * t / n);
        r.t1 = static_cast<int>(static_cast<int64_t>(r.p + 1) * t / n);
        r.first = base + acc;
        r.valid = true;
        return r;
      }
      acc += n;
    }
    return r;
  }

  // Unit u (units numbered like the pieces) and the index of its piece 0
  __device__ PrefillPiece unit(int u) const {
    PrefillPiece r{0, 0, 0, 1, 0, 0, 0, false};
    if (u >= total_units) return r;
    int off = 0, base = 0;
    const int seg = locate(u, false, off, base);
    if (seg < 0) return r;
    const int owner = seg / RPL;
    int pre = __shfl(piece_pre, owner);
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      if (i < seg - owner * RPL) pre += __shfl(pieces[i], owner);
    int q, pr;
    segment(seg, q, pr);
    const int nu = (q + ROWS - 1) / ROWS;
    const int qb = nu - 1 - off;
    int acc = 0;
    for (int k = nu - 1; k > qb; --k) acc += pieces_of(unit_tiles(pr, q, k, ROWS));
    r.s = seg;
    r.qb = qb;
    r.n = pieces_of(unit_tiles(pr, q, qb, ROWS));
    r.first = __builtin_amdgcn_readfirstlane(pre) + acc;
    r.valid = true;
    return r;
  }
};

// Runs workgroup wg's prefill piece if it has one; returns the number of
// prefill workgroups (pieces x KV heads).
template <int D, int G, bool FP8, int RPL>
__device__ __forceinline__ int prefill_dispatch_rpl(const VarlenArgs& va, int wg, uint16_t* lds0,
                                                    uint16_t* lds1, int32_t num_kv_heads,
                                                    int32_t num_blocks, int32_t log2b, int slots,
                                                    float* part_o, float* part_ml) {
  constexpr int ROWS = PrefillCfg<G>::ROWS;
  PrefillSplit<ROWS, RPL> sp;
  sp.init(va, slots, 1 << log2b);
  const int np = sp.total_pieces * num_kv_heads;
  if (wg < np) {
    const PrefillPiece pc = sp.piece(wg / num_kv_heads);
    const int g = wg % num_kv_heads;
    if (pc.valid) {
      PrefillDest dst{nullptr, nullptr, 0};
      if (pc.n > 1) {  // workspace columns of this piece and KV head
        dst.part_o = part_o;
        dst.part_ml = part_ml;
        dst.col0 = (static_cast<int64_t>(pc.first + pc.p) * num_kv_heads + g) * (kWaves * kCols);
      }
      prefill_body<D, G, FP8>(va, pc.qb, g, pc.s, lds0, lds1, num_kv_heads, num_blocks, log2b,
                              pc.t0, pc.t1, dst);
    }
  }
  return np;
}

template <int D, int G, bool FP8>
__device__ __forceinline__ int prefill_dispatch(const VarlenArgs& va, int wg, uint16_t* lds0,
                                                uint16_t* lds1, int32_t num_kv_heads,
                                                int32_t num_blocks, int32_t log2b, int slots,
                                                float* part_o, float* part_ml) {
  if (va.num_seqs <= 64)
    return prefill_dispatch_rpl<D, G, FP8, 1>(va, wg, lds0, lds1, num_kv_heads, num_blocks, log2b,
                                              slots, part_o, part_ml);
  if (va.num_seqs <= 256)
    return prefill_dispatch_rpl<D, G, FP8, 4>(va, wg, lds0, lds1, num_kv_heads, num_blocks, log2b,
                                              slots, part_o, part_ml);
  return prefill_dispatch_rpl<D, G, FP8, kPlanMaxRows / 64>(va, wg, lds0, lds1, num_kv_heads,
                                                            num_blocks, log2b, slots, part_o,
                                                            part_ml);
}

// Combines the pieces of cut prefill units: four workgroups per (unit, KV
// head), workgroup w taking the 32 columns of the unit's wave w; thread t
// takes column t / 8 and head dims 16 (t % 8) .. +15 of it.  out =
// sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, M = max_p m_p, in piece
// order.
template <int D, int G, int RPL>
__device__ void prefill_merge_rpl(const VarlenArgs& va, int32_t num_kv_heads, int32_t log2b, int slots,
                                  const float* part_o, const float* part_ml) {
  constexpr int ROWS = PrefillCfg<G>::ROWS, RPW = PrefillCfg<G>::RPW;
  constexpr int PARTS = 8, DPT = D / PARTS;  // threads per column, dims per thread
  static_assert(kThreads == kCols * PARTS, "one thread per (column, dim part)");
  PrefillSplit<ROWS, RPL> sp;
  sp.init(va, slots, 1 << log2b);
  if (!sp.split) return;
  const int item = blockIdx.x / kWaves, w = blockIdx.x % kWaves;  // (unit, head), column group
  const PrefillPiece un = sp.unit(item / num_kv_heads);
  const int g = item % num_kv_heads;
  if (!un.valid || un.n <= 1) return;
  const int n = threadIdx.x / PARTS, part = threadIdx.x % PARTS;
  const int q0 = va.query_start_loc[un.s];
  const int qlen = va.query_start_loc[un.s + 1] - q0;
  const int qrow = un.qb * ROWS + w * RPW + n / G;
  if (qrow >= qlen) return;
  const int H = num_kv_heads * G;
  const int64_t per_piece = static_cast<int64_t>(num_kv_heads) * (kWaves * kCols);  // columns
  const int64_t col0 = (static_cast<int64_t>(un.first) * num_kv_heads + g) * (kWaves * kCols) +
                       w * kCols + n;
  float M = -INFINITY;
  for (int p = 0; p < un.n; ++p) M = fmaxf(M, part_ml[(col0 + p * per_piece) * 2]);
  float acc[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
  float den = 0.f;
#pragma unroll 4
  for (int p = 0; p < un.n; ++p) {
    const int64_t col = col0 + p * per_piece;
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + col * 2);
    const float wt = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
    den = fmaf(wt, ml.y, den);
    const float4* src = reinterpret_cast<const float4*>(part_o + col * D + part * DPT);
#pragma unroll
    for (int e = 0; e < DPT / 4; ++e) {
      const float4 v = src[e];
      acc[4 * e] = fmaf(wt, v.x, acc[4 * e]);
      acc[4 * e + 1] = fmaf(wt, v.y, acc[4 * e + 1]);
      acc[4 * e + 2] = fmaf(wt, v.z, acc[4 * e + 2]);
      acc[4 * e + 3] = fmaf(wt, v.w, acc[4 * e + 3]);
    }
  }
  const float inv = 1.f / den;
  u32x4* op = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(va.out) +
      (static_cast<int64_t>(q0 + qrow) * H + g * G + n % G) * D + part * DPT);
#pragma unroll
  for (int e = 0; e < DPT / 8; ++e)
    op[e] = u32x4{pack_bf16(acc[8 * e] * inv, acc[8 * e + 1] * inv),
                  pack_bf16(acc[8 * e + 2] * inv, acc[8 * e + 3] * inv),
                  pack_bf16(acc[8 * e + 4] * inv, acc[8 * e + 5] * inv),
                  pack_bf16(acc[8 * e + 6] * inv, acc[8 * e + 7] * inv)};
}

template <int D, int G>
__global__ void __launch_bounds__(kThreads)
prefill_merge_kernel(const VarlenArgs va, int32_t num_kv_heads, int32_t log2b, int32_t slots,
                     const float* part_o, const float* part_ml) {
  if (va.num_seqs <= 64) prefill_merge_rpl<D, G, 1>(va, num_kv_heads, log2b, slots, part_o, part_ml);
  else if (va.num_seqs <= 256) prefill_merge_rpl<D, G, 4>(va, num_kv_heads, log2b, slots, part_o, part_ml);
  else prefill_merge_rpl<D, G, kPlanMaxRows / 64>(va, num_kv_heads, log2b, slots, part_o, part_ml);
}

// One launch for a whole varlen step (bf16): the first units x H_kv
// workgroups run the prefill units (KV head fastest, so the query blocks of
// one KV head share an XCD and its L2), the next ones run 4 decode
// wavefronts each (the balanced split of the one-row segments, KV head
// fastest); the remaining workgroups of the host's upper bound exit.
// Workgroups are dispatched in index order, so the compute-bound prefill
// units start first and the memory-bound decode waves take each workgroup
// slot as soon as its prefill workgroup ends, instead of waiting for the
// slowest one.  (Issuing one prefill and one decode workgroup per CU first,
// so that the two kinds share CUs, measured 30% slower: the prefill then
// runs one wave per SIMD and becomes the critical path.)
template <int D, int G, bool FP8>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
varlen_fused_kernel(const VarlenArgs va, const DecodeArgs da, int32_t num_kv_heads,
                    int32_t num_blocks, int32_t log2b, int32_t slots, float* part_o,
                    float* part_ml) {
  // prefill tiles (lds0, lds1), or the four decode waves' work lists and
  // tables (lds0)
  constexpr int kHalf = 2 * Tile<D>::ELEMS;
  constexpr int kLds0 = kHalf > kWaves * kDecodeLdsInts * 2 ? kHalf : kWaves * kDecodeLdsInts * 2;
  __shared__ __attribute__((aligned(16))) uint16_t lds0[kLds0];
  __shared__ __attribute__((aligned(16))) uint16_t lds1[kHalf];
  const int wg = blockIdx.x;
  PA_TL(const unsigned long long t_start = __builtin_amdgcn_s_memrealtime();)
  // The first kDecodeFirst workgroups are decode ones: with bf16 caches the
  // decode rows' reads then start beside the prefill units instead of
  // waiting for the short units to free their slots (FP8 prefill, which
  // widens its codes in registers, loses more to them than the decode gains)
  constexpr int kDecodeFirst = FP8 ? 0 : 96;
  const int nd = (da.max_partitions * num_kv_heads + kWaves - 1) / kWaves;  // decode workgroups
  const int d0 = min(kDecodeFirst, nd);
  int dwg;  // decode workgroup index
  if (wg < d0) {
    dwg = wg;
  } else {
    const int np = prefill_dispatch<D, G, FP8>(va, wg - d0, lds0, lds1, num_kv_heads, num_blocks,
                                               log2b, slots, part_o, part_ml);
    if (wg - d0 < np) return;
    dwg = wg - np;
  }
  const int wave = threadIdx.x >> 6;
  const int item = dwg * kWaves + wave;
  const int y = item / num_kv_heads;
  // decode workgroups: wave 0's start and end
  PA_TL(struct TraceEnd {
          unsigned long long* t;
          unsigned long long t0;
          __device__ ~TraceEnd() {
            if (!t) return;
            t[0] = t0;
            t[1] = __builtin_amdgcn_s_memrealtime();
            t[2] = 2ull << 62;
            t[3] = __builtin_amdgcn_s_getreg((31 << 11) | 20);
          }
        } trace_end{(va.trace && threadIdx.x == 0 && wg < kTraceVarlenWgs) ? va.trace + wg * 4
                                                                            : nullptr,
                    t_start};)
  if (y >= da.max_partitions) return;
  // FP8 waves of 8 heads keep the per-chunk offsets: the hoisted ones would
  // not fit the 256 registers two waves per SIMD leave
  int32_t* wl = reinterpret_cast<int32_t*>(lds0) + wave * kDecodeLdsInts;
  if constexpr (UseMfma<true, D, G>::value)
    decode_mfma_body<G, FP8>(da, item % num_kv_heads, y, 0, wl, num_kv_heads, num_blocks, log2b);
  else
    decode_partition_body<true, D, G, FP8, !(FP8 && G >= 8)>(da, item % num_kv_heads, y, 0, wl,
                                                             num_kv_heads, num_blocks, log2b);
}

bool varlen_prefill_supported(const pa_cache_dims& d) {
  if (d.dtype != PA_DTYPE_BF16 && d.dtype != PA_DTYPE_FP8_E4M3) return false;
  if (d.head_dim != 64 && d.head_dim != 128) return false;
  const int G = d.num_heads / d.num_kv_heads;
  return G == 1 || G == 2 || G == 4 || G == 8 || G == 16;
}

template <int D, int G, bool FP8>
static hipError_t launch_prefill_t(const VarlenArgs& a, const pa_cache_dims& d, hipStream_t st) {
  constexpr int ROWS = PrefillCfg<G>::ROWS;
  const dim3 grid((a.max_query_len + ROWS - 1) / ROWS, d.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((varlen_prefill_kernel<D, G, FP8>), grid, dim3(kThreads), 0, st, a,
                     d.num_kv_heads, d.num_blocks, ilog2(d.block_size));
  return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t prefill_group(const VarlenArgs& a, const pa_cache_dims& d, hipStream_t st) {
  switch (d.num_heads / d.num_kv_heads) {
    case 1: return launch_prefill_t<D, 1, FP8>(a, d, st);
    case 2: return launch_prefill_t<D, 2, FP8>(a, d, st);
    case 4: return launch_prefill_t<D, 4, FP8>(a, d, st);
    case 8: return launch_prefill_t<D, 8, FP8>(a, d, st);
    case 16: return launch_prefill_t<D, 16, FP8>(a, d, st);
    default: return hipErrorInvalidValue;
  }
}

int32_t varlen_prefill_cols() { return kWaves * kCols; }

int32_t varlen_prefill_rows(const pa_cache_dims& d) {
  return kWaves * kCols / (d.num_heads / d.num_kv_heads);  // PrefillCfg<G>::ROWS
}

template <int D, int G, bool FP8>
static hipError_t launch_fused_t(const VarlenArgs& va, const DecodeArgs& da, const pa_cache_dims& d,
                                 const PrefillSplitArgs& ps, hipStream_t st) {
  const int64_t items = static_cast<int64_t>(d.num_kv_heads) * da.max_partitions;
  const int64_t pieces = static_cast<int64_t>(ps.unit_bound) + ps.slots;
  const int64_t grid = pieces * d.num_kv_heads + (items + kWaves - 1) / kWaves;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  const int log2b = ilog2(d.block_size);
  hipLaunchKernelGGL((varlen_fused_kernel<D, G, FP8>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                     st, va, da, d.num_kv_heads, d.num_blocks, log2b, ps.slots, ps.part_o, ps.part_ml);
  if (hipError_t e = hipGetLastError(); e != hipSuccess || ps.slots <= 0) return e;
  hipLaunchKernelGGL((prefill_merge_kernel<D, G>),
                     dim3(static_cast<unsigned>(static_cast<int64_t>(ps.unit_bound) * d.num_kv_heads * kWaves)),
                     dim3(kThreads), 0, st, va, d.num_kv_heads, log2b, ps.slots, ps.part_o, ps.part_ml);
  return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t fused_group(const VarlenArgs& va, const DecodeArgs& da, const pa_cache_dims& d,
                              const PrefillSplitArgs& ps, hipStream_t st) {
  switch (d.num_heads / d.num_kv_heads) {
    case 1: return launch_fused_t<D, 1, FP8>(va, da, d, ps, st);
    case 2: return launch_fused_t<D, 2, FP8>(va, da, d, ps, st);
    case 4: return launch_fused_t<D, 4, FP8>(va, da, d, ps, st);
    case 8: return launch_fused_t<D, 8, FP8>(va, da, d, ps, st);
    default: return hipErrorInvalidValue;
  }
}

// G = 16's decode waves need more registers than two waves per SIMD allow,
// so that grouping keeps separate launches.
bool varlen_fused_supported(const pa_cache_dims& d) {
  return varlen_prefill_supported(d) && decode_supported(d) && d.num_heads / d.num_kv_heads <= 8;
}

hipError_t launch_varlen_fused(const VarlenArgs& va, const DecodeArgs& da, const pa_cache_dims& d,
                               const PrefillSplitArgs& ps, hipStream_t stream) {
  if (!varlen_fused_supported(d) || va.num_seqs > kPlanMaxRows || !da.balanced || ps.slots < 0 ||
      (ps.slots > 0 && (ps.part_o == nullptr || ps.part_ml == nullptr)))
    return hipErrorInvalidValue;
  if (d.dtype == PA_DTYPE_FP8_E4M3)
    return d.head_dim == 128 ? fused_group<128, true>(va, da, d, ps, stream)
                             : fused_group<64, true>(va, da, d, ps, stream);
  return d.head_dim == 128 ? fused_group<128, false>(va, da, d, ps, stream)
                           : fused_group<64, false>(va, da, d, ps, stream);
}

hipError_t launch_varlen_prefill(const VarlenArgs& a, const pa_cache_dims& d, hipStream_t stream) {
  if (!varlen_prefill_supported(d)) return hipErrorInvalidValue;
  if (a.max_query_len < 2 || a.num_seqs == 0) return hipSuccess;
  if (d.dtype == PA_DTYPE_FP8_E4M3)
    return d.head_dim == 128 ? prefill_group<128, true>(a, d, stream) : prefill_group<64, true>(a, d, stream);
  return d.head_dim == 128 ? prefill_group<128, false>(a, d, stream) : prefill_group<64, false>(a, d, stream);
}

}  // namespace pa
