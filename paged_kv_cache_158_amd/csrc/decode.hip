// Paged decode attention for gfx950: split-K partitions over the block table
// and a log-sum-exp merge.
//
// What is computed (SourceAIX vLLM page §5.1.1, decode step): for sequence s
// and query head h, softmax over the s's context tokens t of
// scale * q[s][h] . K[t][h/G], weighted sum of V[t][h/G], where token t lives
// in slot block_tables[s][t / B] * B + t % B of the paged cache.
//
// Work decomposition.  One wavefront (64 lanes) per (kv head, partition,
// sequence): it serves all G query heads that share the KV head, so each
// K/V byte is read from HBM once.  Inside the wave, a token row of D
// elements is read by LPT lanes with one 16-byte load each (LPT = 16 for
// bf16 D=128), so a wave load instruction covers TPI = 64/LPT tokens and
// lane row r owns J = 4 consecutive tokens of every CHUNK = TPI*J tokens.
//
// Scores.  Each lane forms partial dot products over its 16 bytes for every
// (head, token) pair, then a reduce-scatter across the LPT lanes of its row:
// the first log2(G) exchange stages each halve the set of heads a lane
// keeps (the halves are chosen by loading q into lane-dependent head slots,
// so no select is needed), the remaining stages all-reduce.  Afterwards
// every lane holds the full scores of ONE head for its row's J tokens, so
// the exponentials are computed once per (row, head, token), not LPT times.
//
// Online softmax in base 2 with a lazily moved reference maximum: the
// reference only moves (and the accumulators are rescaled) when a score
// exceeds it by more than 2^8, which keeps exp2 values in [0, 256].  PV:
// probabilities of each head are broadcast inside the row and, for bf16,
// rounded to bf16 pairs so that v_dot2_f32_bf16 consumes two tokens per
// instruction; the softmax denominator sums the same rounded values.
//
// The J tokens of a row always lie in one block (B >= 4, rows start at a
// multiple of 4), so each lane needs one block-table entry per chunk; the
// entries of all the wave's row segments are staged in LDS once, clamped
// into [0, num_blocks).
//
// Work: a wave processes a list of row segments (the balanced split gives
// every wave an equal share of all rows' chunks, which may span rows; the
// fixed split one partition).  For each segment it writes the (max, sum,
// unnormalised output) of each head, or, when the segment is the whole row,
// the normalised output directly, and the merge kernel skips that row.
#include <cfloat>
#include <cmath>

#include "decode_body.h"
#include "decode_mfma.h"

namespace pa {

template <bool BF16, int D, int G, bool FP8>
__global__ void __launch_bounds__(64)
decode_partition_kernel(const DecodeArgs a, int32_t num_kv_heads, int32_t num_blocks,
                        int32_t log2b) {
  __shared__ __attribute__((aligned(16))) int32_t lds[kDecodeLdsInts];
  decode_partition_body<BF16, D, G, FP8>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds, num_kv_heads,
                                         num_blocks, log2b);
}

// The matrix-core wave (bf16 and FP8 caches, head dim 128, 4-16 heads per
// KV head), held to two waves per SIMD.  A workgroup holds MfmaGroup waves
// of one KV head, ranges y = MfmaGroup * grid y + wave; with shared
// prefixes they split the plan's table probes between them.  FP8 waves run
// one per workgroup: the split's registers cost their wave more than the
// probes it saves.
template <bool FP8>
struct MfmaGroup {
  static constexpr int value = FP8 ? 1 : 4;
};
template <int G, bool FP8>
__global__ void __launch_bounds__(64 * MfmaGroup<FP8>::value) __attribute__((amdgpu_waves_per_eu(2)))
decode_mfma_kernel(const DecodeArgs a, int32_t num_kv_heads, int32_t num_blocks, int32_t log2b) {
  constexpr int NW = MfmaGroup<FP8>::value;
  __shared__ __attribute__((aligned(16))) int32_t lds[NW * (kDecodeLdsInts + 64)];
  const int w = NW > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  decode_mfma_body<G, FP8>(a, blockIdx.x, blockIdx.y * NW + w, blockIdx.z,
                           lds + w * kDecodeLdsInts, num_kv_heads, num_blocks, log2b,
                           lds + NW * kDecodeLdsInts, w, NW);
}

// Log-sum-exp combination, by one wave, of `count` of one (row, query head)'s
// partitions: p = p0 + k * pstep, k < count, in that order.  Partition p < nown
// is the row's own (workspace index base + p stride); with SH a later one is
// its group's shared partial (index sbase + (p - nown) sstride of the shared
// region).  Leaves M = the partitions' largest max, lsum = sum_p 2^(m_p - M)
// l_p and acc = sum_p 2^(m_p - M) o_p for this lane's D / 64 dims (M = -inf,
// zeros for count 0).
template <int D, bool SH>
__device__ __forceinline__ void merge_part(const DecodeArgs& a, int nown, int p0, int pstep,
                                           int count, int64_t base, int64_t stride,
                                           int64_t sbase, int64_t sstride, float& M,
                                           float& lsum_out, float (&acc)[D / 64]) {
  constexpr int DPL = D / 64;  // dims per lane
  constexpr int NB = 8;        // partitions whose o rows are loaded together
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  M = -INFINITY;
  lsum_out = 0.f;
  if (count <= 0) return;
  auto ml_at = [&](int k) -> float2 {
    const int p = p0 + k * pstep;
    if constexpr (SH) {
      if (p >= nown) return reinterpret_cast<const float2*>(a.sh_ml)[sbase + (p - nown) * sstride];
    }
    return reinterpret_cast<const float2*>(a.part_ml)[base + p * stride];
  };
  auto o_at = [&](int k) -> const float* {
    const int p = p0 + k * pstep;
    if constexpr (SH) {
      if (p >= nown) return a.sh_o + (sbase + (p - nown) * sstride) * D + lane * DPL;
    }
    return a.part_o + (base + p * stride) * D + lane * DPL;
  };

  // o rows of partitions j0 .. j0+NB-1 of the window starting at k0
  // (indices past the window's cnt partitions are clamped onto its last)
  auto load_batch = [&](float (&x)[NB][DPL], int k0, int j0, int cnt) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float* src = o_at(k0 + min(j0 + j, cnt - 1));
      if constexpr (DPL == 2) {
        const float2 t = *reinterpret_cast<const float2*>(src);
        x[j][0] = t.x;
        x[j][DPL - 1] = t.y;
      } else {
        x[j][0] = src[0];
      }
    }
  };
  // weights 2^(m_p - M) of the window's partitions sit in lane k - k0
  auto add_batch = [&](const float (&x)[NB][DPL], float wl, int j0, int cnt) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float wj = j0 + j < cnt ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                          __builtin_bit_cast(int, wl), min(j0 + j, 63)))
                                    : 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] = fmaf(wj, x[j][i], acc[i]);
    }
  };

  // lane k holds (m, l) of partition k (then k + 64, ...); its load and the
  // first NB o rows are in flight together
  const int cnt0 = min(64, count);
  const float2 v0 = lane < count ? ml_at(lane) : make_float2(-INFINITY, 0.f);
  float x0[NB][DPL];
  load_batch(x0, 0, 0, cnt0);
  float mx = v0.x;
  for (int k = lane + 64; k < count; k += 64) mx = fmaxf(mx, ml_at(k).x);
  mx = wave_max_f(mx);
  float lsum = 0.f;
  for (int k = lane; k < count; k += 64) {
    const float2 u = k == lane ? v0 : ml_at(k);
    lsum += (u.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(u.x - mx) * u.y;
  }
  lsum = wave_sum_f(lsum);

  // numerator, in partition order
  for (int k0 = 0; k0 < count; k0 += 64) {
    const int cnt = min(64, count - k0);
    const float2 u = k0 == 0 ? v0 : (lane < cnt ? ml_at(k0 + lane) : make_float2(-INFINITY, 0.f));
    const float wl = (u.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(u.x - mx);
    int j0 = 0;
    if (k0 == 0) {
      add_batch(x0, wl, 0, cnt);
      j0 = NB;
    }
    for (; j0 < cnt; j0 += NB) {
      float x[NB][DPL];
      load_batch(x, k0, j0, cnt);
      add_batch(x, wl, j0, cnt);
    }
  }
  M = mx;
  lsum_out = lsum;
}

// out row of this lane's dims: acc / lsum in the output dtype
template <bool BF16, int D>
__device__ __forceinline__ void store_row(const DecodeArgs& a, int64_t off, const float (&acc)[D / 64],
                                          float lsum) {
  constexpr int DPL = D / 64;
  const float inv = 1.f / lsum;
  off += (threadIdx.x & 63) * DPL;
  if constexpr (BF16) {
    if constexpr (DPL == 2) {
      reinterpret_cast<uint32_t*>(a.out)[off / 2] = pack_bf16(acc[0] * inv, acc[1] * inv);
    } else {
      const uint32_t pk = pack_bf16(acc[0] * inv, 0.f);
      reinterpret_cast<uint16_t*>(a.out)[off] = static_cast<uint16_t>(pk & 0xffffu);
    }
  } else {
#pragma unroll
    for (int i = 0; i < DPL; ++i) static_cast<float*>(a.out)[off + i] = acc[i] * inv;
  }
}

// The merge of one (row, query head) by WAVES waves: wave w combines the
// partitions w, w + WAVES, ... (merge_part), then wave 0 combines the waves'
// results in wave order, out = sum_w 2^(M_w - M) acc_w / sum_w 2^(M_w - M)
// lsum_w.  One wave for ordinary batches; 16 when few (row, head) pairs
// hold many partitions each (a long row split over many waves), so that
// their loads do not queue in one wave.
template <bool BF16, int D, int WAVES, bool SH>
__device__ __forceinline__ void merge_row(const DecodeArgs& a, int64_t off, int nown, int nparts,
                                          int64_t base, int64_t stride, int64_t sbase,
                                          int64_t sstride) {
  constexpr int DPL = D / 64;
  float M, lsum, acc[DPL];
  if constexpr (WAVES == 1) {
    merge_part<D, SH>(a, nown, 0, 1, nparts, base, stride, sbase, sstride, M, lsum, acc);
    store_row<BF16, D>(a, off, acc, lsum);
  } else {
    __shared__ float part_acc[WAVES][D];
    __shared__ float part_ml[WAVES][2];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int count = nparts > w ? (nparts - w + WAVES - 1) / WAVES : 0;
    merge_part<D, SH>(a, nown, w, WAVES, count, base, stride, sbase, sstride, M, lsum, acc);
#pragma unroll
    for (int i = 0; i < DPL; ++i) part_acc[w][lane * DPL + i] = acc[i];
    if (lane == 0) {
      part_ml[w][0] = M;
      part_ml[w][1] = lsum;
    }
    __syncthreads();
    if (w != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) Mt = fmaxf(Mt, part_ml[v][0]);
    float tot = 0.f, out[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) out[i] = 0.f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) {
      const float f = part_ml[v][0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(part_ml[v][0] - Mt);
      tot += f * part_ml[v][1];
#pragma unroll
      for (int i = 0; i < DPL; ++i) out[i] = fmaf(f, part_acc[v][lane * DPL + i], out[i]);
    }
    store_row<BF16, D>(a, off, out, tot);
  }
}

// One workgroup of WAVES waves per (query head, sequence): the merge of its
// partials, or nothing when the partition kernel wrote the output directly.
template <bool BF16, int D, int WAVES>
__global__ void __launch_bounds__(64 * WAVES)
decode_merge_kernel(const DecodeArgs a, int32_t num_heads, int32_t num_kv_heads,
                    int32_t block_size) {
  const int h = blockIdx.x;
  const int zrow = blockIdx.y;
  // the plan entries do not depend on the row lookup: all loads in flight
  int2 pl = make_int2(0, 0), ps = make_int2(0, 0);
  if (a.balanced) pl = *reinterpret_cast<const int2*>(a.plan + 2 * static_cast<int64_t>(zrow));
  if (a.share) ps = *reinterpret_cast<const int2*>(a.plan_sh + 2 * static_cast<int64_t>(zrow));
  const RowInfo ri = row_info(a, zrow, block_size);
  if (!ri.active) return;
  int nown;
  int64_t base, stride;  // workspace index of own partition p: base + p * stride
  if (a.balanced) {
    nown = pl.y;
    base = static_cast<int64_t>(pl.x) * num_heads + h;
    stride = num_heads;
  } else {
    nown = min((ri.ctx + a.partition_size - 1) / a.partition_size, a.max_partitions);
    base = (static_cast<int64_t>(zrow) * num_heads + h) * a.max_partitions;
    stride = 1;
  }
  const int nsh = ps.y & 0xFFFF;
  const int64_t off = (static_cast<int64_t>(ri.q_row) * num_heads + h) * D;
  if (nsh == 0) {
    if (nown > 1) merge_row<BF16, D, WAVES, false>(a, off, nown, nown, base, stride, 0, 0);
    return;  // else written by the partition kernel
  }
  // shared partition p: index ((ps.x + p) H_kv + g) 16 + m G + h mod G
  const int G = num_heads / num_kv_heads;
  const int64_t sbase = (static_cast<int64_t>(ps.x) * num_kv_heads + h / G) * kShareCols +
                        (ps.y >> 16) * G + h % G;
  merge_row<BF16, D, WAVES, true>(a, off, nown, nown + nsh, base, stride, sbase,
                                  static_cast<int64_t>(num_kv_heads) * kShareCols);
}

template <bool BF16, int D, int G, bool FP8>
static hipError_t launch_partials_t(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t stream) {
  const int log2b = ilog2(d.block_size);
  dim3 grid(d.num_kv_heads, a.max_partitions, a.balanced ? 1 : a.num_rows);
  if constexpr (UseMfma<BF16, D, G>::value)
    hipLaunchKernelGGL((decode_mfma_kernel<G, FP8>),
                       dim3(grid.x, (grid.y + MfmaGroup<FP8>::value - 1) / MfmaGroup<FP8>::value,
                            grid.z),
                       dim3(64 * MfmaGroup<FP8>::value), 0, stream, a, d.num_kv_heads,
                       d.num_blocks, log2b);
  else
    hipLaunchKernelGGL((decode_partition_kernel<BF16, D, G, FP8>), grid, dim3(64), 0, stream, a,
                       d.num_kv_heads, d.num_blocks, log2b);
  return hipGetLastError();
}

template <bool BF16, int D, bool FP8 = false>
static hipError_t dispatch_group(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t s) {
  switch (d.num_heads / d.num_kv_heads) {
    case 1: return launch_partials_t<BF16, D, 1, FP8>(a, d, s);
    case 2: return launch_partials_t<BF16, D, 2, FP8>(a, d, s);
    case 4: return launch_partials_t<BF16, D, 4, FP8>(a, d, s);
    case 8: return launch_partials_t<BF16, D, 8, FP8>(a, d, s);
    case 16:
      if constexpr (Geo<BF16, D>::NST >= 4) return launch_partials_t<BF16, D, 16, FP8>(a, d, s);
      else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

bool decode_supported(const pa_cache_dims& d) {
  if (d.head_dim != 64 && d.head_dim != 128) return false;
  if (d.dtype != PA_DTYPE_BF16 && d.dtype != PA_DTYPE_F32 && d.dtype != PA_DTYPE_FP8_E4M3)
    return false;
  const int G = d.num_heads / d.num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return false;
  if (G == 16 && d.dtype != PA_DTYPE_F32 && d.head_dim == 64) return false;
  return true;
}

hipError_t launch_decode_partials(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t stream) {
  if (!decode_supported(d)) return hipErrorInvalidValue;
  if (d.dtype == PA_DTYPE_FP8_E4M3) {
    return d.head_dim == 128 ? dispatch_group<true, 128, true>(a, d, stream)
                             : dispatch_group<true, 64, true>(a, d, stream);
  }
  if (d.dtype == PA_DTYPE_BF16) {
    return d.head_dim == 128 ? dispatch_group<true, 128>(a, d, stream)
                             : dispatch_group<true, 64>(a, d, stream);
  }
  return d.head_dim == 128 ? dispatch_group<false, 128>(a, d, stream)
                           : dispatch_group<false, 64>(a, d, stream);
}

template <bool BF16, int D>
static void launch_merge_t(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t stream) {
  const dim3 grid(d.num_heads, a.num_rows);
  // few (row, head) pairs over many waves each (a long row split over many
  // waves): 16 waves per pair so that its partials' loads do not queue
  const bool wide = a.balanced && static_cast<int64_t>(a.num_rows) * d.num_heads <= 256 &&
                    a.max_partitions >= 64;
  if (wide)
    hipLaunchKernelGGL((decode_merge_kernel<BF16, D, 16>), grid, dim3(1024), 0, stream, a,
                       d.num_heads, d.num_kv_heads, d.block_size);
  else
    hipLaunchKernelGGL((decode_merge_kernel<BF16, D, 1>), grid, dim3(64), 0, stream, a,
                       d.num_heads, d.num_kv_heads, d.block_size);
}

hipError_t launch_decode_merge(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t stream) {
  if (a.max_partitions <= 1) return hipSuccess;
  if (d.dtype != PA_DTYPE_F32) {  // bf16 output (bf16 and FP8 caches)
    if (d.head_dim == 128) launch_merge_t<true, 128>(a, d, stream);
    else launch_merge_t<true, 64>(a, d, stream);
  } else {
    if (d.head_dim == 128) launch_merge_t<false, 128>(a, d, stream);
    else launch_merge_t<false, 64>(a, d, stream);
  }
  return hipGetLastError();
}

}  // namespace pa
