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
// KV head), held to two waves per SIMD.
template <int G, bool FP8>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
decode_mfma_kernel(const DecodeArgs a, int32_t num_kv_heads, int32_t num_blocks, int32_t log2b) {
  __shared__ __attribute__((aligned(16))) int32_t lds[kDecodeLdsInts];
  decode_mfma_body<G, FP8>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds, num_kv_heads, num_blocks,
                           log2b);
}

// Log-sum-exp merge of one (row, query head): out = sum_p 2^(m_p - M) o_p /
// sum_p 2^(m_p - M) l_p, M = max_p m_p, over the row's own partitions p <
// nown (workspace index base + p stride) and then, with SH, its group's
// shared ones (index sbase + (p - nown) sstride of the shared region), in
// that fixed order.
template <bool BF16, int D, bool SH>
__device__ __forceinline__ void merge_row(const DecodeArgs& a, int64_t off, int nown, int nparts,
                                          int64_t base, int64_t stride, int64_t sbase,
                                          int64_t sstride) {
  constexpr int DPL = D / 64;  // dims per lane
  constexpr int NB = 8;        // partitions whose o rows are loaded together
  const int lane = threadIdx.x;
  auto ml_at = [&](int p) -> float2 {
    if constexpr (SH) {
      if (p >= nown) return reinterpret_cast<const float2*>(a.sh_ml)[sbase + (p - nown) * sstride];
    }
    return reinterpret_cast<const float2*>(a.part_ml)[base + p * stride];
  };
  auto o_at = [&](int p) -> const float* {
    if constexpr (SH) {
      if (p >= nown) return a.sh_o + (sbase + (p - nown) * sstride) * D + lane * DPL;
    }
    return a.part_o + (base + p * stride) * D + lane * DPL;
  };

  // o rows of partitions j0 .. j0+NB-1 of the window starting at p0
  // (indices past the window's cnt partitions are clamped onto its last)
  auto load_batch = [&](float (&x)[NB][DPL], int p0, int j0, int cnt) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float* src = o_at(p0 + min(j0 + j, cnt - 1));
      if constexpr (DPL == 2) {
        const float2 t = *reinterpret_cast<const float2*>(src);
        x[j][0] = t.x;
        x[j][DPL - 1] = t.y;
      } else {
        x[j][0] = src[0];
      }
    }
  };
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  // weights 2^(m_p - M) of the window's partitions sit in lane p - p0
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

  // lane p holds (m, l) of partition p (then p + 64, ...); its load and the
  // first NB o rows are in flight together
  const int cnt0 = min(64, nparts);
  const float2 v0 = lane < nparts ? ml_at(lane) : make_float2(-INFINITY, 0.f);
  float x0[NB][DPL];
  load_batch(x0, 0, 0, cnt0);
  float mx = v0.x;
  for (int p = lane + 64; p < nparts; p += 64) mx = fmaxf(mx, ml_at(p).x);
  mx = wave_max_f(mx);
  float lsum = 0.f;
  for (int p = lane; p < nparts; p += 64) {
    const float2 u = p == lane ? v0 : ml_at(p);
    lsum += (u.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(u.x - mx) * u.y;
  }
  lsum = wave_sum_f(lsum);

  // numerator, in partition order
  for (int p0 = 0; p0 < nparts; p0 += 64) {
    const int cnt = min(64, nparts - p0);
    const float2 u = p0 == 0 ? v0 : (lane < cnt ? ml_at(p0 + lane) : make_float2(-INFINITY, 0.f));
    const float wl = (u.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(u.x - mx);
    int j0 = 0;
    if (p0 == 0) {
      add_batch(x0, wl, 0, cnt);
      j0 = NB;
    }
    for (; j0 < cnt; j0 += NB) {
      float x[NB][DPL];
      load_batch(x, p0, j0, cnt);
      add_batch(x, wl, j0, cnt);
    }
  }
  const float inv = 1.f / lsum;
  off += lane * DPL;
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

// One wave per (query head, sequence): the merge of its partials, or
// nothing when the partition kernel wrote the output directly.
template <bool BF16, int D>
__global__ void __launch_bounds__(64)
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
    if (nown > 1) merge_row<BF16, D, false>(a, off, nown, nown, base, stride, 0, 0);
    return;  // else written by the partition kernel
  }
  // shared partition p: index ((ps.x + p) H_kv + g) 16 + m G + h mod G
  const int G = num_heads / num_kv_heads;
  const int64_t sbase = (static_cast<int64_t>(ps.x) * num_kv_heads + h / G) * kShareCols +
                        (ps.y >> 16) * G + h % G;
  merge_row<BF16, D, true>(a, off, nown, nown + nsh, base, stride, sbase,
                           static_cast<int64_t>(num_kv_heads) * kShareCols);
}

template <bool BF16, int D, int G, bool FP8>
static hipError_t launch_partials_t(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t stream) {
  const int log2b = ilog2(d.block_size);
  dim3 grid(d.num_kv_heads, a.max_partitions, a.balanced ? 1 : a.num_rows);
  if constexpr (UseMfma<BF16, D, G>::value)
    hipLaunchKernelGGL((decode_mfma_kernel<G, FP8>), grid, dim3(64), 0, stream, a, d.num_kv_heads,
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

hipError_t launch_decode_merge(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t stream) {
  if (a.max_partitions <= 1) return hipSuccess;
  const dim3 grid(d.num_heads, a.num_rows);
  if (d.dtype != PA_DTYPE_F32) {  // bf16 output (bf16 and FP8 caches)
    if (d.head_dim == 128)
      hipLaunchKernelGGL((decode_merge_kernel<true, 128>), grid, dim3(64), 0, stream, a, d.num_heads, d.num_kv_heads,
                         d.block_size);
    else
      hipLaunchKernelGGL((decode_merge_kernel<true, 64>), grid, dim3(64), 0, stream, a, d.num_heads, d.num_kv_heads,
                         d.block_size);
  } else {
    if (d.head_dim == 128)
      hipLaunchKernelGGL((decode_merge_kernel<false, 128>), grid, dim3(64), 0, stream, a, d.num_heads, d.num_kv_heads,
                         d.block_size);
    else
      hipLaunchKernelGGL((decode_merge_kernel<false, 64>), grid, dim3(64), 0, stream, a, d.num_heads, d.num_kv_heads,
                         d.block_size);
  }
  return hipGetLastError();
}

}  // namespace pa
