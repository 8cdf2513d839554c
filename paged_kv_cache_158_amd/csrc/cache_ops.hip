// Cache write (slot_mapping scatter), whole-block copy and swap kernels.
//
// Both are pure data movement, bound by HBM bandwidth: every thread moves
// one 16-byte vector of K and one of V with a single global load and store,
// consecutive threads covering consecutive bytes of a token row (or block),
// so each wavefront moves contiguous 1 KiB runs.
#include "common.h"
#include "kernels.h"

namespace pa {

// One thread per 16-byte vector of a token's [num_kv_heads][head_dim] row.
// CSDN "vLLM 0.10.0 flow" page §3.3: the K/V of a token goes to the slot
// slot_mapping names.
__global__ void __launch_bounds__(256)
cache_write_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                   const int32_t* __restrict__ slot_mapping, int64_t num_vecs,
                   int32_t vecs_per_row, int32_t vecs_per_head, int32_t block_mask, int32_t rot,
                   int64_t num_slots, u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= num_vecs) return;
  const int64_t tok = i / vecs_per_row;
  const int32_t col = static_cast<int32_t>(i - tok * vecs_per_row);
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;
  // head h of the token goes to head position kv_head_pos(h, slot % B)
  const int32_t h = col / vecs_per_head;
  const int32_t hp = kv_head_pos(h, static_cast<int32_t>(slot) & block_mask, rot);
  const int64_t dst = slot * vecs_per_row + hp * vecs_per_head + (col - h * vecs_per_head);
  const u32x4 kv = k[i];
  const u32x4 vv = v[i];
  k_cache[dst] = kv;
  v_cache[dst] = vv;
}

// One workgroup per (src, dst) pair; copy-on-write ("vLLM" documentation
// page, section 写时复制): the new block receives the old block's contents.
__global__ void __launch_bounds__(256)
copy_blocks_kernel(u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
                   const int32_t* __restrict__ pairs, int32_t vecs_per_block,
                   int32_t num_blocks) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  const int64_t s0 = static_cast<int64_t>(src) * vecs_per_block;
  const int64_t d0 = static_cast<int64_t>(dst) * vecs_per_block;
  for (int32_t j = threadIdx.x; j < vecs_per_block; j += blockDim.x) {
    const u32x4 kv = k_cache[s0 + j];
    const u32x4 vv = v_cache[s0 + j];
    k_cache[d0 + j] = kv;
    v_cache[d0 + j] = vv;
  }
}

// FP8 caches: one thread per 16-byte cache vector (16 E4M3 codes of one
// head row piece) from 32 bytes of bf16 input.  Code = nearest E4M3 value to
// x / scale[h] in float32 (clamped to +-448 first: the conversion
// instruction turns larger magnitudes into NaN), ties to even.
__global__ void __launch_bounds__(256)
cache_write_fp8_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                       const int32_t* __restrict__ slot_mapping, int64_t num_vecs,
                       int32_t vecs_per_row, int32_t vecs_per_head, int32_t block_mask, int32_t rot,
                       int64_t num_slots, const float* __restrict__ k_scale,
                       const float* __restrict__ v_scale, u32x4* __restrict__ k_cache,
                       u32x4* __restrict__ v_cache) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= num_vecs) return;
  const int64_t tok = i / vecs_per_row;
  const int32_t col = static_cast<int32_t>(i - tok * vecs_per_row);
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;
  const int32_t h = col / vecs_per_head;
  const int32_t hp = kv_head_pos(h, static_cast<int32_t>(slot) & block_mask, rot);
  const int64_t dst = slot * vecs_per_row + hp * vecs_per_head + (col - h * vecs_per_head);
  auto quant = [](const u32x4* src, int64_t at, float s) {
    const uint2 lo = quant_fp8x8(src[2 * at], s), hi = quant_fp8x8(src[2 * at + 1], s);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
  };
  // input vector index: token tok, 16 elements starting at col * 16
  const int64_t at = tok * vecs_per_row + col;
  k_cache[dst] = quant(k, at, k_scale[h]);
  v_cache[dst] = quant(v, at, v_scale[h]);
}

hipError_t launch_cache_write(const void* k, const void* v, const int32_t* slot_mapping,
                              int32_t num_tokens, void* k_cache, void* v_cache,
                              const pa_cache_dims& d, hipStream_t stream) {
  if (d.dtype == PA_DTYPE_FP8_E4M3) {
    const int32_t vecs_per_head = d.head_dim / 16;
    const int32_t vecs_per_row = d.num_kv_heads * vecs_per_head;
    const int64_t num_vecs = static_cast<int64_t>(num_tokens) * vecs_per_row;
    const int64_t num_slots = static_cast<int64_t>(d.num_blocks) * d.block_size;
    const int64_t grid = (num_vecs + 255) / 256;
    hipLaunchKernelGGL(cache_write_fp8_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                       stream, static_cast<const u32x4*>(k), static_cast<const u32x4*>(v),
                       slot_mapping, num_vecs, vecs_per_row, vecs_per_head, d.block_size - 1,
                       layout_rot(d), num_slots, d.k_scale, d.v_scale,
                       static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache));
    return hipGetLastError();
  }
  const int elem = cache_elem_bytes(d);
  const int32_t vecs_per_head = d.head_dim * elem / 16;
  const int32_t vecs_per_row = d.num_kv_heads * vecs_per_head;
  const int64_t num_vecs = static_cast<int64_t>(num_tokens) * vecs_per_row;
  const int64_t num_slots = static_cast<int64_t>(d.num_blocks) * d.block_size;
  const int64_t grid = (num_vecs + 255) / 256;
  hipLaunchKernelGGL(cache_write_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream,
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), slot_mapping,
                     num_vecs, vecs_per_row, vecs_per_head, d.block_size - 1,
                     layout_rot(d), num_slots, static_cast<u32x4*>(k_cache),
                     static_cast<u32x4*>(v_cache));
  return hipGetLastError();
}

// Whole-block moves between two pools (GPU caches and a pool in pinned host
// memory, either way; SourceAIX page §6.2.1, swap out / swap in).  Grid:
// (pieces of a block, pairs); a thread moves kUnroll vectors of K and of V,
// all loads issued before the stores, so each wavefront keeps 2 x kUnroll x
// 1 KiB in flight, which the host link's latency needs.
constexpr int kSwapUnroll = 4;
__global__ void __launch_bounds__(256)
swap_blocks_kernel(const u32x4* __restrict__ src_k, const u32x4* __restrict__ src_v,
                   u32x4* __restrict__ dst_k, u32x4* __restrict__ dst_v,
                   const int32_t* __restrict__ pairs, int32_t vecs_per_block,
                   int32_t src_blocks, int32_t dst_blocks) {
  const int32_t src = pairs[2 * blockIdx.y];
  const int32_t dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const int64_t s0 = static_cast<int64_t>(src) * vecs_per_block;
  const int64_t d0 = static_cast<int64_t>(dst) * vecs_per_block;
  const int32_t j0 = blockIdx.x * (256 * kSwapUnroll) + threadIdx.x;
  u32x4 kv[kSwapUnroll], vv[kSwapUnroll];
#pragma unroll
  for (int u = 0; u < kSwapUnroll; ++u) {
    const int32_t j = j0 + u * 256;
    if (j < vecs_per_block) {
      kv[u] = src_k[s0 + j];
      vv[u] = src_v[s0 + j];
    }
  }
#pragma unroll
  for (int u = 0; u < kSwapUnroll; ++u) {
    const int32_t j = j0 + u * 256;
    if (j < vecs_per_block) {
      dst_k[d0 + j] = kv[u];
      dst_v[d0 + j] = vv[u];
    }
  }
}

hipError_t launch_swap_blocks(const void* src_k, const void* src_v, int32_t src_blocks,
                              void* dst_k, void* dst_v, int32_t dst_blocks,
                              const int32_t* pairs, int32_t num_pairs, const pa_cache_dims& d,
                              hipStream_t stream) {
  const int elem = cache_elem_bytes(d);
  const int32_t vecs_per_block = d.block_size * d.num_kv_heads * d.head_dim * elem / 16;
  const int32_t pieces = (vecs_per_block + 256 * kSwapUnroll - 1) / (256 * kSwapUnroll);
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(pieces, num_pairs), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src_k), static_cast<const u32x4*>(src_v),
                     static_cast<u32x4*>(dst_k), static_cast<u32x4*>(dst_v), pairs,
                     vecs_per_block, src_blocks, dst_blocks);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                              int32_t num_pairs, const pa_cache_dims& d, hipStream_t stream) {
  const int elem = cache_elem_bytes(d);
  const int32_t vecs_per_block = d.block_size * d.num_kv_heads * d.head_dim * elem / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs), dim3(256), 0, stream,
                     static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), pairs,
                     vecs_per_block, d.num_blocks);
  return hipGetLastError();
}

}  // namespace pa
