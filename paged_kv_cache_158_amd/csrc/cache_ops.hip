// Cache write (slot_mapping scatter) and whole-block copy kernels.
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

hipError_t launch_cache_write(const void* k, const void* v, const int32_t* slot_mapping,
                              int32_t num_tokens, void* k_cache, void* v_cache,
                              const pa_cache_dims& d, hipStream_t stream) {
  const int elem = d.dtype == PA_DTYPE_BF16 ? 2 : 4;
  const int32_t vecs_per_head = d.head_dim * elem / 16;
  const int32_t vecs_per_row = d.num_kv_heads * vecs_per_head;
  const int64_t num_vecs = static_cast<int64_t>(num_tokens) * vecs_per_row;
  const int64_t num_slots = static_cast<int64_t>(d.num_blocks) * d.block_size;
  const int64_t grid = (num_vecs + 255) / 256;
  hipLaunchKernelGGL(cache_write_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream,
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), slot_mapping,
                     num_vecs, vecs_per_row, vecs_per_head, d.block_size - 1,
                     kv_rot_mask(d.num_kv_heads), num_slots, static_cast<u32x4*>(k_cache),
                     static_cast<u32x4*>(v_cache));
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                              int32_t num_pairs, const pa_cache_dims& d, hipStream_t stream) {
  const int elem = d.dtype == PA_DTYPE_BF16 ? 2 : 4;
  const int32_t vecs_per_block = d.block_size * d.num_kv_heads * d.head_dim * elem / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs), dim3(256), 0, stream,
                     static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), pairs,
                     vecs_per_block, d.num_blocks);
  return hipGetLastError();
}

}  // namespace pa
