// Internal launchers behind the C ABI (pa_api.cpp validates, these launch).
#pragma once

#include <hip/hip_runtime.h>

#include "pa.h"

namespace pa {

hipError_t launch_cache_write(const void* k, const void* v, const int32_t* slot_mapping,
                              int32_t num_tokens, void* k_cache, void* v_cache,
                              const pa_cache_dims& d, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                              int32_t num_pairs, const pa_cache_dims& d, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t max_context_len;
  float scale;
  void* out;
  int32_t partition_size;
  int32_t max_partitions;  // ceil(max_context_len / partition_size)
  float* part_ml;          // [num_seqs][num_heads][max_partitions][2]
  float* part_o;           // [num_seqs][num_heads][max_partitions][head_dim]
};

// Partition kernel: final rows for one-partition sequences, partials for the
// rest.  Returns hipErrorInvalidValue for a (dtype, head_dim, group) with no
// kernel.
hipError_t launch_decode_partials(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t stream);
// Log-sum-exp merge of the partials (no-op rows for one-partition sequences).
hipError_t launch_decode_merge(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t stream);
bool decode_supported(const pa_cache_dims& d);

}  // namespace pa
