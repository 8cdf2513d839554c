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
  float* part_ml;          // [num_rows][num_heads][max_partitions][2]
  float* part_o;           // [num_rows][num_heads][max_partitions][head_dim]
  // Row mapping (grid z = work row):
  //   kRowsDecode  row z = sequence z: q/out row z, table row z, context_lens[z]
  //   kRowsVarlenDecode  row z = segment z of a varlen batch, handled only when
  //                it has exactly one query row (q/out row query_start_loc[z],
  //                context seq_lens[z] = context_lens[z]); other segments skip
  //   kRowsVarlenAll  row z = query row z of a varlen batch: its segment s is
  //                found in query_start_loc, context = the causal length
  //                seq_lens[s] - q_len + (z - query_start_loc[s]) + 1
  const int32_t* query_start_loc;
  int32_t mode;
  int32_t num_rows;
};

enum : int32_t { kRowsDecode = 0, kRowsVarlenDecode = 1, kRowsVarlenAll = 2 };

// Partition kernel: final rows for one-partition sequences, partials for the
// rest.  Returns hipErrorInvalidValue for a (dtype, head_dim, group) with no
// kernel.
hipError_t launch_decode_partials(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t stream);
// Log-sum-exp merge of the partials (no-op rows for one-partition sequences).
hipError_t launch_decode_merge(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t stream);
bool decode_supported(const pa_cache_dims& d);

struct VarlenArgs {
  const void* q;                  // [total_q][num_heads][head_dim]
  const int32_t* query_start_loc; // [num_seqs + 1]
  const int32_t* seq_lens;        // [num_seqs]
  int32_t num_seqs;
  int32_t max_query_len;
  int32_t max_seq_len;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  float scale;
  void* out;                      // [total_q][num_heads][head_dim]
};

// MFMA chunked-prefill kernel for the segments with >= 2 query rows (bf16).
bool varlen_prefill_supported(const pa_cache_dims& d);
hipError_t launch_varlen_prefill(const VarlenArgs& a, const pa_cache_dims& d, hipStream_t stream);

}  // namespace pa
