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
  // Balanced split (balanced != 0; rows in mode kRowsDecode or
  // kRowsVarlenDecode, num_rows <= kPlanMaxRows).  Instead of fixed
  // partitions, grid y = max_partitions work slots per KV head, and every
  // wave derives the same plan from the context lengths: with a per-wave cap
  // of t chunks, active row r of c_r chunks gets n_r = max(1, ceil(c_r / t))
  // partitions, partition p covering chunks [p c_r / n_r, (p+1) c_r / n_r),
  // and rows take consecutive slots.  t is the smallest cap whose plan fits
  // plan_share slots (one wave per SIMD), or plan_share2 slots (two per
  // SIMD) when that cap is 2.5x smaller, and at most plan_max_tokens.  The
  // partial of slot y and query head h sits at index y * num_heads + h of
  // part_ml / part_o; the wave of partition 0 stores (first slot, n_r) of
  // its row in plan[2r], plan[2r+1] for the merge.
  int32_t balanced;
  int32_t plan_share;       // slots per KV head for one wave per SIMD
  int32_t plan_share2;      // slots per KV head for two waves per SIMD
  int32_t plan_max_tokens;  // longest partition (block-table staging limit)
  int32_t* plan;            // [num_rows][2]
};

enum : int32_t { kRowsDecode = 0, kRowsVarlenDecode = 1, kRowsVarlenAll = 2 };
constexpr int32_t kPlanMaxRows = 1024;  // rows a balanced plan can cover

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
// Query rows per prefill unit (workgroup) for this head grouping.
int32_t varlen_prefill_rows(const pa_cache_dims& d);
// One launch running the prefill units and then the decode rows (bf16,
// balanced decode split, num_seqs <= kPlanMaxRows); unit_bound >= the
// number of prefill units per KV head.  The merge still follows.
bool varlen_fused_supported(const pa_cache_dims& d);
hipError_t launch_varlen_fused(const VarlenArgs& va, const DecodeArgs& da, const pa_cache_dims& d,
                               int32_t unit_bound, hipStream_t stream);

}  // namespace pa
