// Launchers of the varlen (chunked prefill + decode rows) kernels behind the
// C ABI.  Kept apart from kernels.h, which the decode kernels include.
#pragma once

#include "kernels.h"

namespace pa {

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
  const float* k_scale;           // FP8 caches: [num_kv_heads] (as DecodeArgs)
  const float* v_scale;
  int32_t rot;                    // head-order rotation mask of the caches (layout_rot)
  // Fused launch: the host's bound on the prefill units per KV head (from
  // num_seqs, total_q and max_query_len), which sized its grid and the cut
  // pieces' workspace.  A batch whose units exceed it (an understated
  // max_query_len) is never cut, so no piece writes past the workspace;
  // units and decode rows beyond the grid are then not computed.
  int32_t unit_bound;
#ifdef PA_TIMELINE
  // 4 stamps per workgroup of a varlen launch, at its linear index: start,
  // end, kind << 62 | (prefill: key tiles | query block << 16 | segment <<
  // 32 | KV head << 48; kind 1 prefill, 2 decode), XCC_ID | HW_ID << 32
  unsigned long long* trace;
#endif
};
// varlen records that fit the trace buffer
PA_TL(constexpr int64_t kTraceVarlenWgs = (int64_t{1} << 20) / 4;)

// MFMA chunked-prefill kernel for the segments with >= 2 query rows (bf16
// q and output; bf16 or FP8 caches).
bool varlen_prefill_supported(const pa_cache_dims& d);
hipError_t launch_varlen_prefill(const VarlenArgs& a, const pa_cache_dims& d, hipStream_t stream);
// Query rows per prefill unit (workgroup) for this head grouping.
int32_t varlen_prefill_rows(const pa_cache_dims& d);
// Prefill split of a fused launch: unit_bound >= the prefill units per KV
// head; slots = workgroups per KV head that run on the chip at once when the
// units may be cut into key-range pieces (0: no cut); with slots > 0 the
// workspace holds (unit_bound + slots) * num_kv_heads * varlen_prefill_cols()
// columns of partials: part_ml 2 floats and part_o head_dim floats each.
struct PrefillSplitArgs {
  int32_t unit_bound;
  int32_t slots;
  float* part_o;
  float* part_ml;
};
// Query columns ((row, head) pairs) of one prefill workgroup.
int32_t varlen_prefill_cols();
// One launch running the prefill pieces and then the decode rows (bf16 or
// FP8 caches, balanced decode split, num_seqs <= kPlanMaxRows), then, with
// slots > 0, the merge of the cut units.  The decode merge still follows.
bool varlen_fused_supported(const pa_cache_dims& d);
hipError_t launch_varlen_fused(const VarlenArgs& va, const DecodeArgs& da, const pa_cache_dims& d,
                               const PrefillSplitArgs& ps, hipStream_t stream);

}  // namespace pa
