// Internal launchers behind the C ABI (pa_api.cpp validates, these launch).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"
#include "pa.h"

// Timeline build (libpa_timeline.so, compiled with PA_TIMELINE): the decode
// and varlen kernels write s_memrealtime stamps (a 100 MHz clock shared by
// the whole device) into a buffer the host registers with pa_trace_set.
// PA_TL(...) expands to its argument in that build and to nothing in the
// product build, which compiles none of it.
#ifdef PA_TIMELINE
#define PA_TL(...) __VA_ARGS__
#else
#define PA_TL(...)
#endif

namespace pa {

// Bytes of one cache element, and of one element of the decode kernels'
// lane geometry (an FP8 lane covers the same head dims as a bf16 one).
inline int cache_elem_bytes(const pa_cache_dims& d) {
  return d.dtype == PA_DTYPE_F32 ? 4 : (d.dtype == PA_DTYPE_BF16 ? 2 : 1);
}
inline int lane_elem_bytes(const pa_cache_dims& d) { return d.dtype == PA_DTYPE_F32 ? 4 : 2; }
// Rotation mask of the caches' head order (kv_head_pos): 0 for the plain
// layout.
inline int32_t layout_rot(const pa_cache_dims& d) {
  return d.layout == PA_LAYOUT_ROTATED ? kv_rot_mask(d.num_kv_heads) : 0;
}

hipError_t launch_cache_write(const void* k, const void* v, const int32_t* slot_mapping,
                              int32_t num_tokens, void* k_cache, void* v_cache,
                              const pa_cache_dims& d, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                              int32_t num_pairs, const pa_cache_dims& d, hipStream_t stream);

hipError_t launch_swap_blocks(const void* src_k, const void* src_v, int32_t src_blocks,
                              void* dst_k, void* dst_v, int32_t dst_blocks,
                              const int32_t* pairs, int32_t num_pairs, const pa_cache_dims& d,
                              hipStream_t stream);

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
  const float* k_scale;  // FP8 caches: [num_kv_heads] (code c of head h is c * scale[h])
  const float* v_scale;
  int32_t rot;             // head-order rotation mask of the caches (layout_rot)
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
  // kRowsVarlenDecode, num_rows <= kPlanMaxRows).  Per KV head, the active
  // rows are laid end to end on a line of cost units: row r takes
  // kPlanRowCost units (the work of switching to a row) followed by
  // kPlanChunkCost units per chunk of its context.  The line (length T) is
  // cut into W = clamp(ceil(T / plan_max_cost), plan_share, max_partitions)
  // equal ranges, range y = [floor(y T / W), floor((y+1) T / W)), and wave y
  // processes every chunk whose first unit lies in its range, row after row
  // (a wave's piece of one row is a segment).  So every wave gets the same
  // work up to one chunk, whatever the lengths.  The partial of wave y's
  // segment of row r and query head h sits at index (y + r) * num_heads + h
  // of part_ml / part_o (y + r grows along the line, so indices never
  // collide); the wave whose range holds row r's first unit stores (first
  // index, number of segments) of the row in plan[2r], plan[2r+1] for the
  // merge (0 segments: empty context, zero output written directly).
  int32_t balanced;
  int32_t plan_share;       // waves per KV head that fill the chip once
  int32_t plan_max_cost;    // longest range (bound by the LDS staging area)
  int32_t* plan;            // [num_rows][2]
  // Fused append (pa_decode_append; rows in mode kRowsDecode): when
  // new_slots is not null, row s's new token, input row s of new_k / new_v
  // ([num_rows][num_kv_heads][head_dim], the q dtype), is stored into the
  // caches at slot new_slots[s] (skipped when out of range, as a cache write
  // would) and, when stored, attended as position ctx - 1 from registers;
  // k_cache / v_cache are written through.
  const void* new_k;
  const void* new_v;
  const int32_t* new_slots;
  // Shared prefixes (share != 0: balanced split, rows in mode kRowsDecode,
  // num_rows <= 64, a matrix-core wave with room for two or more rows'
  // heads).  Consecutive rows that start on the same physical block form
  // groups of up to 16 / G rows; the leading tokens the plan finds common to
  // a group's block tables (a chunk multiple, checked block by block while
  // the tables are staged) are attended once for all of the group's query
  // heads, as a shared item placed on the line before the first row's own
  // item; each row's own item covers the rest of its context.  The partial
  // of wave y's segment of group k sits at index y + k of sh_ml / sh_o, 16
  // query columns per KV head (column m G + h: row m of the group, head h);
  // plan_sh[2r], plan_sh[2r+1] hold (first index, segments | member m << 16)
  // of row r's shared partials (0 segments: row r is not in a group).
  int32_t share;
  int32_t* plan_sh;  // [num_rows][2]
  float* sh_ml;      // [waves + num_rows / 2][num_kv_heads][16][2]
  float* sh_o;       // [waves + num_rows / 2][num_kv_heads][16][head_dim]
#ifdef PA_TIMELINE
  // 10 stamps per decode wave of a balanced split, at index
  // y * num_kv_heads + g: start, plan done, tables staged, end, XCC_ID |
  // HW_ID << 32, segments | chunks << 32, and four plan phases (plain split:
  // lengths in registers, line length, range, segment list; shared
  // prefixes: lengths and first entries, probes, groups, range)
  unsigned long long* trace;
#endif
};
// decode records that fit the trace buffer
PA_TL(constexpr int64_t kTraceDecodeWaves = (int64_t{1} << 20) / 10;)

enum : int32_t { kRowsDecode = 0, kRowsVarlenDecode = 1, kRowsVarlenAll = 2 };
// Cost units of the balanced split's line: a chunk is 8 units and a row
// switch 32.  A wave drains its load ring at the end of a segment and
// refills it for the next; per-wave timelines put that at about three
// chunks' worth of streaming time, and a sweep of the switch cost over
// 16..48 units is fastest at 32 on the short-context batches (lengths
// 128..2048) and flat on long contexts.  Powers of two, so the plan's
// divisions are shifts.
constexpr int32_t kPlanChunkCost = 8;
constexpr int32_t kPlanRowCost = 32;
constexpr int32_t kPlanMaxRows = 1024;  // rows a balanced plan can cover
// LDS of one decode wave, in int32: its segment descriptors (kSegInts each)
// followed by the block-table entries of all its segments.
constexpr int32_t kDecodeLdsInts = 2048;
constexpr int32_t kSegInts = 8;
constexpr int32_t kShareMaxRows = 64;  // rows a plan with shared prefixes can cover
constexpr int32_t kShareCols = 16;     // query columns of a shared segment
// Tokens per chunk of the decode loop: a token row of head_dim elements is
// read with one 16-byte load per lane, 64 lanes read 64 / lanes-per-row
// rows at once, and every lane row takes 4 consecutive tokens.
constexpr int32_t decode_chunk_tokens(int32_t elem_bytes, int32_t head_dim) {
  return 4 * 64 / (head_dim * elem_bytes / 16);
}

// Partition kernel: final rows for one-partition sequences, partials for the
// rest.  Returns hipErrorInvalidValue for a (dtype, head_dim, group) with no
// kernel.
hipError_t launch_decode_partials(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t stream);
// Log-sum-exp merge of the partials (no-op rows for one-partition sequences).
hipError_t launch_decode_merge(const DecodeArgs& a, const pa_cache_dims& d, hipStream_t stream);
bool decode_supported(const pa_cache_dims& d);

}  // namespace pa
