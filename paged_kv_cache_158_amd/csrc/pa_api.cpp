// C ABI of libpa: argument validation, launch configuration and dispatch to
// the gfx950 kernels.  Everything host-checkable is checked here, before any
// launch; kernels only ever see arguments that passed.
#include <cstdint>
#include <mutex>

#include "kernels.h"
#include "varlen.h"
#include "pa.h"

namespace {

#ifdef PA_TIMELINE
// Timeline buffer of the next launches (decode records first, varlen
// records from kTraceVarlenOffset stamps on); null turns recording off.
void* g_trace = nullptr;
constexpr int64_t kTraceVarlenOffset = int64_t{1} << 20;
#endif


constexpr int kVersion = 200;          // 0.2.0
constexpr int kMaxTableEntries = 1024;  // block-table entries of one fixed partition

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

int check_dims(const pa_cache_dims* d) {
  if (!d) return PA_ERR_INVALID_ARG;
  if (d->num_blocks <= 0 || d->num_heads <= 0 || d->num_kv_heads <= 0) return PA_ERR_INVALID_ARG;
  if (d->num_heads % d->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (d->dtype != PA_DTYPE_F32 && d->dtype != PA_DTYPE_BF16 && d->dtype != PA_DTYPE_FP8_E4M3)
    return PA_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!pow2(d->block_size) || d->block_size < 4 || d->block_size > 256) return PA_ERR_UNSUPPORTED;
  const int64_t slots = static_cast<int64_t>(d->num_blocks) * d->block_size;
  if (slots > INT32_MAX) return PA_ERR_UNSUPPORTED;  // slots are int32
  if (d->layout != PA_LAYOUT_PLAIN && d->layout != PA_LAYOUT_ROTATED) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// FP8 caches are written and read with their per-KV-head scales.
bool scales_ok(const pa_cache_dims* d) {
  return d->dtype != PA_DTYPE_FP8_E4M3 || (d->k_scale != nullptr && d->v_scale != nullptr);
}

// Device memory, or pinned host memory mapped for the GPU (its device
// address equals its host address on this platform); pageable host memory
// (not registered with the runtime) and managed memory are refused.
bool gpu_accessible(const void* p) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of a failed query
    return false;
  }
  if (a.isManaged) return false;
  if (a.type == hipMemoryTypeDevice) return true;
  return a.type == hipMemoryTypeHost && a.devicePointer == p;
}

// Balanced split sizing.  An MI355X runs 256 CUs x 4 SIMDs; the split aims
// at one decode wave per SIMD (1024 waves over all KV heads), each with an
// equal range of the cost line (see pa::DecodeArgs::balanced).
int32_t plan_share(const pa_cache_dims& d) {
  const int32_t share = 1024 / d.num_kv_heads;
  return share < 1 ? 1 : share;
}

constexpr int32_t kChunkCost = pa::kPlanChunkCost;
constexpr int32_t kRowCost = pa::kPlanRowCost;

int32_t chunk_tokens(const pa_cache_dims& d) {
  return pa::decode_chunk_tokens(pa::lane_elem_bytes(d), d.head_dim);
}

// Longest range R (units) whose work list fits the wave's LDS area.  A range
// holding K chunks in n segments spans at least (K - n) Q + (n - 1)(Q + b)
// + 1 units (chunks of one row start Q apart, the first chunk of the next
// row Q + b after the last of the previous), and needs kSegInts n + m K
// ints, m = max(1, chunk / block) table entries per chunk.  Per unit of
// span a segment adds (kSegInts + m) / (Q + b) ints and a further chunk of
// the same segment m / Q, so the list needs at most
// (kSegInts + m) + (R - 1) max((kSegInts + m) / (Q + b), m / Q) ints.
int32_t plan_max_cost(const pa_cache_dims& d) {
  const int64_t ck = chunk_tokens(d);
  const int64_t m = ck > d.block_size ? ck / d.block_size : 1;
  const int64_t x = pa::kDecodeLdsInts - pa::kSegInts - m;
  const int64_t by_seg = x * (kChunkCost + kRowCost) / (pa::kSegInts + m);
  const int64_t by_chunk = x * kChunkCost / m;
  return static_cast<int32_t>(1 + (by_seg < by_chunk ? by_seg : by_chunk));
}

// Waves per KV head (grid y) of a balanced split, or 0 when the rows cannot
// use one: enough for the longest possible line at plan_max_cost units per
// wave, at least plan_share, and no more than there can be chunks.
int64_t plan_slots(const pa_cache_dims& d, int32_t rows, int32_t max_ctx) {
  if (rows <= 0 || rows > pa::kPlanMaxRows) return 0;
  const int64_t cmax = (static_cast<int64_t>(max_ctx) + chunk_tokens(d) - 1) / chunk_tokens(d);
  const int64_t tmax = static_cast<int64_t>(rows) * (kRowCost + kChunkCost * cmax);
  if (tmax >= (int64_t{1} << 30)) return 0;  // the line is measured in int32
  const int64_t rmax = plan_max_cost(d);
  int64_t slots = (tmax + rmax - 1) / rmax;
  if (slots < plan_share(d)) slots = plan_share(d);
  const int64_t most = static_cast<int64_t>(rows) * (cmax > 1 ? cmax : 1);
  if (slots > most) slots = most;
  return slots > 65535 ? 0 : slots;
}

// Workspace layout shared by pa_decode and pa_varlen's decode rows:
// [plan: rows x 2 int32 (balanced only)] [m, l: slots x 2 floats] [o: slots x D floats],
// each region 16-byte aligned; `slots` counts (partial, query head) pairs:
// (waves + rows) x heads for the balanced split (partial index y + row),
// rows x heads x partitions for the fixed one.
struct SplitLayout {
  bool balanced;
  bool share;      // shared prefixes (pa::DecodeArgs::share)
  int32_t P;       // tokens per partition (fixed split)
  int32_t parts;   // grid y: partitions per row (fixed) or work slots (balanced)
  int64_t plan_floats, ml_floats, o_floats;
  int64_t sh_plan_floats, sh_ml_floats, sh_o_floats;  // shared prefixes only
  size_t bytes() const {
    return static_cast<size_t>(
        (plan_floats + ml_floats + o_floats + sh_plan_floats + sh_ml_floats + sh_o_floats) * 4);
  }
};

// Shared prefixes are looked for in balanced plans of 2..64 decode rows
// whose wave is the matrix-core one with room for two or more rows' heads
// (bf16 or FP8 caches, head dim 128, 4 or 8 query heads per KV head), and
// whose block numbers leave the staged entries their mismatch bits.
bool share_possible(const pa_cache_dims& d, int32_t rows) {
  const int32_t G = d.num_heads / d.num_kv_heads;
  return rows >= 2 && rows <= pa::kShareMaxRows && d.head_dim == 128 &&
         (d.dtype == PA_DTYPE_BF16 || d.dtype == PA_DTYPE_FP8_E4M3) && (G == 4 || G == 8) &&
         d.num_blocks < (1 << 27);
}

int64_t round4(int64_t x) { return (x + 3) / 4 * 4; }

SplitLayout split_layout(const pa_cache_dims& d, int32_t rows, int32_t max_ctx, int32_t P,
                         bool allow_share) {
  SplitLayout L{};
  L.P = P;
  if (P == 0) {
    L.balanced = true;
    L.parts = static_cast<int32_t>(plan_slots(d, rows, max_ctx));
    const int64_t slots = (static_cast<int64_t>(L.parts) + rows) * d.num_heads;
    L.plan_floats = round4(static_cast<int64_t>(rows) * 2);
    L.ml_floats = round4(slots * 2);
    L.o_floats = slots * d.head_dim;
    L.share = allow_share && L.parts > 0 && share_possible(d, rows);
    if (L.share) {
      // partial index y + group: waves per KV head + at most rows / 2 groups
      const int64_t cols = (static_cast<int64_t>(L.parts) + rows / 2) * d.num_kv_heads *
                           pa::kShareCols;
      L.sh_plan_floats = round4(static_cast<int64_t>(rows) * 2);
      L.sh_ml_floats = round4(cols * 2);
      L.sh_o_floats = cols * d.head_dim;
    }
    return L;
  }
  const int64_t parts = (static_cast<int64_t>(max_ctx) + P - 1) / P;
  L.parts = static_cast<int32_t>(parts < 1 ? 1 : (parts > 65535 ? 65536 : parts));
  if (parts > 1) {
    const int64_t slots = static_cast<int64_t>(rows) * d.num_heads * parts;
    L.ml_floats = round4(slots * 2);
    L.o_floats = slots * d.head_dim;
  }
  return L;
}

void apply_layout(const SplitLayout& L, const pa_cache_dims& d, void* workspace, pa::DecodeArgs* a) {
  a->partition_size = L.P;
  a->max_partitions = L.parts;
  a->balanced = L.balanced ? 1 : 0;
  PA_TL(a->trace = static_cast<unsigned long long*>(g_trace);)
  a->plan_share = plan_share(d);
  a->plan_max_cost = plan_max_cost(d);
  float* ws = static_cast<float*>(workspace);
  const bool any = L.bytes() > 0 && ws != nullptr;
  a->plan = any && L.balanced ? reinterpret_cast<int32_t*>(ws) : nullptr;
  a->part_ml = any ? ws + L.plan_floats : nullptr;
  a->part_o = any ? ws + L.plan_floats + L.ml_floats : nullptr;
  a->share = any && L.share ? 1 : 0;
  if (a->share) {
    float* sh = ws + L.plan_floats + L.ml_floats + L.o_floats;
    a->plan_sh = reinterpret_cast<int32_t*>(sh);
    a->sh_ml = sh + L.sh_plan_floats;
    a->sh_o = sh + L.sh_plan_floats + L.sh_ml_floats;
  }
}

}  // namespace

extern "C" {

int pa_version(void) { return kVersion; }

#ifdef PA_TIMELINE
// Timeline build only: registers a device buffer of at least 2^21 stamps
// (16 MiB) for the next launches, or turns recording off (null).
void pa_trace_set(void* buffer) { g_trace = buffer; }
#endif

int32_t pa_cache_head_index(int32_t kv_head, int32_t pos_in_block, int32_t num_kv_heads,
                            int32_t layout) {
  if (num_kv_heads <= 0 || kv_head < 0 || kv_head >= num_kv_heads || pos_in_block < 0) return -1;
  if (layout == PA_LAYOUT_PLAIN) return kv_head;
  if (layout != PA_LAYOUT_ROTATED) return -1;
  return pa::kv_head_pos(kv_head, pos_in_block, pa::kv_rot_mask(num_kv_heads));
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument (null/misaligned pointer or bad size)";
    case PA_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, head group or block size";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch failed";
    case PA_ERR_OUT_OF_BLOCKS: return "block pool exhausted";
    case PA_ERR_NO_SEQUENCE: return "unknown or duplicate sequence id";
    default: return "unknown status";
  }
}

int pa_cache_write(const void* k, const void* v, const int32_t* slot_mapping, int32_t num_tokens,
                   void* k_cache, void* v_cache, const pa_cache_dims* dims, hipStream_t stream) {
  if (int st = check_dims(dims)) return st;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_INVALID_ARG;
  if (!scales_ok(dims)) return PA_ERR_INVALID_ARG;
  return from_hip(pa::launch_cache_write(k, v, slot_mapping, num_tokens, k_cache, v_cache, *dims,
                                         stream));
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t num_pairs,
                   const pa_cache_dims* dims, hipStream_t stream) {
  if (int st = check_dims(dims)) return st;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) return PA_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_INVALID_ARG;
  return from_hip(pa::launch_copy_blocks(k_cache, v_cache, block_pairs, num_pairs, *dims, stream));
}

int pa_swap_blocks(const void* src_k, const void* src_v, int32_t src_num_blocks, void* dst_k,
                   void* dst_v, int32_t dst_num_blocks, const int32_t* block_pairs,
                   int32_t num_pairs, const pa_cache_dims* dims, hipStream_t stream) {
  if (int st = check_dims(dims)) return st;
  if (num_pairs < 0 || src_num_blocks <= 0 || dst_num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > 65535) return PA_ERR_UNSUPPORTED;  // grid y
  const void* ptrs[5] = {src_k, src_v, dst_k, dst_v, block_pairs};
  for (const void* p : ptrs) {
    if (!p || !aligned16(p)) return PA_ERR_INVALID_ARG;
    if (!gpu_accessible(p)) return PA_ERR_INVALID_ARG;
  }
  return from_hip(pa::launch_swap_blocks(src_k, src_v, src_num_blocks, dst_k, dst_v,
                                         dst_num_blocks, block_pairs, num_pairs, *dims, stream));
}

int32_t pa_decode_partition_size(const pa_cache_dims* dims, int32_t num_seqs,
                                 int32_t max_context_len, int32_t partition_size) {
  if (check_dims(dims) != PA_OK || num_seqs < 0 || max_context_len < 0 || partition_size < 0)
    return -1;
  int32_t P = partition_size;
  // library choice: the balanced split whenever the rows fit one plan
  if (P == 0 && plan_slots(*dims, num_seqs, max_context_len) > 0) return 0;
  if (P == 0) {
    // Fixed partitions for batches too large for a plan: the largest
    // partition that still gives the grid ~4 (sequence, KV head, partition)
    // waves per CU of an MI355X (256 CUs).
    P = 2048;
    auto waves = [&](int32_t p) {
      return static_cast<int64_t>(num_seqs) * dims->num_kv_heads * ((max_context_len + p - 1) / p);
    };
    while (P > 64 && waves(P) < 1024) P /= 2;
  }
  if (P % 64 != 0) return -1;
  // the partition's block-table entries must fit the LDS staging area
  if (P / dims->block_size + 3 > kMaxTableEntries) return -1;
  return P;
}

size_t pa_decode_workspace_bytes(const pa_cache_dims* dims, int32_t num_seqs,
                                 int32_t max_context_len, int32_t partition_size) {
  const int32_t P = pa_decode_partition_size(dims, num_seqs, max_context_len, partition_size);
  if (P < 0) return 0;
  return split_layout(*dims, num_seqs, max_context_len, P, true).bytes();
}

}  // extern "C"

namespace {

// Validates the decode arguments shared by pa_decode / pa_decode_partials /
// pa_decode_merge and fills the kernel argument block.  `need_inputs` is
// false for the merge phase, which reads only lengths, workspace and out.
int build_decode_args(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                      float scale, void* out, const pa_cache_dims* dims, int32_t partition_size,
                      void* workspace, size_t workspace_bytes, bool need_inputs,
                      pa::DecodeArgs* a) {
  if (int st = check_dims(dims)) return st;
  if (!pa::decode_supported(*dims)) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs > 65535) return PA_ERR_UNSUPPORTED;  // grid z
  if (num_seqs > 0) {
    if (!context_lens || !out || !aligned16(out)) return PA_ERR_INVALID_ARG;
    if (need_inputs && (!q || !k_cache || !v_cache || !block_tables || !aligned16(q) ||
                        !aligned16(k_cache) || !aligned16(v_cache) || !scales_ok(dims)))
      return PA_ERR_INVALID_ARG;
  }
  const int32_t P = pa_decode_partition_size(dims, num_seqs, max_context_len, partition_size);
  if (P < 0) return PA_ERR_INVALID_ARG;
  const SplitLayout L = split_layout(*dims, num_seqs, max_context_len, P, true);
  if (L.parts > 65535) return PA_ERR_UNSUPPORTED;  // grid y
  const size_t need = L.bytes();
  if (num_seqs > 0 && need > 0 &&
      (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return PA_ERR_WORKSPACE;
  *a = pa::DecodeArgs{};
  a->q = q;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->block_tables = block_tables;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->context_lens = context_lens;
  a->num_seqs = num_seqs;
  a->max_context_len = max_context_len;
  a->scale = scale;
  a->out = out;
  a->k_scale = dims->k_scale;
  a->v_scale = dims->v_scale;
  a->rot = pa::layout_rot(*dims);
  a->query_start_loc = nullptr;
  a->mode = pa::kRowsDecode;
  a->num_rows = num_seqs;
  apply_layout(L, *dims, workspace, a);
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode_partials(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                       float scale, void* out, const pa_cache_dims* dims, int32_t partition_size,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pa::DecodeArgs a;
  if (int st = build_decode_args(q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                 context_lens, num_seqs, max_context_len, scale, out, dims,
                                 partition_size, workspace, workspace_bytes, true, &a))
    return st;
  if (num_seqs == 0) return PA_OK;
  return from_hip(pa::launch_decode_partials(a, *dims, stream));
}

int pa_decode_merge(const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                    int32_t max_blocks_per_seq, void* out, const pa_cache_dims* dims,
                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  pa::DecodeArgs a;
  if (int st = build_decode_args(nullptr, nullptr, nullptr, nullptr, max_blocks_per_seq,
                                 context_lens, num_seqs, max_context_len, 1.0f, out, dims,
                                 partition_size, workspace, workspace_bytes, false, &a))
    return st;
  if (num_seqs == 0) return PA_OK;
  return from_hip(pa::launch_decode_merge(a, *dims, stream));
}

int pa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
              int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
              int32_t max_context_len, float scale, void* out, const pa_cache_dims* dims,
              int32_t partition_size, void* workspace, size_t workspace_bytes,
              hipStream_t stream) {
  pa::DecodeArgs a;
  if (int st = build_decode_args(q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                 context_lens, num_seqs, max_context_len, scale, out, dims,
                                 partition_size, workspace, workspace_bytes, true, &a))
    return st;
  if (num_seqs == 0) return PA_OK;
  if (int st = from_hip(pa::launch_decode_partials(a, *dims, stream))) return st;
  return from_hip(pa::launch_decode_merge(a, *dims, stream));
}

}  // extern "C"

// Scratch of pa_decode_noalloc: one fixed array in every device's copy of
// the code object, allocated by the runtime when the library's code is
// loaded on that device and held until the process ends.  Host code never
// uses this name as an address (on the host it is only a stand-in for the
// symbol); it uses the device address looked up once per device below.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device, looked up on the
// first call made with that device current.
int current_device_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    if (g_scratch_err[dev] != hipSuccess) (void)hipGetLastError();
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return PA_ERR_HIP;
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                      float scale, void* out, const pa_cache_dims* dims, int32_t partition_size,
                      hipStream_t stream) {
  if (int st = check_dims(dims)) return st;
  if (num_seqs < 0 || max_context_len < 0 || partition_size < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (pa_decode_partition_size(dims, num_seqs, max_context_len, partition_size) < 0)
    return PA_ERR_INVALID_ARG;
  const size_t need = pa_decode_workspace_bytes(dims, num_seqs, max_context_len, partition_size);
  if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0)
    if (int st = current_device_scratch(&ws)) return st;
  return pa_decode(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                   max_context_len, scale, out, dims, partition_size, ws, need, stream);
}

}  // extern "C"

namespace {

int decode_append_impl(const void* q, const void* k, const void* v, const int32_t* slot_mapping,
                       void* k_cache, void* v_cache, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                       int32_t max_context_len, float scale, void* out, const pa_cache_dims* dims,
                       int32_t partition_size, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, bool merge) {
  pa::DecodeArgs a;
  if (int st = build_decode_args(q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                 context_lens, num_seqs, max_context_len, scale, out, dims,
                                 partition_size, workspace, workspace_bytes, true, &a))
    return st;
  if (num_seqs == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !aligned16(k) || !aligned16(v)) return PA_ERR_INVALID_ARG;
  a.new_k = k;
  a.new_v = v;
  a.new_slots = slot_mapping;
  if (int st = from_hip(pa::launch_decode_partials(a, *dims, stream))) return st;
  return merge ? from_hip(pa::launch_decode_merge(a, *dims, stream)) : PA_OK;
}

}  // namespace

extern "C" {

int pa_decode_append(const void* q, const void* k, const void* v, const int32_t* slot_mapping,
                     void* k_cache, void* v_cache, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                     int32_t max_context_len, float scale, void* out, const pa_cache_dims* dims,
                     int32_t partition_size, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  return decode_append_impl(q, k, v, slot_mapping, k_cache, v_cache, block_tables,
                            max_blocks_per_seq, context_lens, num_seqs, max_context_len, scale,
                            out, dims, partition_size, workspace, workspace_bytes, stream, true);
}

int pa_decode_append_partials(const void* q, const void* k, const void* v,
                              const int32_t* slot_mapping, void* k_cache, void* v_cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_context_len, float scale, void* out,
                              const pa_cache_dims* dims, int32_t partition_size, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  return decode_append_impl(q, k, v, slot_mapping, k_cache, v_cache, block_tables,
                            max_blocks_per_seq, context_lens, num_seqs, max_context_len, scale,
                            out, dims, partition_size, workspace, workspace_bytes, stream, false);
}

}  // extern "C"

namespace {

// Varlen decode rows use the decode kernels in one of two row modes:
// segments of one row (bf16 path, split-K over max_seq_len), or every query
// row with its causal length (fp32 path, one partition per row).
bool varlen_uses_prefill(const pa_cache_dims& d) { return pa::varlen_prefill_supported(d); }

int32_t varlen_row_partition(const pa_cache_dims* dims, int32_t num_seqs, int32_t max_seq_len) {
  if (varlen_uses_prefill(*dims)) return pa_decode_partition_size(dims, num_seqs, max_seq_len, 0);
  const int32_t P = (max_seq_len + 63) / 64 * 64;
  return P < 64 ? 64 : P;
}

// Upper bound on the prefill units per KV head of a varlen batch: a segment
// of q rows has ceil(q / ROWS) units, and there are at most
// min(num_seqs, total_q / 2) segments of >= 2 rows.
int64_t prefill_unit_bound(const pa_cache_dims& d, int32_t num_seqs, int32_t total_q,
                           int32_t max_query_len) {
  const int64_t R = pa::varlen_prefill_rows(d);
  const int64_t by_len = static_cast<int64_t>(num_seqs) * ((max_query_len + R - 1) / R);
  const int64_t by_sum = (total_q + R - 1) / R + (num_seqs < total_q / 2 ? num_seqs : total_q / 2);
  return by_len < by_sum ? by_len : by_sum;
}

// Workgroup slots per KV head that the fused launch may fill with pieces of
// cut prefill units: two per CU of an MI355X (256 CUs), when even the most
// units the batch can have fill at most half of them (so a batch of many
// units never pays for a cut or a merge); else 0.  A constant rather than
// the current device's count, so that the workspace size and the cut plan
// depend on the arguments alone (a device with fewer CUs runs the pieces
// in more than one round).
constexpr int64_t kCutCUs = 256;
int32_t prefill_cut_slots(const pa_cache_dims& d, int64_t unit_bound) {
  const int64_t slots = 2 * kCutCUs / d.num_kv_heads;
  return 2 * unit_bound <= slots ? static_cast<int32_t>(slots) : 0;
}

bool varlen_fused_path(const pa_cache_dims& d, int32_t num_seqs, int32_t max_query_len,
                       const SplitLayout& L) {
  return max_query_len >= 2 && L.balanced && pa::varlen_fused_supported(d) &&
         num_seqs <= pa::kPlanMaxRows;
}

// Bytes of the cut units' partials (after the decode layout).
size_t prefill_cut_bytes(const pa_cache_dims& d, int64_t unit_bound, int32_t slots) {
  if (slots <= 0) return 0;
  const int64_t cols = (unit_bound + slots) * d.num_kv_heads * pa::varlen_prefill_cols();
  return static_cast<size_t>(round4(cols * 2) + cols * d.head_dim) * 4;
}

}  // namespace

extern "C" {

size_t pa_varlen_workspace_bytes(const pa_cache_dims* dims, int32_t num_seqs, int32_t total_q,
                                 int32_t max_query_len, int32_t max_seq_len) {
  if (check_dims(dims) != PA_OK || num_seqs < 0 || total_q < 0 || max_query_len < 0 ||
      max_seq_len < 0)
    return 0;
  if (!varlen_uses_prefill(*dims)) return 0;  // one partition per row, no partials
  const int32_t P = varlen_row_partition(dims, num_seqs, max_seq_len);
  if (P < 0) return 0;
  // the decode rows' layout, without shared prefixes (not used by varlen)
  const SplitLayout L = split_layout(*dims, num_seqs, max_seq_len, P, false);
  const size_t decode = L.bytes();
  if (!varlen_fused_path(*dims, num_seqs, max_query_len, L)) return decode;
  const int64_t bound = prefill_unit_bound(*dims, num_seqs, total_q, max_query_len);
  const size_t cut = prefill_cut_bytes(*dims, bound, prefill_cut_slots(*dims, bound));
  return cut == 0 ? decode : round4(static_cast<int64_t>(decode / 4)) * 4 + cut;
}

int pa_varlen(const void* q, const int32_t* query_start_loc, const int32_t* seq_lens,
              int32_t num_seqs, int32_t total_q, int32_t max_query_len, int32_t max_seq_len,
              const void* k_cache, const void* v_cache, const int32_t* block_tables,
              int32_t max_blocks_per_seq, float scale, void* out, const pa_cache_dims* dims,
              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (int st = check_dims(dims)) return st;
  if (num_seqs < 0 || total_q < 0 || max_query_len < 0 || max_seq_len < 0 ||
      max_blocks_per_seq < 0)
    return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_q == 0) return PA_OK;
  if (num_seqs > 65535 || total_q > 65535) return PA_ERR_UNSUPPORTED;  // grid limits
  if (!q || !query_start_loc || !seq_lens || !k_cache || !v_cache || !block_tables || !out)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return PA_ERR_INVALID_ARG;
  if (!scales_ok(dims)) return PA_ERR_INVALID_ARG;
  const bool prefill = varlen_uses_prefill(*dims);
  // the prefill kernels address a cache block's bytes with 32-bit offsets
  if (prefill && static_cast<int64_t>(dims->block_size) * dims->num_kv_heads * dims->head_dim *
                         pa::cache_elem_bytes(*dims) > INT64_C(0xFFFFFFFF))
    return PA_ERR_UNSUPPORTED;
  // one-row segments always run the decode kernels (checked before any
  // launch, whether or not the batch has such rows)
  if (!pa::decode_supported(*dims)) return PA_ERR_UNSUPPORTED;
  const int32_t rows = prefill ? num_seqs : total_q;
  const int32_t P = varlen_row_partition(dims, num_seqs, max_seq_len);
  if (P < 0 || P / dims->block_size + 3 > kMaxTableEntries) return PA_ERR_UNSUPPORTED;
  const SplitLayout L = split_layout(*dims, prefill ? num_seqs : total_q, max_seq_len, P, false);
  if (L.parts > 65535) return PA_ERR_UNSUPPORTED;
  const size_t need = pa_varlen_workspace_bytes(dims, num_seqs, total_q, max_query_len,
                                                max_seq_len);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return PA_ERR_WORKSPACE;

  pa::VarlenArgs v{};
  PA_TL(v.trace = g_trace ? static_cast<unsigned long long*>(g_trace) + kTraceVarlenOffset : nullptr;)
  v.q = q;
  v.query_start_loc = query_start_loc;
  v.seq_lens = seq_lens;
  v.num_seqs = num_seqs;
  v.max_query_len = max_query_len;
  v.max_seq_len = max_seq_len;
  v.k_cache = k_cache;
  v.v_cache = v_cache;
  v.block_tables = block_tables;
  v.max_blocks_per_seq = max_blocks_per_seq;
  v.scale = scale;
  v.out = out;
  v.k_scale = dims->k_scale;
  v.v_scale = dims->v_scale;
  v.rot = pa::layout_rot(*dims);
  pa::DecodeArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.max_context_len = max_seq_len;
  a.scale = scale;
  a.out = out;
  a.k_scale = dims->k_scale;
  a.v_scale = dims->v_scale;
  a.rot = v.rot;
  apply_layout(L, *dims, workspace, &a);
  a.query_start_loc = query_start_loc;
  a.mode = prefill ? pa::kRowsVarlenDecode : pa::kRowsVarlenAll;
  a.num_rows = rows;
  if (prefill && varlen_fused_path(*dims, num_seqs, max_query_len, L)) {
    // prefill pieces and decode rows in one launch (then the merge of cut
    // prefill units); the cut units' partials follow the decode layout
    pa::PrefillSplitArgs ps{};
    const int64_t bound = prefill_unit_bound(*dims, num_seqs, total_q, max_query_len);
    ps.unit_bound = static_cast<int32_t>(bound);
    v.unit_bound = ps.unit_bound;
    ps.slots = prefill_cut_slots(*dims, bound);
    if (ps.slots > 0) {
      const int64_t cols = (bound + ps.slots) * dims->num_kv_heads * pa::varlen_prefill_cols();
      float* base = static_cast<float*>(workspace) + round4(static_cast<int64_t>(L.bytes() / 4));
      ps.part_ml = base;
      ps.part_o = base + round4(cols * 2);
    }
    if (int st = from_hip(pa::launch_varlen_fused(v, a, *dims, ps, stream))) return st;
  } else {
    if (prefill && max_query_len >= 2)
      if (int st = from_hip(pa::launch_varlen_prefill(v, *dims, stream))) return st;
    if (int st = from_hip(pa::launch_decode_partials(a, *dims, stream))) return st;
  }
  if (need == 0) return PA_OK;
  return from_hip(pa::launch_decode_merge(a, *dims, stream));
}

}  // extern "C"
