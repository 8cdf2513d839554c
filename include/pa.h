/*
 * pa.h — C ABI of libpa, a paged KV-cache attention library for AMD Instinct
 * MI355X (gfx950).
 *
 * The operations follow the PagedAttention description in the pages this
 * library is built from:
 *   - The KV cache of a layer is one tensor cut into fixed-size blocks of
 *     `block_size` token slots; each request reaches its tokens through a
 *     block table mapping logical block i to a physical block number
 *     ("vLLM" documentation page, section PagedAttention; SourceAIX vLLM
 *     code-reading page, section 5.1.1).
 *   - Each new token's K/V is written into the slot the model runner
 *     computed for it (slot_mapping), and attention finds the data through
 *     the same block/slot structure (CSDN "vLLM 0.10.0 flow" page, sections
 *     3.3 and 3.5: block table, slot_mapping and query_start_loc metadata).
 *
 * Conventions shared by every entry point:
 *   - Cache layout: k_cache and v_cache are separate tensors
 *     [num_blocks][block_size][num_kv_heads][head_dim], contiguous, in the
 *     element type `dtype`.  A slot is one row of the
 *     [num_blocks*block_size][num_kv_heads][head_dim] view:
 *     slot = physical_block * block_size + position % block_size.  The
 *     order of the KV heads inside a slot is pa_cache_dims.layout (see
 *     pa_layout): the plain order by default, or a rotation by the in-block
 *     position; pa_cache_head_index() maps a KV head to its index in either.
 *     Whole-block copies keep the layout.
 *   - Query head h reads KV head h / (num_heads / num_kv_heads) (GQA).
 *   - Pointers named in the argument lists are DEVICE pointers unless the
 *     comment says host.  Device buffers are owned by the caller; the
 *     attention entry points allocate nothing and keep no state between
 *     calls.  Tensors must be contiguous and 16-byte aligned.
 *   - Every GPU call is enqueued on `stream` and returns without waiting.
 *   - Errors: a negative pa_status is returned before anything is launched
 *     when an argument is invalid or unsupported; PA_ERR_HIP when a launch
 *     fails.  Nothing aborts or throws across this boundary.
 *   - Device-side contents (slot values, block-table entries, lengths) are
 *     trusted for speed, but kernels clamp every block number they
 *     dereference into [0, num_blocks) and every length into the stated
 *     maxima, so bad metadata gives wrong numbers, never an access outside
 *     the buffers.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,   /* null / misaligned pointer, bad size */
  PA_ERR_UNSUPPORTED = -2,   /* dtype, head_dim, group or block size not built */
  PA_ERR_WORKSPACE = -3,     /* workspace missing or too small */
  PA_ERR_HIP = -4,           /* a HIP launch failed */
  PA_ERR_OUT_OF_BLOCKS = -5, /* block manager: the pool has too few free blocks */
  PA_ERR_NO_SEQUENCE = -6,   /* block manager: unknown or duplicate sequence id */
} pa_status;

typedef enum pa_dtype {
  PA_DTYPE_F32 = 0,
  PA_DTYPE_BF16 = 1,
  /* Caches of 8-bit E4M3 codes (OCP 8-bit floating point, E4M3: bias 7,
   * largest magnitude 448, no infinities) with one float scale per KV head:
   * a code c of KV head h stands for c * scale[h].  q, the new tokens' k
   * and v, and out are bf16.  pa_cache_write stores the code nearest to
   * x / scale[h] (float32 division, clamped to +-448, ties to even).  This
   * halves the bytes decode reads; the pages name 8-bit floats only for
   * weights, so it is an extension. */
  PA_DTYPE_FP8_E4M3 = 2,
} pa_dtype;

/* Order of the KV heads inside a slot (the pages fix none: they only cut
 * the per-layer cache tensor into blocks of token slots). */
typedef enum pa_layout {
  /* KV head h of every slot at head index h: the plain
   * [num_blocks][block_size][num_kv_heads][head_dim] tensor.  The default
   * (a zero-initialised pa_cache_dims). */
  PA_LAYOUT_PLAIN = 0,
  /* Inside the slot of in-block position p = slot % block_size, KV head h
   * at head index (h + p) % num_kv_heads when num_kv_heads is a power of
   * two (at h otherwise).  One head's reads then cover every head offset of
   * the slot rows instead of always the same one, which spreads them over
   * the HBM address interleave (decode 2-3% faster on MI355X).  Only code
   * that maps heads with pa_cache_head_index() may read such caches. */
  PA_LAYOUT_ROTATED = 1,
} pa_layout;

/* Shape and element type of the paged cache and of the attention heads. */
typedef struct pa_cache_dims {
  int32_t num_blocks;    /* physical blocks in the pool (>= 1) */
  int32_t block_size;    /* token slots per block: power of two, 4..256 */
  int32_t num_heads;     /* query heads H (multiple of num_kv_heads) */
  int32_t num_kv_heads;  /* KV heads H_kv */
  int32_t head_dim;      /* D: 64 or 128 */
  int32_t dtype;         /* pa_dtype of q, k, v, caches and out (FP8: of the caches) */
  const float* k_scale;  /* FP8_E4M3 only: device [num_kv_heads] K scales (else unused) */
  const float* v_scale;  /* FP8_E4M3 only: device [num_kv_heads] V scales (else unused) */
  int32_t layout;        /* pa_layout of both caches (0: plain) */
} pa_cache_dims;

/* Head index, inside the slot of in-block position pos_in_block, that KV
 * head kv_head occupies under `layout`; -1 for arguments out of range
 * (kv_head outside [0, num_kv_heads), pos_in_block < 0, unknown layout).
 * Host function, no GPU. */
int32_t pa_cache_head_index(int32_t kv_head, int32_t pos_in_block, int32_t num_kv_heads,
                            int32_t layout);

/* Library version, major*10000 + minor*100 + patch. */
int pa_version(void);

/* Static, human-readable text for a pa_status value. */
const char* pa_status_string(int status);

/* ------------------------------------------------------------------------
 * pa_cache_write — scatter new tokens' K/V into their slots.
 * CSDN "vLLM 0.10.0 flow" page §3.3 (steps 4-5) and §4 (step 4): the model
 * runner computes slot_mapping for the batch's new tokens and the K/V of
 * each is stored in that slot.
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim] new rows
 *   slot_mapping  [num_tokens] int32; a negative slot skips that token
 *                 (padding); a slot >= num_blocks*block_size is skipped too
 *   k_cache, v_cache  the caches, written in place
 * Exact element copies (FP8_E4M3 caches: the codes of the bf16 rows, see
 * pa_dtype); no other slot changes.  num_tokens == 0 is a no-op.
 * Two tokens with the same slot in one call race (one of them wins).
 * ---------------------------------------------------------------------- */
int pa_cache_write(const void* k, const void* v, const int32_t* slot_mapping,
                   int32_t num_tokens, void* k_cache, void* v_cache,
                   const pa_cache_dims* dims, hipStream_t stream);

/* ------------------------------------------------------------------------
 * pa_copy_blocks — whole-block copies for copy-on-write.
 * "vLLM" documentation page, section 写时复制 (copy-on-write) and SourceAIX
 * page §5.2.1: a request about to write into a block that other requests
 * still share gets a new block holding a copy of the old block's contents.
 *
 *   block_pairs  [num_pairs][2] int32 (src, dst) physical block numbers;
 *                pairs with an out-of-range number are skipped
 * Copies all block_size slots of every KV head, K and V.  Destinations must
 * be distinct and must not be the source of another pair in the same call.
 * ---------------------------------------------------------------------- */
int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs,
                   int32_t num_pairs, const pa_cache_dims* dims, hipStream_t stream);

/* ------------------------------------------------------------------------
 * pa_swap_blocks — whole-block moves between two pools, e.g. the GPU caches
 * and a pool in pinned host memory.  SourceAIX page §6.2.1 (a preempted
 * sequence group with several sequences has its KV blocks swapped out from
 * the GPU to CPU memory, and swapped back in when the GPU has room again)
 * and the dn008 overview §3.5 / §4.3 (the scheduler's swap phase moves the
 * blocks of swapped requests between CPU and GPU memory).
 *
 *   src_k, src_v  source pool [src_num_blocks][block_size][num_kv_heads][head_dim]
 *   dst_k, dst_v  destination pool [dst_num_blocks][...] of the same dims
 *   block_pairs   [num_pairs][2] int32 (src block, dst block); pairs with
 *                 an out-of-range number are skipped
 * Each pool, and block_pairs, is device memory or pinned host memory
 * (hipHostMalloc, or torch's pin_memory); the kernel reads and writes
 * pinned host memory directly over the host link.  Pageable host memory is
 * rejected with PA_ERR_INVALID_ARG before any launch.  dims gives
 * block_size, heads, head_dim and dtype (its num_blocks is not used).
 * Exact copies of all slots of every KV head, K and V; the in-block layout
 * is kept, so blocks can move between pools of any size.  The two pools
 * must not overlap (pa_copy_blocks copies within one pool) and destinations
 * must be distinct.  Enqueued on `stream`; a host pool is complete only
 * after the stream is synchronised.
 * ---------------------------------------------------------------------- */
int pa_swap_blocks(const void* src_k, const void* src_v, int32_t src_num_blocks,
                   void* dst_k, void* dst_v, int32_t dst_num_blocks,
                   const int32_t* block_pairs, int32_t num_pairs,
                   const pa_cache_dims* dims, hipStream_t stream);

/* ------------------------------------------------------------------------
 * pa_decode — one query row per sequence attending over its paged context.
 * SourceAIX page §5.1.1, decode step: attention reads the request's logical
 * blocks as one contiguous sequence while the data comes from the physical
 * blocks named by the block table.  out[s][h] = softmax_t(scale * q[s][h] .
 * K_s[t][h/G]) weighted sum of V_s[t][h/G] over t < context_lens[s].
 *
 *   q             [num_seqs][num_heads][head_dim]
 *   block_tables  [num_seqs][max_blocks_per_seq] int32 physical block numbers;
 *                 entries at index >= ceil(context_len/block_size) are ignored
 *   context_lens  [num_seqs] int32 tokens to attend (<= max_context_len and
 *                 <= max_blocks_per_seq*block_size); 0 gives a zero row
 *   out           [num_seqs][num_heads][head_dim]
 *   partition_size  tokens per split-K partition: a multiple of 64, or 0
 *                 for the library's choice.  For up to 1024 rows that is
 *                 a balanced split, reported as 0 by pa_decode_partition_size:
 *                 per KV head, the rows' chunks are laid end to end and cut
 *                 into equal ranges, one per wave of the launch (a range may
 *                 span the end of one row and the start of the next), so
 *                 every wave gets the same number of tokens up to one chunk
 *                 whatever the length mix.  Above 1024 rows it is the fixed
 *                 size pa_decode_partition_size returns.
 *   workspace     device scratch of pa_decode_workspace_bytes(); may be NULL
 *                 when that is 0 (every context fits one partition)
 * Shared prefixes (vLLM docs page, 写时复制 and Prefix Caching): in a
 * balanced split of 2..64 rows with bf16 or FP8 caches, head_dim 128 and 4
 * or 8 query heads per KV head, consecutive rows whose tables start with
 * the same physical blocks (forks after copy-on-write, prefix-cache hits)
 * have their common leading tokens, all but each row's last, attended once
 * for all of their query heads.  The kernels find such rows from the
 * tables themselves and check every shared block, so any tables give the
 * same results as rows attended one by one (up to rounding).
 * Results are bitwise reproducible run to run and independent of which
 * physical blocks hold the tokens (the reduction order depends only on
 * logical position and on which rows share blocks).  Calls that share a
 * workspace must be ordered on one stream.
 * ---------------------------------------------------------------------- */
int32_t pa_decode_partition_size(const pa_cache_dims* dims, int32_t num_seqs,
                                 int32_t max_context_len, int32_t partition_size);
size_t pa_decode_workspace_bytes(const pa_cache_dims* dims, int32_t num_seqs,
                                 int32_t max_context_len, int32_t partition_size);
int pa_decode(const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
              float scale, void* out, const pa_cache_dims* dims, int32_t partition_size,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* pa_decode_noalloc — pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the
 * same kernels and results.  The split-K scratch is a fixed
 * PA_NOALLOC_SCRATCH_BYTES array inside the library's device code, one per
 * GPU the library runs on, held until the process ends; the call allocates
 * nothing (no hipMalloc or hipFree, no allocating library routine).  A
 * call whose pa_decode_workspace_bytes() exceeds that size returns
 * PA_ERR_WORKSPACE before any launch.  Every call on one GPU shares its
 * array and leaves its partials there: calls that may overlap on one GPU
 * (different streams, or other threads) race and must be ordered by the
 * caller.  The first call on each device looks up the array's device
 * address (PA_ERR_HIP if that fails). */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                      float scale, void* out, const pa_cache_dims* dims, int32_t partition_size,
                      hipStream_t stream);

/* The two phases of pa_decode, for callers that time or distribute them.
 * pa_decode_partials (same arguments as pa_decode) runs the partition
 * kernel: a sequence with a single partition gets its final row in out; the
 * others leave per-partition (max, sum, unnormalised output) rows in the
 * workspace.  pa_decode_merge then combines those rows in partition order
 * (a log-sum-exp merge) into out; it needs the same context_lens,
 * max_context_len, max_blocks_per_seq, dims and partition_size, and the
 * workspace the partials were written to.  pa_decode == partials + merge. */
int pa_decode_partials(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                       float scale, void* out, const pa_cache_dims* dims, int32_t partition_size,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);
int pa_decode_merge(const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                    int32_t max_blocks_per_seq, void* out, const pa_cache_dims* dims,
                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* pa_decode_append — the decode step's cache write and attention in one
 * launch: the same result as pa_cache_write(k, v, slot_mapping, num_seqs
 * tokens) followed by pa_decode, for a step that appends one token per
 * sequence.  CSDN "vLLM 0.10.0 flow" page §3.3/§3.5 (the new token's K/V
 * goes to the slot slot_mapping names, then attention reads the request's
 * blocks through its table) and SourceAIX page §5.1.1 (decode step: the new
 * token is stored in the current block, then attended).
 *
 *   k, v          [num_seqs][num_kv_heads][head_dim], the q dtype (bf16 for
 *                 FP8 caches, which receive codes as pa_cache_write makes)
 *   slot_mapping  [num_seqs] int32: row s's new token goes to this slot and
 *                 is position context_lens[s] - 1 of row s, i.e. the slot
 *                 block_tables[s] gives that position (as pa_bm_append
 *                 returns it).  A negative or out-of-range slot writes
 *                 nothing, and that position is read from the cache as is.
 *   k_cache, v_cache  written (one slot per row) and read
 * Other arguments, the workspace and the results are those of pa_decode.
 * The new token is attended from registers by the wave that writes it; no
 * other wave reads its slot, which holds because a token is appended to a
 * block its row alone references (copy-on-write).  A row with context 0
 * writes nothing.  Errors as pa_decode, plus PA_ERR_INVALID_ARG for a NULL
 * or misaligned k, v or slot_mapping. */
int pa_decode_append(const void* q, const void* k, const void* v, const int32_t* slot_mapping,
                     void* k_cache, void* v_cache, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                     int32_t max_context_len, float scale, void* out, const pa_cache_dims* dims,
                     int32_t partition_size, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);
/* Its partition phase alone (the write and the partition kernel; same
 * arguments): pa_decode_append == pa_decode_append_partials followed by
 * pa_decode_merge, as for pa_decode. */
int pa_decode_append_partials(const void* q, const void* k, const void* v,
                              const int32_t* slot_mapping, void* k_cache, void* v_cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_context_len, float scale, void* out,
                              const pa_cache_dims* dims, int32_t partition_size, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * pa_varlen — one continuous-batching step mixing chunked prefill and decode.
 * CSDN "vLLM 0.10.0 flow" page §3.2 (a long prefill is cut into chunks that
 * run in the same batch as decode requests) and §3.5 (query_start_loc marks
 * where each request's rows start in the flattened Q); dn008 overview §2.1
 * (each token attends only to itself and earlier tokens).
 *
 *   q                [total_q][num_heads][head_dim], the batch's new tokens
 *   query_start_loc  [num_seqs+1] int32, non-decreasing, [0] = 0,
 *                    [num_seqs] = total_q; segment s owns rows [qsl[s], qsl[s+1])
 *   seq_lens         [num_seqs] int32: tokens of sequence s after this step
 *                    (the segment's own tokens included, already written with
 *                    pa_cache_write); <= max_seq_len and <= max_blocks*block_size
 *   max_query_len    max over segments of qsl[s+1]-qsl[s]
 *   out              [total_q][num_heads][head_dim]
 * Row i of segment s (position P+i, P = seq_lens[s] - q_len) attends keys
 * 0..P+i.  bf16 and FP8_E4M3 caches (bf16 q and out): segments with >= 2
 * rows run an MFMA flash-attention kernel (FP8 codes widened to bf16 in
 * registers as each operand is read, exactly), one-row segments the split-K
 * decode kernels; a batch with
 * few query blocks (e.g. one chunk of a long prompt) has them cut into
 * key-range pieces merged by log-sum-exp, so that the chip fills.  fp32:
 * every row runs the decode kernel with its causal length (correct, not
 * tuned).
 * workspace: device scratch of pa_varlen_workspace_bytes() (may be NULL when
 * that is 0).  Rows of segments with seq_lens < q_len see P = 0.
 * PA_ERR_UNSUPPORTED (before any launch) also when one cache block (K or V)
 * of a bf16/FP8 cache exceeds 4 GiB (block_size * num_kv_heads * head_dim
 * elements), which the prefill kernels address with 32-bit offsets.
 * ---------------------------------------------------------------------- */
size_t pa_varlen_workspace_bytes(const pa_cache_dims* dims, int32_t num_seqs, int32_t total_q,
                                 int32_t max_query_len, int32_t max_seq_len);
int pa_varlen(const void* q, const int32_t* query_start_loc, const int32_t* seq_lens,
              int32_t num_seqs, int32_t total_q, int32_t max_query_len, int32_t max_seq_len,
              const void* k_cache, const void* v_cache, const int32_t* block_tables,
              int32_t max_blocks_per_seq, float scale, void* out, const pa_cache_dims* dims,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Block manager (host C++, no GPU) — the logical-to-physical mapping.
 * "vLLM" documentation page, sections 算法流程 (allocation flow), 引用计数管理
 * (reference counts) and 写时复制 (copy-on-write); SourceAIX page §5.1.1
 * (prefill/decode block filling) and §5.2.1 (parallel sampling).
 *
 * A sequence starts with an empty table.  Each appended token takes the
 * next slot of its last block; when that block is full (or there is none)
 * a block is taken from the front of the free list.  When the last block
 * is not full but shared (reference count > 1), a new block is taken, the
 * caller must copy src -> dst (pa_copy_blocks) before writing, the table
 * is repointed and the old block's count drops by one.  pa_bm_fork shares
 * every block of the parent (+1 each).  pa_bm_free drops one reference per
 * block and returns blocks reaching zero to the back of the free list, in
 * table order.  The initial free-list order is `free_order` (host, a
 * permutation of 0..num_blocks-1) or 0,1,2,... when NULL.
 *
 * Prefix caching ("vLLM" page, sections 共享前缀检测 and Prefix Caching; the
 * free list is doubly linked and least recently released first, CSDN
 * "vLLM 0.10.0 flow" page §3.3): a sequence started with pa_bm_new_prefix
 * hashes every full block of its prompt together with all tokens before it
 * (64-bit FNV-1a chained over the previous block's hash and the block's
 * token ids).  A block whose hash is cached is reused on a hit; a block of
 * the prompt enters the cache when appended tokens fill it, unless that
 * hash is cached already.  A released block keeps its entry while it waits
 * in the free list and can still be hit (it then leaves the list); taking
 * a block from the front of the list for allocation drops its entry.
 * Equal hashes are trusted as equal prefixes (a collision would share a
 * wrong block; at 2^-64 per pair it is not checked).
 * The object is not thread-safe; use one per thread or lock around it.
 * ---------------------------------------------------------------------- */
typedef struct pa_block_manager pa_block_manager;

int pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                 pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);
int pa_bm_new(pa_block_manager* bm, int64_t seq_id);
/* Start seq_id with its prompt (host tokens[n_tokens], token ids).  Reuses
 * the longest run of leading full blocks whose prefix hashes are cached
 * (reference +1 each) and sets *cached_tokens to the tokens they cover
 * (a multiple of block_size, at most n_tokens); the sequence then holds
 * exactly those tokens.  The caller appends the remaining
 * n_tokens - *cached_tokens prompt tokens next, in order, with pa_bm_append
 * and writes their K/V; the cached tokens' K/V is already in the pool.
 * Errors: PA_ERR_INVALID_ARG for a NULL pointer or n_tokens < 0,
 * PA_ERR_NO_SEQUENCE when seq_id exists.  Never allocates a block. */
int pa_bm_new_prefix(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                     int32_t n_tokens, int32_t* cached_tokens);
/* Share every block of parent_id with a new child_id.  The child offers no
 * prompt blocks of its own to the prefix cache. */
int pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id);
int pa_bm_free(pa_block_manager* bm, int64_t seq_id);
/* Give n_tokens new tokens of seq_id their slots (host slots_out[n_tokens]).
 * At most the first token can trigger a copy-on-write: copy_src and copy_dst
 * receive that block pair, or -1/-1.  All-or-nothing: with too few free
 * blocks nothing changes and PA_ERR_OUT_OF_BLOCKS is returned. */
int pa_bm_append(pa_block_manager* bm, int64_t seq_id, int32_t n_tokens,
                 int32_t* slots_out, int32_t* copy_src, int32_t* copy_dst);
int pa_bm_num_tokens(const pa_block_manager* bm, int64_t seq_id, int32_t* out);
/* Copy seq_id's table into host out[cap]; *len_out = its length. */
int pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out,
                      int32_t cap, int32_t* len_out);
int pa_bm_ref_count(const pa_block_manager* bm, int32_t block, int32_t* out);
/* Blocks in the free list (cached ones included: they are evictable). */
int32_t pa_bm_num_free(const pa_block_manager* bm);
/* *out = 1 when block holds a cached prefix, else 0. */
int pa_bm_block_cached(const pa_block_manager* bm, int32_t block, int32_t* out);
/* Host tables_out[n][width] (-1 padded) and context_lens_out[n] for a batch. */
int pa_bm_batch_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                       int32_t* tables_out, int32_t width, int32_t* context_lens_out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
