// Host block manager: logical token blocks of each sequence mapped onto a
// pool of physical KV blocks, with on-demand allocation, reference counts,
// copy-on-write and prefix caching.
//
// Follows the allocation flow, reference counting and copy-on-write rules of
// the "vLLM" documentation page (sections 算法流程, 引用计数管理, 写时复制) and
// the SourceAIX code-reading page (§5.1.1 block filling, §5.2.1 parallel
// sampling).  The free pool is a doubly linked list in LRU order: blocks are
// taken from the front and released to the back (the CSDN "vLLM 0.10.0 flow"
// page, §3.3, keeps free blocks in a doubly linked list with LRU eviction).
//
// Prefix caching (the "vLLM" page, sections 共享前缀检测 and Prefix
// Caching): every full block of a prompt started with pa_bm_new_prefix gets
// a hash of the whole token prefix up to its end; a new prompt reuses the
// longest run of leading blocks whose hashes are cached (reference +1, and
// those tokens skip prefill).  A released block keeps its hash while it sits
// in the free list, so a later request can still reuse it; it is evicted
// (hash dropped) only when allocation takes it from the front of the list.
//
// Data layout: one flat vector of block numbers per sequence; reference
// counts, free-list links and block hashes in dense arrays indexed by
// physical block; a hash map from prefix hash to block.
#include <algorithm>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  // free list: doubly linked through prev/next, -1 terminated
  std::vector<int32_t> prev, next;
  int32_t front = -1, back = -1;
  int64_t count = 0;  // blocks in the free list
  std::vector<int32_t> refs;
  std::vector<uint64_t> hash;   // prefix hash of a cached block
  std::vector<uint8_t> cached;  // block is registered in `by_hash`
  std::unordered_map<uint64_t, int32_t> by_hash;
  struct Seq {
    std::vector<int32_t> table;
    int32_t tokens = 0;
    std::vector<uint64_t> hashes;  // prefix hashes of the prompt's full blocks
    int32_t registered = 0;        // leading blocks whose hash has been offered
  };
  std::unordered_map<int64_t, Seq> seqs;

  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else front = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else back = prev[b];
    prev[b] = next[b] = -1;
    --count;
  }
  int32_t take() {
    const int32_t b = front;
    unlink(b);
    if (cached[b]) {  // evict: the least recently released cached block
      by_hash.erase(hash[b]);
      cached[b] = 0;
    }
    refs[b] = 1;
    return b;
  }
  void give_back(int32_t b) {
    prev[b] = back;
    next[b] = -1;
    if (back >= 0) next[back] = b; else front = b;
    back = b;
    ++count;
  }
  // offers the hashes of the sequence's blocks that are now full
  void register_full(Seq& s) {
    const int32_t full = s.tokens / block_size;
    const int32_t upto = std::min<int32_t>(full, static_cast<int32_t>(s.hashes.size()));
    for (; s.registered < upto; ++s.registered) {
      const int32_t b = s.table[s.registered];
      const uint64_t h = s.hashes[s.registered];
      if (cached[b] || by_hash.count(h)) continue;  // already cached (here or elsewhere)
      by_hash.emplace(h, b);
      hash[b] = h;
      cached[b] = 1;
    }
  }
};

namespace {

// Prefix hash of block i: FNV-1a over the previous block's hash and this
// block's token ids, so equal hashes mean (up to collisions) equal prefixes.
uint64_t chain_hash(uint64_t prev_hash, const int32_t* tokens, int32_t n) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&](uint64_t v) {
    for (int i = 0; i < 8; ++i) {
      h ^= (v >> (8 * i)) & 0xFF;
      h *= 1099511628211ull;
    }
  };
  mix(prev_hash);
  for (int32_t i = 0; i < n; ++i) mix(static_cast<uint32_t>(tokens[i]));
  return h;
}

}  // namespace

extern "C" {

int pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                 pa_block_manager** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (!bm) return PA_ERR_INVALID_ARG;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->prev.assign(num_blocks, -1);
  bm->next.assign(num_blocks, -1);
  bm->refs.assign(num_blocks, 0);
  bm->hash.assign(num_blocks, 0);
  bm->cached.assign(num_blocks, 0);
  std::vector<uint8_t> seen(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {
      delete bm;
      return PA_ERR_INVALID_ARG;  // not a permutation of the pool
    }
    seen[b] = 1;
    bm->give_back(b);
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_new(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_INVALID_ARG;
  if (bm->seqs.count(seq_id)) return PA_ERR_NO_SEQUENCE;
  bm->seqs.emplace(seq_id, pa_block_manager::Seq{});
  return PA_OK;
}

int pa_bm_new_prefix(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                     int32_t n_tokens, int32_t* cached_tokens) {
  if (!bm || n_tokens < 0 || (n_tokens > 0 && !tokens) || !cached_tokens)
    return PA_ERR_INVALID_ARG;
  if (bm->seqs.count(seq_id)) return PA_ERR_NO_SEQUENCE;
  pa_block_manager::Seq s;
  const int32_t B = bm->block_size;
  uint64_t h = 0;
  for (int32_t i = 0; i + 1 <= n_tokens / B; ++i) {
    h = chain_hash(h, tokens + static_cast<int64_t>(i) * B, B);
    s.hashes.push_back(h);
  }
  // the longest run of leading blocks already cached
  for (const uint64_t hb : s.hashes) {
    auto it = bm->by_hash.find(hb);
    if (it == bm->by_hash.end()) break;
    const int32_t b = it->second;
    if (bm->refs[b] == 0) bm->unlink(b);  // it was free: in use again
    ++bm->refs[b];
    s.table.push_back(b);
  }
  s.tokens = static_cast<int32_t>(s.table.size()) * B;
  s.registered = static_cast<int32_t>(s.table.size());
  *cached_tokens = s.tokens;
  bm->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

int pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end() || bm->seqs.count(child_id)) return PA_ERR_NO_SEQUENCE;
  pa_block_manager::Seq child = it->second;  // copy before emplace may rehash
  child.hashes.clear();  // the parent offers the prompt's blocks; the child shares them
  child.registered = 0;
  for (int32_t b : child.table) ++bm->refs[b];
  bm->seqs.emplace(child_id, std::move(child));
  return PA_OK;
}

int pa_bm_free(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
  for (int32_t b : it->second.table) {
    if (--bm->refs[b] == 0) bm->give_back(b);
  }
  bm->seqs.erase(it);
  return PA_OK;
}

int pa_bm_append(pa_block_manager* bm, int64_t seq_id, int32_t n_tokens, int32_t* slots_out,
                 int32_t* copy_src, int32_t* copy_dst) {
  if (!bm || n_tokens < 0 || (n_tokens > 0 && !slots_out)) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
  if (copy_src) *copy_src = -1;
  if (copy_dst) *copy_dst = -1;
  if (n_tokens == 0) return PA_OK;
  auto& s = it->second;
  const int64_t B = bm->block_size;
  const int64_t n0 = s.tokens;
  const int64_t have = static_cast<int64_t>(s.table.size());
  // Blocks this append needs from the pool: the ones its tokens open, plus
  // one when the first token lands in a shared, partly filled last block.
  const int64_t need_total = (n0 + n_tokens + B - 1) / B;
  const bool cow = (n0 < have * B) && bm->refs[s.table.back()] > 1;
  const int64_t need = (need_total - have) + (cow ? 1 : 0);
  if (need > bm->count) return PA_ERR_OUT_OF_BLOCKS;
  if (n0 + n_tokens > INT32_MAX) return PA_ERR_INVALID_ARG;

  if (cow) {
    const int32_t old = s.table.back();
    const int32_t nb = bm->take();
    s.table.back() = nb;
    --bm->refs[old];
    if (copy_src) *copy_src = old;
    if (copy_dst) *copy_dst = nb;
  }
  for (int32_t i = 0; i < n_tokens; ++i) {
    const int64_t pos = n0 + i;
    if (pos == static_cast<int64_t>(s.table.size()) * B) s.table.push_back(bm->take());
    slots_out[i] = static_cast<int32_t>(static_cast<int64_t>(s.table[pos / B]) * B + pos % B);
  }
  s.tokens = static_cast<int32_t>(n0 + n_tokens);
  bm->register_full(s);
  return PA_OK;
}

int pa_bm_num_tokens(const pa_block_manager* bm, int64_t seq_id, int32_t* out) {
  if (!bm || !out) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
  *out = it->second.tokens;
  return PA_OK;
}

int pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out, int32_t cap,
                      int32_t* len_out) {
  if (!bm || cap < 0 || (cap > 0 && !out)) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
  const auto& t = it->second.table;
  const int32_t n = static_cast<int32_t>(t.size());
  if (len_out) *len_out = n;
  std::copy(t.begin(), t.begin() + std::min(n, cap), out);
  return n <= cap ? PA_OK : PA_ERR_INVALID_ARG;
}

int pa_bm_ref_count(const pa_block_manager* bm, int32_t block, int32_t* out) {
  if (!bm || !out || block < 0 || block >= bm->num_blocks) return PA_ERR_INVALID_ARG;
  *out = bm->refs[block];
  return PA_OK;
}

int32_t pa_bm_num_free(const pa_block_manager* bm) {
  return bm ? static_cast<int32_t>(bm->count) : -1;
}

int pa_bm_block_cached(const pa_block_manager* bm, int32_t block, int32_t* out) {
  if (!bm || !out || block < 0 || block >= bm->num_blocks) return PA_ERR_INVALID_ARG;
  *out = bm->cached[block];
  return PA_OK;
}

int pa_bm_batch_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                       int32_t* tables_out, int32_t width, int32_t* context_lens_out) {
  if (!bm || n < 0 || width < 0 || (n > 0 && (!seq_ids || !context_lens_out)) ||
      (n > 0 && width > 0 && !tables_out))
    return PA_ERR_INVALID_ARG;
  for (int32_t r = 0; r < n; ++r) {
    auto it = bm->seqs.find(seq_ids[r]);
    if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
    if (static_cast<int32_t>(it->second.table.size()) > width) return PA_ERR_INVALID_ARG;
  }
  for (int32_t r = 0; r < n; ++r) {
    const auto& s = bm->seqs.find(seq_ids[r])->second;
    int32_t* row = tables_out + static_cast<int64_t>(r) * width;
    std::fill(row, row + width, -1);
    std::copy(s.table.begin(), s.table.end(), row);
    context_lens_out[r] = s.tokens;
  }
  return PA_OK;
}

}  // extern "C"
