// pool.cpp -- host page table with exact prefix sharing (Vosti: Specifying,
// Implementing, and Verifying Deterministic LLM Inference, §4.1 "Exact prefix
// matching" and "Separate cache reuse from generation", §4.2-4.3 "Sharing and
// write isolation", "State updates", Figure 2).
//
// Pages are refcounted by live sequences.  A page is published -- entered in
// the prefix index with (parent page, depth, tokens) -- once it is full and
// its K/V are computed; published pages are immutable.  A rolling hash over
// the token chain finds candidate pages; reuse then requires the exact
// tokens, the same depth and the same physical parent page, so a hash
// collision never justifies reuse.  Unreferenced published pages are retained
// until evicted, and only leaves (no published child) are evicted, least
// recently released first (ties by page id).  Free pages are handed out lowest
// id first.  Integer bookkeeping only; no device memory.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/invattn.h"
#include "errors.hpp"

using ia::fail;
using ia::ok;

struct ia_seq {
  std::vector<int32_t> history;  // prompt + appended tokens
  std::vector<int32_t> pages;    // physical page of each logical page
  std::vector<uint64_t> chain;   // chain hash of each full page of the history
  int32_t reserved = 0;          // positions that have a write slot
  int32_t computed = 0;          // positions whose K/V are computed
  int32_t n_published = 0;       // leading pages that are published
};

struct ia_pool {
  int32_t num_pages = 0;
  int32_t P = 0;
  bool constant_hash = false;
  std::vector<int32_t> refs;
  std::vector<uint8_t> published;
  std::vector<int32_t> parent;
  std::vector<int32_t> depth;
  std::vector<int32_t> children;  // published children of a published page
  std::vector<int32_t> tokens;    // [num_pages][P]
  std::vector<uint64_t> hash;
  std::vector<int64_t> released_at;
  int64_t clock = 0;
  std::set<int32_t> free_pages;
  std::set<std::pair<int64_t, int32_t>> evictable;  // (released_at, page)
  std::unordered_multimap<uint64_t, int32_t> index;
};

namespace {

uint64_t mix(uint64_t h, uint64_t x) {
  // splitmix64 step over (h ^ x)
  uint64_t z = h ^ (x + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2));
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t block_hash(const ia_pool* pool, uint64_t parent_hash, const int32_t* toks) {
  if (pool->constant_hash) return 0;
  uint64_t h = mix(parent_hash, 0x5EEDull);
  for (int32_t i = 0; i < pool->P; ++i) h = mix(h, (uint32_t)toks[i]);
  return h;
}

bool is_evictable(const ia_pool* pool, int32_t pg) {
  return pool->published[pg] && pool->refs[pg] == 0 && pool->children[pg] == 0;
}

void refresh_evictable(ia_pool* pool, int32_t pg) {
  auto key = std::make_pair(pool->released_at[pg], pg);
  if (is_evictable(pool, pg))
    pool->evictable.insert(key);
  else
    pool->evictable.erase(key);
}

// The published page (parent, depth, toks) or -1.
int32_t find_page(const ia_pool* pool, uint64_t h, int32_t parent, int32_t depth, const int32_t* toks) {
  auto range = pool->index.equal_range(h);
  for (auto it = range.first; it != range.second; ++it) {
    const int32_t pg = it->second;
    if (!pool->published[pg] || pool->parent[pg] != parent || pool->depth[pg] != depth) continue;
    if (std::memcmp(&pool->tokens[(size_t)pg * pool->P], toks, sizeof(int32_t) * pool->P) == 0) return pg;
  }
  return -1;
}

void publish(ia_pool* pool, int32_t pg, uint64_t h, int32_t parent, int32_t depth, const int32_t* toks) {
  pool->published[pg] = 1;
  pool->parent[pg] = parent;
  pool->depth[pg] = depth;
  pool->hash[pg] = h;
  pool->children[pg] = 0;
  std::memcpy(&pool->tokens[(size_t)pg * pool->P], toks, sizeof(int32_t) * pool->P);
  pool->index.emplace(h, pg);
  if (parent >= 0) {
    pool->children[parent] += 1;
    refresh_evictable(pool, parent);
  }
  refresh_evictable(pool, pg);
}

void unpublish_and_free(ia_pool* pool, int32_t pg) {
  pool->evictable.erase(std::make_pair(pool->released_at[pg], pg));
  auto range = pool->index.equal_range(pool->hash[pg]);
  for (auto it = range.first; it != range.second; ++it)
    if (it->second == pg) {
      pool->index.erase(it);
      break;
    }
  pool->published[pg] = 0;
  const int32_t parent = pool->parent[pg];
  pool->parent[pg] = -1;
  if (parent >= 0) {
    pool->children[parent] -= 1;
    refresh_evictable(pool, parent);
  }
  pool->free_pages.insert(pg);
}

int32_t evict_n(ia_pool* pool, int32_t want) {
  int32_t done = 0;
  while (done < want && !pool->evictable.empty()) {
    const int32_t pg = pool->evictable.begin()->second;
    unpublish_and_free(pool, pg);
    ++done;
  }
  return done;
}

// Chain hash of full page i of the sequence's history (computed on demand).
uint64_t chain_hash(const ia_pool* pool, ia_seq* seq, int32_t i) {
  while ((int32_t)seq->chain.size() <= i) {
    const int32_t k = (int32_t)seq->chain.size();
    const uint64_t prev = k == 0 ? 0 : seq->chain[k - 1];
    seq->chain.push_back(block_hash(pool, prev, &seq->history[(size_t)k * pool->P]));
  }
  return seq->chain[i];
}

}  // namespace

extern "C" {

ia_status ia_pool_create(int32_t num_pages, int32_t page_size, int32_t flags, ia_pool** out) {
  if (!out) return fail(IA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (num_pages <= 0 || page_size <= 0) return fail(IA_ERR_INVALID_ARG, "num_pages and page_size must be positive");
  if (flags & ~IA_POOL_CONSTANT_HASH) return fail(IA_ERR_INVALID_ARG, "unknown pool flags %d", flags);
  ia_pool* pool = new (std::nothrow) ia_pool;
  if (!pool) return fail(IA_ERR_INTERNAL, "out of host memory");
  try {
    pool->num_pages = num_pages;
    pool->P = page_size;
    pool->constant_hash = (flags & IA_POOL_CONSTANT_HASH) != 0;
    pool->refs.assign(num_pages, 0);
    pool->published.assign(num_pages, 0);
    pool->parent.assign(num_pages, -1);
    pool->depth.assign(num_pages, -1);
    pool->children.assign(num_pages, 0);
    pool->tokens.assign((size_t)num_pages * page_size, 0);
    pool->hash.assign(num_pages, 0);
    pool->released_at.assign(num_pages, 0);
    for (int32_t i = 0; i < num_pages; ++i) pool->free_pages.insert(pool->free_pages.end(), i);
  } catch (...) {
    delete pool;
    return fail(IA_ERR_INTERNAL, "out of host memory");
  }
  *out = pool;
  return ok();
}

void ia_pool_destroy(ia_pool* pool) { delete pool; }

ia_status ia_seq_begin(ia_pool* pool, const int32_t* tokens, int32_t n, ia_seq** out, int32_t* cached_len) {
  if (!pool || !tokens || !out || !cached_len) return fail(IA_ERR_INVALID_ARG, "NULL argument");
  if (n <= 0) return fail(IA_ERR_INVALID_ARG, "a sequence needs at least one token (got %d)", n);
  *out = nullptr;
  ia_seq* seq = new (std::nothrow) ia_seq;
  if (!seq) return fail(IA_ERR_INTERNAL, "out of host memory");
  try {
    seq->history.assign(tokens, tokens + n);
    const int32_t P = pool->P;
    int32_t parent = -1, depth = 0;
    // Resolve every hit before this sequence registers anything; keep at least
    // one token to compute.
    while ((int64_t)(depth + 1) * P < n) {
      const uint64_t h = chain_hash(pool, seq, depth);
      const int32_t pg = find_page(pool, h, parent, depth, &seq->history[(size_t)depth * P]);
      if (pg < 0) break;
      pool->refs[pg] += 1;
      refresh_evictable(pool, pg);
      seq->pages.push_back(pg);
      parent = pg;
      ++depth;
    }
    seq->reserved = seq->computed = depth * P;
    seq->n_published = depth;
  } catch (...) {
    delete seq;
    return fail(IA_ERR_INTERNAL, "out of host memory");
  }
  *cached_len = seq->computed;
  *out = seq;
  return ok();
}

ia_status ia_seq_append_tokens(ia_pool* pool, ia_seq* seq, const int32_t* tokens, int32_t n) {
  if (!pool || !seq || (n > 0 && !tokens) || n < 0) return fail(IA_ERR_INVALID_ARG, "bad argument");
  try {
    seq->history.insert(seq->history.end(), tokens, tokens + n);
  } catch (...) {
    return fail(IA_ERR_INTERNAL, "out of host memory");
  }
  return ok();
}

ia_status ia_seq_reserve(ia_pool* pool, ia_seq* seq, int32_t n_new, int64_t* slot_mapping_out) {
  if (!pool || !seq || n_new < 0 || (n_new > 0 && !slot_mapping_out)) return fail(IA_ERR_INVALID_ARG, "bad argument");
  if ((int64_t)seq->reserved + n_new > (int64_t)seq->history.size())
    return fail(IA_ERR_INVALID_ARG, "reserving %d positions past the %zu-token history", n_new, seq->history.size());
  const int32_t P = pool->P;
  const int64_t need = ((int64_t)seq->reserved + n_new + P - 1) / P - (int64_t)seq->pages.size();
  if (need > (int64_t)pool->free_pages.size()) evict_n(pool, (int32_t)(need - (int64_t)pool->free_pages.size()));
  if (need > (int64_t)pool->free_pages.size())
    return fail(IA_ERR_OUT_OF_PAGES, "need %lld free pages, %zu left after eviction", (long long)need,
                pool->free_pages.size());
  try {
    for (int64_t k = 0; k < need; ++k) {
      const int32_t pg = *pool->free_pages.begin();
      pool->free_pages.erase(pool->free_pages.begin());
      pool->refs[pg] = 1;
      seq->pages.push_back(pg);
    }
  } catch (...) {
    return fail(IA_ERR_INTERNAL, "out of host memory");
  }
  for (int32_t k = 0; k < n_new; ++k) {
    const int64_t pos = (int64_t)seq->reserved + k;
    slot_mapping_out[k] = (int64_t)seq->pages[pos / P] * P + pos % P;
  }
  seq->reserved += n_new;
  return ok();
}

ia_status ia_seq_commit(ia_pool* pool, ia_seq* seq, int32_t n_done) {
  if (!pool || !seq || n_done < 0 || (int64_t)seq->computed + n_done > seq->reserved)
    return fail(IA_ERR_INVALID_ARG, "commit of %d positions exceeds the reservation", n_done);
  seq->computed += n_done;
  const int32_t P = pool->P;
  try {
    // Publish full, computed pages in order; the chain stops at the first page
    // that duplicates a published one.
    for (int32_t i = seq->n_published; (int64_t)(i + 1) * P <= seq->computed; ++i) {
      const int32_t pg = seq->pages[i];
      const int32_t parent = i > 0 ? seq->pages[i - 1] : -1;
      const uint64_t h = chain_hash(pool, seq, i);
      const int32_t* toks = &seq->history[(size_t)i * P];
      if (find_page(pool, h, parent, i, toks) >= 0) break;
      publish(pool, pg, h, parent, i, toks);
      seq->n_published = i + 1;
    }
  } catch (...) {
    return fail(IA_ERR_INTERNAL, "out of host memory");
  }
  return ok();
}

ia_status ia_seq_block_table(const ia_seq* seq, int32_t* out, int32_t cap, int32_t* n_pages) {
  if (!seq || !n_pages) return fail(IA_ERR_INVALID_ARG, "NULL argument");
  *n_pages = (int32_t)seq->pages.size();
  if (cap < *n_pages || (*n_pages > 0 && !out))
    return fail(IA_ERR_INVALID_ARG, "block table needs %d entries (cap %d)", *n_pages, cap);
  if (*n_pages > 0) std::memcpy(out, seq->pages.data(), sizeof(int32_t) * seq->pages.size());
  return ok();
}

int32_t ia_seq_len(const ia_seq* seq) { return seq ? seq->computed : -1; }

ia_status ia_seq_end(ia_pool* pool, ia_seq* seq) {
  if (!pool || !seq) return fail(IA_ERR_INVALID_ARG, "NULL argument");
  for (const int32_t pg : seq->pages) {
    pool->refs[pg] -= 1;
    if (pool->published[pg]) {
      if (pool->refs[pg] == 0) {
        pool->released_at[pg] = pool->clock++;
        refresh_evictable(pool, pg);
      }
    } else {
      pool->refs[pg] = 0;
      pool->free_pages.insert(pg);
    }
  }
  delete seq;
  return ok();
}

ia_status ia_pool_evict(ia_pool* pool, int32_t want, int32_t* evicted) {
  if (!pool || !evicted || want < 0) return fail(IA_ERR_INVALID_ARG, "bad argument");
  *evicted = evict_n(pool, want);
  return ok();
}

int32_t ia_pool_page_refs(const ia_pool* pool, int32_t page) {
  if (!pool || page < 0 || page >= pool->num_pages) return -1;
  return pool->refs[page];
}

int32_t ia_pool_page_published(const ia_pool* pool, int32_t page) {
  if (!pool || page < 0 || page >= pool->num_pages) return -1;
  return pool->published[page];
}

int32_t ia_pool_num_free(const ia_pool* pool) { return pool ? (int32_t)pool->free_pages.size() : -1; }

// ---------------------------------------------------------------------------
// Opt-in host checks of the preconditions the launches leave unchecked (Vosti
// §4.3 "Sharing and write isolation": new K/V go only to private, disjoint
// slots; shared pages are never written).

ia_status ia_validate_slots(const ia_pool* pool, const int64_t* slot_mapping, int32_t T, int32_t num_pages,
                            int32_t page_size) {
  if (T < 0 || num_pages <= 0 || page_size <= 0 || (T > 0 && !slot_mapping))
    return fail(IA_ERR_INVALID_ARG, "bad argument");
  if (pool && (pool->num_pages != num_pages || pool->P != page_size))
    return fail(IA_ERR_INVALID_ARG, "pool has %d pages of %d tokens, the call names %d of %d", pool->num_pages,
                pool->P, num_pages, page_size);
  const int64_t limit = (int64_t)num_pages * page_size;
  std::vector<int64_t> seen;
  try {
    seen.reserve((size_t)T);
  } catch (...) {
    return fail(IA_ERR_INTERNAL, "out of host memory");
  }
  for (int32_t i = 0; i < T; ++i) {
    const int64_t s = slot_mapping[i];
    if (s < 0) continue;  // a padding row writes nothing
    if (s >= limit) return fail(IA_ERR_INVALID_ARG, "slot_mapping[%d] = %lld is past the pool", i, (long long)s);
    if (pool && pool->published[(size_t)(s / page_size)])
      return fail(IA_ERR_PAGE_REFERENCED, "slot_mapping[%d] = %lld lands on published page %lld", i, (long long)s,
                  (long long)(s / page_size));
    seen.push_back(s);
  }
  std::sort(seen.begin(), seen.end());
  for (size_t i = 1; i < seen.size(); ++i)
    if (seen[i] == seen[i - 1]) return fail(IA_ERR_INVALID_ARG, "slot %lld is written twice", (long long)seen[i]);
  return ok();
}

ia_status ia_validate_attention_args(const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t B, int32_t total_q,
                                     const int32_t* block_table, int32_t bt_stride, int32_t num_pages,
                                     int32_t page_size, int32_t max_seq_len) {
  if (B < 0 || (B > 0 && (!seq_lens || !block_table)) || num_pages <= 0 || page_size <= 0 || bt_stride < 0)
    return fail(IA_ERR_INVALID_ARG, "bad argument");
  if (cu_q_lens) {
    if (cu_q_lens[0] != 0) return fail(IA_ERR_INVALID_ARG, "cu_q_lens[0] = %d, not 0", cu_q_lens[0]);
    if (cu_q_lens[B] != total_q)
      return fail(IA_ERR_INVALID_ARG, "cu_q_lens[%d] = %d, not total_q = %d", B, cu_q_lens[B], total_q);
  }
  for (int32_t b = 0; b < B; ++b) {
    const int64_t q_len = cu_q_lens ? (int64_t)cu_q_lens[b + 1] - cu_q_lens[b] : 1;
    const int64_t n = seq_lens[b];
    if (q_len < 1 || q_len > n || n > max_seq_len)
      return fail(IA_ERR_INVALID_ARG, "sequence %d: need 1 <= q_len (%lld) <= seq_len (%lld) <= max_seq_len (%d)", b,
                  (long long)q_len, (long long)n, max_seq_len);
    const int64_t pages = (n + page_size - 1) / page_size;
    if (pages > bt_stride)
      return fail(IA_ERR_INVALID_ARG, "sequence %d: %lld pages do not fit a block-table row of %d", b,
                  (long long)pages, bt_stride);
    for (int64_t j = 0; j < pages; ++j) {
      const int32_t e = block_table[(size_t)b * bt_stride + j];
      if (e < 0 || e >= num_pages)
        return fail(IA_ERR_INVALID_ARG, "sequence %d: block_table entry %lld = %d is not a page", b, (long long)j, e);
    }
  }
  return ok();
}

}  // extern "C"
