// Host block manager of libpa: block pool, reference counts, LRU free queue
// and prefix-cache index.  Declarations and the passages followed:
// include/pa_blocks.h.
//
// The free queue is an intrusive doubly linked list over block ids with two
// sentinels, so taking a cached block off the queue on a prefix hit is O(1)
// ("vllm 深度解析：一切从 PagedAttention 谈起", FreeKVCacheBlockQueue).  The
// prefix index maps a block hash to the blocks holding it in insertion order
// (insertion does not deduplicate: "vLLM 深度解析（二）" §4.1).
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/pa.h"
#include "../../include/pa_blocks.h"

struct pa_block_pool {
  int32_t n;                      // blocks, ids 0 .. n-1; 0 is the null block
  bool caching;
  int32_t head, tail;             // sentinel ids n and n+1
  int32_t num_free;
  std::vector<int32_t> prev, next;
  std::vector<char> queued;
  std::vector<int32_t> ref;
  std::vector<char> has_hash;
  std::vector<uint64_t> hash;
  std::unordered_map<uint64_t, std::vector<int32_t>> index;
};

namespace {

void unlink(pa_block_pool* p, int32_t b) {
  p->next[p->prev[b]] = p->next[b];
  p->prev[p->next[b]] = p->prev[b];
  p->queued[b] = 0;
  --p->num_free;
}

void insert_before(pa_block_pool* p, int32_t at, int32_t b) {
  const int32_t pr = p->prev[at];
  p->next[pr] = b;
  p->prev[b] = pr;
  p->next[b] = at;
  p->prev[at] = b;
  p->queued[b] = 1;
  ++p->num_free;
}

void uncache(pa_block_pool* p, int32_t b) {
  if (!p->has_hash[b]) return;
  auto it = p->index.find(p->hash[b]);
  if (it != p->index.end()) {
    auto& v = it->second;
    for (size_t i = 0; i < v.size(); ++i)
      if (v[i] == b) {
        v.erase(v.begin() + (ptrdiff_t)i);
        break;
      }
    if (v.empty()) p->index.erase(it);
  }
  p->has_hash[b] = 0;
}

bool valid_id(const pa_block_pool* p, int32_t b) { return b >= 0 && b < p->n; }

// FNV-1a (64-bit) over little-endian bytes, then the splitmix64 finaliser.
struct Fnv {
  uint64_t h = 0xcbf29ce484222325ull;
  void byte(uint8_t c) {
    h ^= c;
    h *= 0x100000001b3ull;
  }
  void u32(uint32_t v) {
    for (int i = 0; i < 4; ++i) byte((uint8_t)(v >> (8 * i)));
  }
  void u64(uint64_t v) {
    for (int i = 0; i < 8; ++i) byte((uint8_t)(v >> (8 * i)));
  }
};

uint64_t splitmix64_finalise(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

}  // namespace

extern "C" {

int32_t pa_block_hashes(const int32_t* token_ids, int32_t num_tokens, int32_t block_size,
                        uint64_t extra_key, uint64_t* hashes) {
  if (num_tokens < 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
  const int32_t full = num_tokens / block_size;
  if (full > 0 && (!token_ids || !hashes)) return PA_ERR_INVALID_ARG;
  uint64_t parent = PA_NONE_HASH;
  for (int32_t i = 0; i < full; ++i) {
    Fnv f;
    f.u64(parent);
    for (int32_t t = 0; t < block_size; ++t) f.u32((uint32_t)token_ids[(int64_t)i * block_size + t]);
    f.u64(extra_key);
    parent = hashes[i] = splitmix64_finalise(f.h);
  }
  return full;
}

int pa_pool_create(int32_t num_blocks, int32_t enable_caching, pa_block_pool** pool) {
  if (num_blocks < 1 || !pool) return PA_ERR_INVALID_ARG;
  pa_block_pool* p = new pa_block_pool();
  p->n = num_blocks;
  p->caching = enable_caching != 0;
  p->head = num_blocks;
  p->tail = num_blocks + 1;
  p->prev.assign(num_blocks + 2, -1);
  p->next.assign(num_blocks + 2, -1);
  p->queued.assign(num_blocks, 0);
  p->ref.assign(num_blocks, 0);
  p->has_hash.assign(num_blocks, 0);
  p->hash.assign(num_blocks, 0);
  p->num_free = 0;
  p->next[p->head] = p->tail;
  p->prev[p->tail] = p->head;
  for (int32_t b = 1; b < num_blocks; ++b) insert_before(p, p->tail, b);   // 0: null block
  *pool = p;
  return PA_OK;
}

void pa_pool_destroy(pa_block_pool* pool) { delete pool; }

int32_t pa_pool_num_free(const pa_block_pool* pool) { return pool ? pool->num_free : 0; }

double pa_pool_usage(const pa_block_pool* pool) {
  if (!pool || pool->n <= 1) return 0.0;
  return 1.0 - (double)pool->num_free / (double)(pool->n - 1);
}

int32_t pa_pool_ref_count(const pa_block_pool* pool, int32_t block_id) {
  if (!pool || !valid_id(pool, block_id)) return -1;
  return pool->ref[block_id];
}

int32_t pa_pool_lookup(const pa_block_pool* pool, uint64_t hash) {
  if (!pool) return -1;
  auto it = pool->index.find(hash);
  return it == pool->index.end() ? -1 : it->second.front();
}

int pa_pool_get_new_blocks(pa_block_pool* pool, int32_t n, int32_t* block_ids) {
  if (!pool || n < 0 || (n > 0 && !block_ids)) return PA_ERR_INVALID_ARG;
  if (n > pool->num_free) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = pool->next[pool->head];
    unlink(pool, b);
    uncache(pool, b);                 // evict its cached content, if any
    pool->ref[b] += 1;
    block_ids[i] = b;
  }
  return PA_OK;
}

int pa_pool_touch(pa_block_pool* pool, const int32_t* block_ids, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !block_ids)) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (!valid_id(pool, block_ids[i])) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = block_ids[i];
    if (pool->ref[b] == 0 && b != 0 && pool->queued[b]) unlink(pool, b);
    pool->ref[b] += 1;
  }
  return PA_OK;
}

int pa_pool_free_blocks(pa_block_pool* pool, const int32_t* block_ids, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !block_ids)) return PA_ERR_INVALID_ARG;
  std::unordered_map<int32_t, int32_t> dec;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = block_ids[i];
    if (!valid_id(pool, b)) return PA_ERR_INVALID_ARG;
    if (++dec[b] > pool->ref[b]) return PA_ERR_INVALID_ARG;
  }
  std::vector<int32_t> to_head;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = block_ids[i];
    pool->ref[b] -= 1;
    if (pool->ref[b] != 0 || b == 0) continue;
    if (pool->has_hash[b])
      insert_before(pool, pool->tail, b);         // cached: least recently freed first
    else
      to_head.push_back(b);                       // nothing to keep: reused first
  }
  const int32_t first = pool->next[pool->head];
  for (int32_t b : to_head) insert_before(pool, first, b);   // given order, at the head
  return PA_OK;
}

int pa_pool_cache_block(pa_block_pool* pool, int32_t block_id, uint64_t hash) {
  if (!pool || !valid_id(pool, block_id) || block_id == 0) return PA_ERR_INVALID_ARG;
  if (!pool->caching || pool->has_hash[block_id]) return PA_OK;
  pool->has_hash[block_id] = 1;
  pool->hash[block_id] = hash;
  pool->index[hash].push_back(block_id);
  return PA_OK;
}

int pa_pool_allocate_prompt(pa_block_pool* pool, const uint64_t* hashes, int32_t num_hashes,
                            int32_t num_tokens, int32_t block_size, int32_t* block_ids,
                            int32_t max_blocks, int32_t* num_cached_tokens) {
  if (!pool || num_tokens < 0 || block_size <= 0 || num_hashes < 0) return PA_ERR_INVALID_ARG;
  if (num_hashes > num_tokens / block_size || (num_hashes > 0 && !hashes))
    return PA_ERR_INVALID_ARG;
  const int32_t nblk = (num_tokens + block_size - 1) / block_size;
  if (nblk > max_blocks || (nblk > 0 && !block_ids)) return PA_ERR_INVALID_ARG;
  // longest cached prefix, leaving at least the last token to compute
  std::vector<int32_t> hit;
  if (pool->caching) {
    for (int32_t i = 0; i < num_hashes; ++i) {
      if ((int64_t)(i + 1) * block_size > (int64_t)num_tokens - 1) break;
      const int32_t b = pa_pool_lookup(pool, hashes[i]);
      if (b < 0) break;
      hit.push_back(b);
    }
  }
  int32_t queued_hits = 0;
  for (int32_t b : hit) queued_hits += (pool->ref[b] == 0 && pool->queued[b]) ? 1 : 0;
  const int32_t need = nblk - (int32_t)hit.size();
  if (need > pool->num_free - queued_hits) return PA_ERR_INVALID_ARG;
  if (!hit.empty()) pa_pool_touch(pool, hit.data(), (int32_t)hit.size());
  for (size_t i = 0; i < hit.size(); ++i) block_ids[i] = hit[i];
  if (need > 0) pa_pool_get_new_blocks(pool, need, block_ids + hit.size());
  if (num_cached_tokens) *num_cached_tokens = (int32_t)hit.size() * block_size;
  return PA_OK;
}

int pa_pool_commit(pa_block_pool* pool, const int32_t* block_ids, const uint64_t* hashes,
                   int32_t num_hashes) {
  if (!pool || num_hashes < 0 || (num_hashes > 0 && (!block_ids || !hashes)))
    return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < num_hashes; ++i)
    if (!valid_id(pool, block_ids[i]) || block_ids[i] == 0) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < num_hashes; ++i) pa_pool_cache_block(pool, block_ids[i], hashes[i]);
  return PA_OK;
}

int pa_pool_free_request(pa_block_pool* pool, const int32_t* block_ids, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !block_ids)) return PA_ERR_INVALID_ARG;
  std::vector<int32_t> rev(block_ids, block_ids + n);
  for (int32_t i = 0; i < n / 2; ++i) std::swap(rev[i], rev[n - 1 - i]);
  return pa_pool_free_blocks(pool, rev.data(), n);
}

int pa_map_to_kernel_blocks(const int32_t* ids, int32_t n, int32_t blocks_per_kv_block,
                            int32_t* out) {
  const int32_t k = blocks_per_kv_block;
  if (n < 0 || k < 1 || (n > 0 && (!ids || !out))) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] >= 0 && (int64_t)ids[i] * k + (k - 1) > INT32_MAX) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    for (int32_t j = 0; j < k; ++j)
      out[(int64_t)i * k + j] = ids[i] < 0 ? ids[i] : ids[i] * k + j;
  return PA_OK;
}

}  // extern "C"
