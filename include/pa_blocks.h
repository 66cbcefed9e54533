/*
 * pa_blocks.h -- host-side block manager of libpa: the pool of physical KV
 * cache blocks, their reference counts, the LRU free queue and the
 * prefix-cache index that let requests share full blocks.  It produces the
 * block-table rows the attention kernels of pa.h read.  Host memory only;
 * no GPU call is made.
 *
 * Follows:
 *   [P1] "vLLM 深度解析（二）：PagedAttention 核心机制" §4.1 (chained block hash
 *        H_i = H(H_{i-1}, token_ids_i, extra_keys_i); only full blocks are
 *        cached; touch() takes a cached block off the free queue and raises
 *        its count; free_blocks() lowers counts and queues blocks that reach
 *        zero; at least the last prompt token is always recomputed)
 *   [P3] "vllm 深度解析：一切从 PagedAttention 谈起" (BlockPool,
 *        FreeKVCacheBlockQueue, BlockHashToBlockMap, the ref_cnt timeline of
 *        two requests sharing a block)
 *   [P4] "LLM 推理基础与 vLLM 内部机制：KV 缓存、PagedAttention、调度器" §9-§10
 *        (block LRU model: least recently freed evicted first, tail blocks
 *        queued first, partial blocks carry no hash)
 *
 * Conventions: return PA_OK (0) or a negative pa_status of pa.h; every
 * array is a HOST pointer owned by the caller; a pool is not thread-safe
 * (one owner, e.g. the scheduler thread).  Block 0 is the null block: it is
 * taken off the queue at creation and never handed out, so a pool of
 * num_blocks blocks has num_blocks - 1 usable ones.
 *
 * Free queue order (this library's reading of the pages): the head is
 * evicted first.  free_blocks() appends blocks that reach count zero in the
 * order given, except blocks with no cached hash, which go to the head:
 * they hold nothing reusable, so they are handed out before any cached
 * block is evicted (the pages' LRU model treats a freed partial block as
 * immediately reusable).
 */
#ifndef PA_BLOCKS_H_
#define PA_BLOCKS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_pool pa_block_pool;

/* Hash of the parent of the first block (P1 §4.1: a missing parent hash is
 * replaced by a fixed NONE_HASH). */
#define PA_NONE_HASH 0x9e3779b97f4a7c15ull

/*
 * Chained hashes of the full blocks of a token sequence (P1 §4.1):
 *     hashes[i] = H(parent_i, token_ids[i*B .. i*B+B-1], extra_key),
 *     parent_0 = PA_NONE_HASH, parent_i = hashes[i-1].
 * H is 64-bit FNV-1a over the little-endian bytes of parent, the B token ids
 * (int32) and extra_key (uint64), followed by the splitmix64 finaliser.
 * Writes floor(num_tokens / B) hashes; returns that count (or a negative
 * status for bad arguments).  A trailing partial block gets no hash.
 */
int32_t pa_block_hashes(const int32_t* token_ids, int32_t num_tokens, int32_t block_size,
                        uint64_t extra_key, uint64_t* hashes);

/* Create / destroy a pool (enable_caching = 0: no prefix index). */
int pa_pool_create(int32_t num_blocks, int32_t enable_caching, pa_block_pool** pool);
void pa_pool_destroy(pa_block_pool* pool);

/* Blocks in the free queue (cached, evictable blocks included). */
int32_t pa_pool_num_free(const pa_block_pool* pool);
/* 1 - num_free / (num_blocks - 1)  (P3 get_usage). */
double pa_pool_usage(const pa_block_pool* pool);
/* Reference count of a block, -1 for an id out of range. */
int32_t pa_pool_ref_count(const pa_block_pool* pool, int32_t block_id);
/* The block holding hash h in the prefix index, or -1 (any one of several). */
int32_t pa_pool_lookup(const pa_block_pool* pool, uint64_t hash);

/*
 * n blocks from the head of the free queue (P3 get_new_blocks): each block
 * leaves the prefix index if it was cached (eviction) and gets count 1.
 * PA_ERR_INVALID_ARG (nothing taken) when fewer than n blocks are free.
 */
int pa_pool_get_new_blocks(pa_block_pool* pool, int32_t n, int32_t* block_ids);

/* Count +1 for each block; blocks at count 0 leave the free queue first
 * (P1 §4.1 touch).  The null block is never queued. */
int pa_pool_touch(pa_block_pool* pool, const int32_t* block_ids, int32_t n);

/* Count -1 for each block; those reaching 0 are queued (see the order above;
 * the first block given is evicted first).  PA_ERR_INVALID_ARG, with no
 * change, if a count would go negative. */
int pa_pool_free_blocks(pa_block_pool* pool, const int32_t* block_ids, int32_t n);

/* Record that block_id holds the full block with hash h (a block is cached
 * once; several blocks may hold one hash -- insertion does not deduplicate,
 * P1 §4.1). */
int pa_pool_cache_block(pa_block_pool* pool, int32_t block_id, uint64_t hash);

/*
 * Blocks for a prompt of num_tokens tokens whose full blocks have the given
 * chained hashes (pa_block_hashes): the longest run of leading hashes found
 * in the prefix index is reused (touched), stopping so that at least the
 * last token is computed ((hits + 1) * B <= num_tokens - 1); the remaining
 * ceil(num_tokens / B) - hits blocks are new.  Writes the block-table row to
 * block_ids (ceil(num_tokens / B) entries, at most max_blocks) and the
 * number of tokens whose K/V are already cached to *num_cached_tokens.
 * PA_ERR_INVALID_ARG (no change) if the pool cannot supply the new blocks.
 */
int pa_pool_allocate_prompt(pa_block_pool* pool, const uint64_t* hashes, int32_t num_hashes,
                            int32_t num_tokens, int32_t block_size, int32_t* block_ids,
                            int32_t max_blocks, int32_t* num_cached_tokens);

/* After the prompt's K/V are written: cache its full blocks (block_ids[i]
 * holds hashes[i], i < num_hashes; blocks already cached are left alone). */
int pa_pool_commit(pa_block_pool* pool, const int32_t* block_ids, const uint64_t* hashes,
                   int32_t num_hashes);

/* A finished request: free its row tail first (its last block is evicted
 * first, P4 §10). */
int pa_pool_free_request(pa_block_pool* pool, const int32_t* block_ids, int32_t n);

/*
 * Block-table entries for kernels whose block is smaller than the manager's
 * ("vllm 深度解析：一切从 PagedAttention 谈起", BlockTable.map_to_kernel_blocks):
 * a manager block of k kernel blocks (k = manager block size / 16) with id b
 * covers kernel blocks b*k .. b*k + k - 1, so
 *     out[i*k + j] = ids[i]*k + j,   i < n, j < k      (n*k entries).
 * With the pool layout [kernel block][KV head][16][head_dim] a manager block
 * is k consecutive kernel blocks.  Negative ids (padding) stay negative.
 * Returns PA_OK, or PA_ERR_INVALID_ARG for k < 1, a NULL array or an id whose
 * expansion overflows int32.
 */
int pa_map_to_kernel_blocks(const int32_t* ids, int32_t n, int32_t blocks_per_kv_block,
                            int32_t* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H_ */
