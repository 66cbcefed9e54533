/*
 * pa.h -- C ABI of libpa: paged attention over a block-table-addressed KV
 * cache, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow these pages:
 *   [P1] "vLLM 深度解析（二）：PagedAttention 核心机制"
 *   [P2] "第11章 分块预填充与混合批处理"
 *   [P3] "vllm 深度解析：一切从 PagedAttention 谈起"
 *   [P4] "LLM 推理基础与 vLLM 内部机制：KV 缓存、PagedAttention、调度器"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument except `layout`, `bytes_per_pool` and the host
 *    arrays of pa_validate_metadata is a DEVICE pointer owned by the caller;
 *    the library never allocates, frees or retains memory, and keeps no state
 *    besides pa_decode_auto_static's static scratch array (one per device).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it and returns; nothing synchronises the stream.
 *  - Return value: PA_OK (0) on success, a negative pa_status otherwise.
 *    Only host-visible arguments are checked (scalars, NULL pointers, 16-byte
 *    alignment of K/V/Q/output buffers); on any error nothing is launched.
 *  - Device metadata is trusted: block ids outside [0, num_blocks), slots
 *    outside [0, num_blocks*block_size), seq_lens above bt_stride*block_size
 *    or above the host limits (max_seq_len, max_query_len) are undefined
 *    behaviour.  pa_validate_metadata checks host copies of the metadata.
 *  - Block-table entries at or past ceil(seq_len / block_size) are never
 *    read, whatever they hold.
 *
 * KV cache layout (chosen for 64-lane wavefronts; the pages' split
 * x-interleaved K and dim-major V are not used):
 *    k_cache, v_cache : [num_blocks][num_kv_heads][block_size][head_dim]
 *  One (block, KV head) tile is block_size rows of head_dim contiguous
 *  elements.  Element type: bf16 (raw 16-bit patterns) or OCP FP8 E4M3FN codes
 *  (1 byte) with one fp32 scale per tensor, read from device memory.
 *  Slot s (P1 §3.1: slot = physical_block * B + offset) is block s / B, row
 *  s % B of every KV-head tile.
 *
 * Supported: block_size 16, head_dim 64 or 128, num_q_heads a multiple of
 * num_kv_heads (query head h reads KV head h / (num_q_heads/num_kv_heads)).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,  /* NULL / misaligned pointer, bad count or scalar */
  PA_ERR_UNSUPPORTED = -2,  /* head_dim, block_size, dtype or head ratio not built */
  PA_ERR_HIP = -3,          /* a HIP launch failed */
  PA_ERR_METADATA = -4,     /* pa_validate_metadata found an inconsistency */
  PA_ERR_SCRATCH = -5,      /* pa_decode_auto_static: the plan needs more than
                               PA_STATIC_SCRATCH_BYTES of scratch */
};

enum pa_cache_dtype {
  PA_CACHE_BF16 = 0,
  PA_CACHE_FP8_E4M3 = 1,    /* OCP E4M3FN, per-tensor fp32 scale */
};

typedef struct pa_kv_layout {
  int32_t num_blocks;       /* physical blocks in each pool */
  int32_t num_kv_heads;
  int32_t head_dim;         /* 64 or 128 */
  int32_t block_size;       /* 16 */
  int32_t cache_dtype;      /* enum pa_cache_dtype */
} pa_kv_layout;

/* Human-readable name of a status code (static string). */
const char* pa_status_string(int status);

/*
 * Bytes of ONE pool (K or V) for `layout` (P1 §1 and P4 §2: per token the
 * cache holds num_kv_heads * head_dim elements for K and as many for V).
 * Host-only; writes *bytes_per_pool.
 */
int pa_kv_cache_bytes(const pa_kv_layout* layout, size_t* bytes_per_pool);

/*
 * Slot mapping (P1 §3.1 equations and the compute_slot_mapping listing;
 * P3 _compute_slot_mappings_kernel).  For token j of request r, with
 * q_len = query_start_loc[r+1] - query_start_loc[r] and
 * pos = seq_lens[r] - q_len + (j - query_start_loc[r]):
 *     slot_mapping[j] = block_table[r*bt_stride + pos/B] * B + pos % B.
 *  slot_mapping    : int64 [num_tokens]            (output)
 *  block_table     : int32 [num_reqs][bt_stride]
 *  query_start_loc : int32 [num_reqs + 1], query_start_loc[num_reqs] == num_tokens
 *  seq_lens        : int32 [num_reqs], K/V tokens visible this step, new ones included
 */
int pa_compute_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                            int32_t bt_stride, const int32_t* query_start_loc,
                            const int32_t* seq_lens, int32_t num_reqs,
                            int32_t num_tokens, int32_t block_size, void* stream);

/*
 * Scatter new K/V into the cache (P3 PagedAttention.write_to_paged_cache ->
 * reshape_and_cache; P1 §3.1 table: slot_mapping writes the new tokens,
 * block_table reads history).  Writes key[j][g][:] to k_cache slot
 * slot_mapping[j], KV head g (and value likewise).  A negative slot skips
 * token j.  Slots must be distinct.
 *  key, value : bf16 [num_tokens][num_kv_heads][head_dim], contiguous
 *  k_scale, v_scale : device fp32 per-tensor scales; required for
 *    PA_CACHE_FP8_E4M3 layouts, ignored (may be NULL) for bf16
 * bf16 caches receive a bit copy.  FP8 caches receive, per element x, the
 * E4M3FN code nearest to the correctly rounded fp32 quotient x / scale, ties
 * to the even code, saturating at +-448, NaN kept -- the inverse of the read
 * side, which takes code value * scale (P1 §3.2.1: FP8 vectors are converted
 * with the scale; the rounding and saturation are this library's reading).
 */
int pa_reshape_and_cache(const pa_kv_layout* layout, void* k_cache, void* v_cache,
                         const void* key, const void* value, int32_t num_tokens,
                         const int64_t* slot_mapping, const float* k_scale,
                         const float* v_scale, void* stream);

/*
 * Slot mapping and scatter fused into one launch (the two steps above,
 * P1 §3.1 and P3 reshape_and_cache): token j of request r (rows
 * query_start_loc[r] .. query_start_loc[r+1]-1) lands at the slot
 * pa_compute_slot_mapping would give it; its key/value rows are copied
 * there bit for bit.  Requests own contiguous, increasing row ranges.
 *  slot_mapping : int64 [num_tokens] output, or NULL when not wanted
 *  k_scale, v_scale : as pa_reshape_and_cache (FP8 caches are quantised the
 *                     same way)
 */
int pa_reshape_and_cache_varlen(const pa_kv_layout* layout, void* k_cache, void* v_cache,
                                const void* key, const void* value, const int32_t* block_table,
                                int32_t bt_stride, const int32_t* query_start_loc,
                                const int32_t* seq_lens, int32_t num_reqs, int32_t num_tokens,
                                int64_t* slot_mapping, const float* k_scale,
                                const float* v_scale, void* stream);

/*
 * Single-query decode attention (P1 §3.2: block-table walk, QK with GQA,
 * masked tail, softmax, PV; P1 §2.2: exact result via the online-softmax
 * state (m, l, A)).  For request r and query head h (g = h / G):
 *     out[r][h] = softmax_t( scale * <q[r][h], K_r[t][g]> + b_h(t) ) . V_r[t][g],
 * t over 0 .. seq_lens[r]-1, K_r/V_r read through block_table row r, and
 * b_h(t) = alibi_slopes[h] * (t - seq_lens[r] + 1) when slopes are given
 * (the ALiBi term of P1 §3.2.4), else 0.
 * One pass per (request, KV head) -- no temporaries.  seq_lens[r] == 0
 * gives a zero row.
 *  out, q     : bf16 [num_reqs][num_q_heads][head_dim]
 *  max_seq_len: host upper bound of seq_lens (grid sizing only)
 *  scale      : softmax scale, e.g. 1/sqrt(head_dim)
 *  k_scale, v_scale : device fp32 scalars, required for FP8 caches,
 *                     ignored (may be NULL) for bf16
 *  alibi_slopes : device fp32 [num_q_heads], or NULL for no bias
 */
int pa_decode(const pa_kv_layout* layout, void* out, const void* q, int32_t num_reqs,
              int32_t num_q_heads, const void* k_cache, const void* v_cache,
              const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
              int32_t max_seq_len, float scale, const float* k_scale,
              const float* v_scale, const float* alibi_slopes, void* stream);

/*
 * Work-balanced decode: the same result as pa_decode (P1 §2.2, §3.2), with
 * the work split evenly over the GPU instead of one work-group per
 * (request, KV head).  The 16-token blocks of all (request, KV head) units
 * are laid end to end and every wave takes an equal contiguous share;
 * units a wave covers whole are written directly, the others are split-KV
 * pieces merged by the cross-partition formula of P1 §3.2.9 in a second
 * launch.  Suited to batches whose context lengths differ widely.
 *  workspace : device buffer of at least pa_decode_workspace_size() bytes,
 *              16-byte aligned, owned by the caller; its contents on entry
 *              do not matter and calls that overlap on one workspace race
 *  num_reqs  : at most 4096 (PA_ERR_UNSUPPORTED above)
 * Other arguments as pa_decode.
 */
size_t pa_decode_workspace_size(const pa_kv_layout* layout, int32_t num_reqs,
                                int32_t num_q_heads);
int pa_decode_balanced(const pa_kv_layout* layout, void* out, const void* q, int32_t num_reqs,
                       int32_t num_q_heads, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                       int32_t max_seq_len, float scale, const float* k_scale,
                       const float* v_scale, const float* alibi_slopes, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * One decode step with its write: each request's newest token -- position
 * seq_lens[r] - 1, its slot block_table[r][pos / 16] * 16 + pos % 16 (P1
 * §3.1) -- gets key[r] / value[r] written into the pools (P3's
 * reshape_and_cache; FP8 pools quantised as pa_reshape_and_cache does),
 * then pa_decode runs over the contexts that now include it.  Same pools
 * and output as pa_reshape_and_cache with that slot mapping followed by
 * pa_decode.  Where the vector-ALU decode runs with one head chunk per KV
 * head (bf16 caches with GQA groups up to 7, FP8 caches with groups up to
 * 3), the write happens inside the decode's own work-groups (one launch);
 * otherwise it is a launch of its own before the decode.
 *  key, value    : bf16 [num_reqs][num_kv_heads][head_dim], one row per request
 *  slot_mapping  : int64 [num_reqs], written with each request's slot (NULL: not written)
 *  k_cache, v_cache : written (the token's row), then read
 * Other arguments as pa_decode; every seq_len must be >= 1.
 */
int pa_decode_append(const pa_kv_layout* layout, void* out, const void* q, int32_t num_reqs,
                     int32_t num_q_heads, void* k_cache, void* v_cache, const void* key,
                     const void* value, int64_t* slot_mapping, const int32_t* block_table,
                     int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len,
                     float scale, const float* k_scale, const float* v_scale,
                     const float* alibi_slopes, void* stream);

/*
 * Split-KV decode, first stage (P1 §3.2.7 and §3.3, the V2 partitioning).
 * Partition p of request r covers tokens [p*P, min((p+1)*P, seq_len)).
 * For every partition p < ceil(seq_lens[r]/P) and query head h writes
 *     max_logits[i] = max of s_t = scale*<q,k_t> + b_h(t) over the partition
 *                     (natural log units; b_h as in pa_decode)
 *     exp_sums[i]   = sum of exp(s_t - max_logits[i])
 *     tmp_out[i][:] = sum of exp(...) * v / exp_sums[i]   (fp32)
 * with i = (r*num_q_heads + h)*max_num_partitions + p (the pages' V2 index).
 * Other entries are not written.
 *  partition_size : P, a positive multiple of block_size
 *  max_num_partitions : row length of the partial arrays, >= ceil(max_seq_len/P)
 *  tmp_out    : fp32 [num_reqs][num_q_heads][max_num_partitions][head_dim]
 *  max_logits, exp_sums : fp32 [num_reqs][num_q_heads][max_num_partitions]
 */
int pa_decode_partitioned(const pa_kv_layout* layout, const void* q, int32_t num_reqs,
                          int32_t num_q_heads, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int32_t bt_stride,
                          const int32_t* seq_lens, int32_t max_seq_len, float scale,
                          const float* k_scale, const float* v_scale,
                          const float* alibi_slopes, int32_t partition_size,
                          int32_t max_num_partitions,
                          float* tmp_out, float* max_logits, float* exp_sums,
                          void* stream);

/*
 * Split-KV decode over a range of partitions: as pa_decode_partitioned but
 * only partitions p with part_begin <= p < part_end (and p < ceil(seq_len/P))
 * are written; 0 <= part_begin <= part_end <= max_num_partitions.  Calls on
 * disjoint ranges fill one set of partial arrays, merged once by
 * pa_merge_partitions -- the building block of sharding a long context by
 * token range (each device computes its partitions; the partials are
 * gathered; the merge of P1 §3.2.9 is associative).
 */
int pa_decode_partitioned_range(const pa_kv_layout* layout, const void* q, int32_t num_reqs,
                                int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, int32_t bt_stride,
                                const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                const float* k_scale, const float* v_scale,
                                const float* alibi_slopes, int32_t partition_size,
                                int32_t max_num_partitions, int32_t part_begin,
                                int32_t part_end, float* tmp_out, float* max_logits,
                                float* exp_sums, void* stream);

/*
 * Decode for a batch whose requests begin with the same cached blocks
 * (prefix caching: every request maps its first logical blocks onto the
 * same physical blocks, P1 §4.1 and the shared-block figure of P4 §4).  The
 * result is pa_decode's.  The shared prefix is read once per KV head: its
 * key partitions are multiplied into the decode queries of all requests
 * together on the matrix cores (K.Q^T and V^T.P^T over 64-key tiles, each
 * partition's (m, l, O) written as the split-KV partials of P1 §3.2.7);
 * the private tails go through the split-KV decode (partitions from
 * shared_blocks * 16 / partition_size on); pa_merge_partitions' merge
 * (P1 §3.2.9) combines the two.
 *  shared_blocks : leading block-table entries the requests share: request
 *                  0 holds the whole prefix (seq_lens[0] >= 16 *
 *                  shared_blocks) and every other request's entries among
 *                  the first shared_blocks that it uses equal request 0's
 *                  (the caller knows this from its prefix cache; the
 *                  kernels read the prefix through request 0's row).
 *                  shared_blocks * 16 must be a multiple of partition_size
 *                  and <= max_seq_len; other requests may be shorter than
 *                  the prefix.
 *  partition_size: tokens per partition, a multiple of 64
 *  tmp_out, max_logits, exp_sums : caller-owned scratch laid out as for
 *                  pa_decode_partitioned (max_num_partitions >=
 *                  ceil(max_seq_len / partition_size)); overwritten.
 *  out           : bf16 [num_reqs][num_q_heads][head_dim]
 * Other arguments as pa_decode.  Three launches on `stream` (prefix
 * partials, tail partials, merge); calls sharing scratch race.
 */
int pa_decode_shared_prefix(const pa_kv_layout* layout, void* out, const void* q,
                            int32_t num_reqs, int32_t num_q_heads, const void* k_cache,
                            const void* v_cache, const int32_t* block_table, int32_t bt_stride,
                            const int32_t* seq_lens, int32_t max_seq_len, float scale,
                            const float* k_scale, const float* v_scale,
                            const float* alibi_slopes, int32_t shared_blocks,
                            int32_t partition_size, int32_t max_num_partitions, float* tmp_out,
                            float* max_logits, float* exp_sums, void* stream);

/*
 * Split-KV decode, merge stage (P1 §3.2.9 equations):
 *     m = max_j m_j,  L = sum_j l_j e^(m_j - m),
 *     out = sum_j tmp_out_j * l_j e^(m_j - m) / L     -> bf16, round to nearest even
 * over j < ceil(seq_lens[r] / partition_size).  Arguments as in
 * pa_decode_partitioned; out is bf16 [num_reqs][num_q_heads][head_dim].
 */
int pa_merge_partitions(void* out, const float* tmp_out, const float* max_logits,
                        const float* exp_sums, const int32_t* seq_lens, int32_t num_reqs,
                        int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                        int32_t max_num_partitions, void* stream);

/*
 * Choice between the single pass and split-KV for a decode batch (the role
 * of P1 §3.3's V1/V2 condition, whose thresholds were set for NVIDIA SM
 * counts; these were measured on MI355X with equal context lengths,
 * Hq/Hkv 32/8 and 28/4, head_dim 128).  With U = num_reqs * num_kv_heads *
 * ceil(G / 8) work units, L = max_seq_len and w = min(G, 8):
 *     split  iff  U <= 64 and L * w >= 7168,
 *            or   64 < U < 256 and L * w >= 14336;   otherwise single pass.
 *     partition_size = 256 if U * L <= 2^16, 512 if U * L <= 2^17, else 1024.
 * workspace_bytes is what pa_decode_auto needs for the plan (0 for the
 * single pass).  Host-only.
 */
typedef struct pa_decode_plan {
  int32_t split;              /* 0: pa_decode; 1: pa_decode_partitioned + merge */
  int32_t partition_size;
  int32_t max_num_partitions;
  int32_t reserved;
  size_t workspace_bytes;
} pa_decode_plan;

int pa_decode_plan_for(const pa_kv_layout* layout, int32_t num_reqs, int32_t num_q_heads,
                       int32_t max_seq_len, pa_decode_plan* plan);

/*
 * Decode by a plan (pa_decode_plan_for's, or the caller's own): the single
 * pass, or split-KV + merge with tmp_out, max_logits and exp_sums carved
 * from `workspace` (caller-owned device memory, 256-byte aligned, at least
 * plan->workspace_bytes; calls that overlap on one workspace race).
 * Arguments otherwise as pa_decode; the result is the same.
 */
int pa_decode_auto(const pa_kv_layout* layout, void* out, const void* q, int32_t num_reqs,
                   int32_t num_q_heads, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                   int32_t max_seq_len, float scale, const float* k_scale,
                   const float* v_scale, const float* alibi_slopes,
                   const pa_decode_plan* plan, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * pa_decode_auto without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split path's partials (tmp_out,
 * max_logits, exp_sums, laid out as pa_decode_auto carves them) live in a
 * static device array of PA_STATIC_SCRATCH_BYTES inside the library, one
 * per device, held until the process ends; the call allocates nothing.
 * Its device address is looked up on the first call made with a device
 * current.  The result equals pa_decode_auto's.
 *  - A split plan whose workspace_bytes would exceed PA_STATIC_SCRATCH_BYTES
 *    returns PA_ERR_SCRATCH and launches nothing (32 MiB hold, e.g., 8
 *    requests x 32 query heads x 64 partitions of head_dim 128 with room to
 *    spare); single-pass plans need no scratch.
 *  - Every call on one device shares that device's array: calls that
 *    overlap in time on one device (two streams, or two host threads) race.
 *    Calls in order on one stream are safe.  Nothing in the array needs to
 *    start at zero (every partial a merge reads is written first).
 * Arguments as pa_decode_auto, minus workspace and workspace_bytes; the
 * stream must belong to the current device.
 */
#define PA_STATIC_SCRATCH_BYTES (32u * 1024u * 1024u)

int pa_decode_auto_static(const pa_kv_layout* layout, void* out, const void* q,
                          int32_t num_reqs, int32_t num_q_heads, const void* k_cache,
                          const void* v_cache, const int32_t* block_table, int32_t bt_stride,
                          const int32_t* seq_lens, int32_t max_seq_len, float scale,
                          const float* k_scale, const float* v_scale,
                          const float* alibi_slopes, const pa_decode_plan* plan, void* stream);

/*
 * Varlen (chunked) prefill over the paged cache (P2 §11.6: query_start_loc
 * as cu_seqlens_q, seq_lens as seqused_k, block_table for the paged K/V).
 * Request r owns query rows query_start_loc[r] .. query_start_loc[r+1]-1;
 * row i of it sits at position p = seq_lens[r] - q_len + i and attends keys
 * 0 .. p (causal).  With alibi_slopes, key t's score for head h gains
 * alibi_slopes[h] * (t - p) (P1 §3.2.4's decode term, whose query sits at
 * p = seq_len - 1).  Requests with q_len <= 1 take the decode
 * path (P1 §5.2 split_decodes_and_prefills, threshold 1); q_len == 0 writes
 * nothing.  With bf16 caches, GQA groups below 8 and at least a device's
 * worth of decode work-groups, both kinds of rows run in one launch (the
 * prefill tiles and the decode rows share the compute units); otherwise the
 * decode rows, then the prefill rows.  The K/V of this step's tokens must
 * already be in the cache (pa_reshape_and_cache first).
 *  out, q : bf16 [num_tokens][num_q_heads][head_dim]
 *  max_query_len, max_seq_len : host upper bounds (grid sizing only)
 */
int pa_prefill_varlen(const pa_kv_layout* layout, void* out, const void* q,
                      int32_t num_tokens, int32_t num_q_heads, const void* k_cache,
                      const void* v_cache, const int32_t* query_start_loc,
                      const int32_t* seq_lens, const int32_t* block_table,
                      int32_t bt_stride, int32_t num_reqs, int32_t max_query_len,
                      int32_t max_seq_len, float scale, const float* k_scale,
                      const float* v_scale, const float* alibi_slopes, void* stream);

/*
 * Test support: gather the logical K and V of every request through the
 * block table with the same addressing code the attention kernels use
 * (P1 §3.1).  Row cu_seq_lens[r] + t of k_out/v_out is token t of request r.
 *  k_out, v_out : [cu_seq_lens[num_reqs]][num_kv_heads][head_dim], cache dtype
 *  cu_seq_lens  : int32 [num_reqs + 1], prefix sums of seq_lens
 */
int pa_debug_gather_kv(const pa_kv_layout* layout, void* k_out, void* v_out,
                       const void* k_cache, const void* v_cache,
                       const int32_t* block_table, int32_t bt_stride,
                       const int32_t* seq_lens, const int32_t* cu_seq_lens,
                       int32_t num_reqs, int32_t max_seq_len, void* stream);

/*
 * Test support: decode n FP8 E4M3FN codes to fp32 with the conversion the
 * attention kernels use.
 */
int pa_debug_fp8_to_f32(const uint8_t* codes, float* out, int32_t n, void* stream);

/*
 * Test support: decode n FP8 E4M3FN codes to f16 bit patterns with the
 * conversion the decode kernels use for FP8 V rows.
 */
int pa_debug_fp8_to_f16(const uint8_t* codes, uint16_t* out, int32_t n, void* stream);

/*
 * Measurement support (not part of the attention path): read `bytes` (a
 * multiple of 16) of device memory at `src` (16-byte aligned) once, as a
 * grid-strided stream of 16-byte non-temporal loads (eight in flight per
 * thread) by `work_groups` 256-thread work-groups (<= 0: eight per compute
 * unit), enqueued on `stream`.  The caller times it: bytes / time is the
 * device's streaming-read rate, the ceiling the decode kernels' HBM rates
 * are compared with besides the published peak.  sink: one device uint32,
 * written only if some thread's data XOR to 0xffffffff (it keeps the loads
 * from being removed).
 */
int pa_measure_read_stream(const void* src, size_t bytes, uint32_t* sink, int32_t work_groups,
                           void* stream);

/*
 * Host-side check of metadata the kernels trust.  All arrays are HOST
 * pointers.  Checks: query_start_loc starts at 0 and is non-decreasing;
 * 0 <= q_len <= seq_len; seq_len <= bt_stride*block_size; every block-table
 * entry a request can read is in [0, num_blocks); when slot_mapping is not
 * NULL, its non-negative entries are distinct and < num_blocks*block_size.
 * Returns PA_OK or PA_ERR_METADATA (PA_ERR_INVALID_ARG for bad arguments).
 */
int pa_validate_metadata(const int32_t* block_table, int32_t bt_stride,
                         const int32_t* query_start_loc, const int32_t* seq_lens,
                         int32_t num_reqs, const int64_t* slot_mapping,
                         int32_t num_tokens, int32_t num_blocks, int32_t block_size);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
