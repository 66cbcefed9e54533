// C ABI of libpa: host-side validation, grid sizing and launches on the
// caller's stream.  Declarations and argument documentation: include/pa.h.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/pa.h"
#include "pa_launch.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_layout(const pa_kv_layout* L) {
  if (L == nullptr) return PA_ERR_INVALID_ARG;
  if (L->num_blocks <= 0 || L->num_kv_heads <= 0) return PA_ERR_INVALID_ARG;
  if (L->block_size != 16) return PA_ERR_UNSUPPORTED;
  if (L->head_dim != 64 && L->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (L->cache_dtype != PA_CACHE_BF16 && L->cache_dtype != PA_CACHE_FP8_E4M3)
    return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int check_heads(const pa_kv_layout* L, int32_t num_q_heads) {
  if (num_q_heads <= 0) return PA_ERR_INVALID_ARG;
  if (num_q_heads % L->num_kv_heads != 0) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int check_scales(const pa_kv_layout* L, float scale, const float* k_scale,
                 const float* v_scale) {
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (L->cache_dtype == PA_CACHE_FP8_E4M3 && (k_scale == nullptr || v_scale == nullptr))
    return PA_ERR_INVALID_ARG;
  return PA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

#define PA_TRY(x)            \
  do {                       \
    const int s_ = (x);      \
    if (s_ != PA_OK) return s_; \
  } while (0)

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_HIP: return "HIP launch error";
    case PA_ERR_METADATA: return "inconsistent metadata";
    case PA_ERR_SCRATCH: return "more scratch memory needed than the static buffer holds";
    default: return "unknown status";
  }
}

int pa_kv_cache_bytes(const pa_kv_layout* layout, size_t* bytes_per_pool) {
  PA_TRY(check_layout(layout));
  if (bytes_per_pool == nullptr) return PA_ERR_INVALID_ARG;
  const size_t eb = layout->cache_dtype == PA_CACHE_BF16 ? 2 : 1;
  *bytes_per_pool = (size_t)layout->num_blocks * layout->num_kv_heads * layout->block_size *
                    layout->head_dim * eb;
  return PA_OK;
}

int pa_compute_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                            int32_t bt_stride, const int32_t* query_start_loc,
                            const int32_t* seq_lens, int32_t num_reqs, int32_t num_tokens,
                            int32_t block_size, void* stream) {
  if (num_reqs < 0 || num_tokens < 0 || bt_stride <= 0) return PA_ERR_INVALID_ARG;
  if (block_size != 16) return PA_ERR_UNSUPPORTED;
  if (num_reqs == 0) return PA_OK;
  if (!block_table || !query_start_loc || !seq_lens) return PA_ERR_INVALID_ARG;
  if (num_tokens > 0 && !slot_mapping) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_slot_mapping(slot_mapping, block_table, bt_stride,
                                            query_start_loc, seq_lens, num_reqs, num_tokens,
                                            (hipStream_t)stream));
}

int pa_reshape_and_cache(const pa_kv_layout* layout, void* k_cache, void* v_cache,
                         const void* key, const void* value, int32_t num_tokens,
                         const int64_t* slot_mapping, const float* k_scale,
                         const float* v_scale, void* stream) {
  PA_TRY(check_layout(layout));
  PA_TRY(check_scales(layout, 1.f, k_scale, v_scale));
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || !key || !value || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(key) || !aligned16(value))
    return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_reshape_and_cache(
      k_cache, v_cache, key, value, num_tokens, slot_mapping, layout->num_kv_heads,
      layout->head_dim, layout->cache_dtype == PA_CACHE_FP8_E4M3, k_scale, v_scale,
      (hipStream_t)stream));
}

int pa_reshape_and_cache_varlen(const pa_kv_layout* layout, void* k_cache, void* v_cache,
                                const void* key, const void* value, const int32_t* block_table,
                                int32_t bt_stride, const int32_t* query_start_loc,
                                const int32_t* seq_lens, int32_t num_reqs, int32_t num_tokens,
                                int64_t* slot_mapping, const float* k_scale,
                                const float* v_scale, void* stream) {
  PA_TRY(check_layout(layout));
  PA_TRY(check_scales(layout, 1.f, k_scale, v_scale));
  if (num_tokens < 0 || num_reqs < 0 || bt_stride <= 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0 || num_reqs == 0) return PA_OK;
  if (!k_cache || !v_cache || !key || !value || !block_table || !query_start_loc || !seq_lens)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(key) || !aligned16(value))
    return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_reshape_and_cache_varlen(
      k_cache, v_cache, key, value, block_table, bt_stride, query_start_loc, seq_lens, num_reqs,
      num_tokens, layout->num_kv_heads, layout->head_dim, slot_mapping,
      layout->cache_dtype == PA_CACHE_FP8_E4M3, k_scale, v_scale, (hipStream_t)stream));
}

static int decode_common(const pa_kv_layout* layout, const void* q, int32_t num_reqs,
                         int32_t num_q_heads, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, int32_t bt_stride,
                         const int32_t* seq_lens, int32_t max_seq_len, float scale,
                         const float* k_scale, const float* v_scale) {
  PA_TRY(check_layout(layout));
  PA_TRY(check_heads(layout, num_q_heads));
  PA_TRY(check_scales(layout, scale, k_scale, v_scale));
  if (num_reqs < 0 || max_seq_len < 0 || bt_stride <= 0) return PA_ERR_INVALID_ARG;
  if ((int64_t)max_seq_len > (int64_t)bt_stride * layout->block_size) return PA_ERR_INVALID_ARG;
  if (num_reqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens) return PA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

static pa::DecodeArgs decode_args(const pa_kv_layout* layout, const void* q, int32_t num_reqs,
                                  int32_t num_q_heads, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  int32_t bt_stride, const int32_t* seq_lens,
                                  int32_t max_seq_len, float scale, const float* k_scale,
                                  const float* v_scale, const float* alibi_slopes) {
  pa::DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.query_start_loc = nullptr;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.alibi_slopes = alibi_slopes;
  a.num_reqs = num_reqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = layout->num_kv_heads;
  a.head_dim = layout->head_dim;
  a.cache_dtype = layout->cache_dtype;
  a.bt_stride = bt_stride;
  a.max_seq_len = max_seq_len;
  a.scale = scale;
  return a;
}

int pa_decode(const pa_kv_layout* layout, void* out, const void* q, int32_t num_reqs,
              int32_t num_q_heads, const void* k_cache, const void* v_cache,
              const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
              int32_t max_seq_len, float scale, const float* k_scale, const float* v_scale,
              const float* alibi_slopes, void* stream) {
  PA_TRY(decode_common(layout, q, num_reqs, num_q_heads, k_cache, v_cache, block_table,
                       bt_stride, seq_lens, max_seq_len, scale, k_scale, v_scale));
  if (num_reqs == 0) return PA_OK;
  if (!out || !aligned16(out)) return PA_ERR_INVALID_ARG;
  pa::DecodeArgs a = decode_args(layout, q, num_reqs, num_q_heads, k_cache, v_cache,
                                 block_table, bt_stride, seq_lens, max_seq_len, scale,
                                 k_scale, v_scale, alibi_slopes);
  a.out = out;
  return hip_status(pa::launch_decode(a, false, (hipStream_t)stream));
}

size_t pa_decode_workspace_size(const pa_kv_layout* layout, int32_t num_reqs,
                                int32_t num_q_heads) {
  if (check_layout(layout) != PA_OK || check_heads(layout, num_q_heads) != PA_OK || num_reqs < 0)
    return 0;
  return (size_t)pa::balanced_workspace_bytes(num_reqs, num_q_heads, layout->num_kv_heads,
                                              layout->head_dim);
}

int pa_decode_balanced(const pa_kv_layout* layout, void* out, const void* q, int32_t num_reqs,
                       int32_t num_q_heads, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                       int32_t max_seq_len, float scale, const float* k_scale,
                       const float* v_scale, const float* alibi_slopes, void* workspace,
                       size_t workspace_bytes, void* stream) {
  PA_TRY(decode_common(layout, q, num_reqs, num_q_heads, k_cache, v_cache, block_table,
                       bt_stride, seq_lens, max_seq_len, scale, k_scale, v_scale));
  if (num_reqs == 0) return PA_OK;
  if (!out || !aligned16(out)) return PA_ERR_INVALID_ARG;
  if (num_reqs > pa::balanced_max_reqs()) return PA_ERR_UNSUPPORTED;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < pa_decode_workspace_size(layout, num_reqs, num_q_heads))
    return PA_ERR_INVALID_ARG;
  pa::DecodeArgs a = decode_args(layout, q, num_reqs, num_q_heads, k_cache, v_cache,
                                 block_table, bt_stride, seq_lens, max_seq_len, scale,
                                 k_scale, v_scale, alibi_slopes);
  a.out = out;
  return hip_status(pa::launch_decode_balanced(a, workspace, (hipStream_t)stream));
}

int pa_decode_append(const pa_kv_layout* layout, void* out, const void* q, int32_t num_reqs,
                     int32_t num_q_heads, void* k_cache, void* v_cache, const void* key,
                     const void* value, int64_t* slot_mapping, const int32_t* block_table,
                     int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len,
                     float scale, const float* k_scale, const float* v_scale,
                     const float* alibi_slopes, void* stream) {
  PA_TRY(decode_common(layout, q, num_reqs, num_q_heads, k_cache, v_cache, block_table,
                       bt_stride, seq_lens, max_seq_len, scale, k_scale, v_scale));
  if (num_reqs == 0) return PA_OK;
  if (!out || !aligned16(out) || !key || !value || !aligned16(key) || !aligned16(value))
    return PA_ERR_INVALID_ARG;
  pa::DecodeArgs a = decode_args(layout, q, num_reqs, num_q_heads, k_cache, v_cache,
                                 block_table, bt_stride, seq_lens, max_seq_len, scale, k_scale,
                                 v_scale, alibi_slopes);
  a.out = out;
  a.new_k = key;
  a.new_v = value;
  a.slot_out = slot_mapping;
  return hip_status(pa::launch_decode_append(a, (hipStream_t)stream));
}

int pa_decode_partitioned(const pa_kv_layout* layout, const void* q, int32_t num_reqs,
                          int32_t num_q_heads, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int32_t bt_stride,
                          const int32_t* seq_lens, int32_t max_seq_len, float scale,
                          const float* k_scale, const float* v_scale,
                          const float* alibi_slopes, int32_t partition_size,
                          int32_t max_num_partitions, float* tmp_out, float* max_logits,
                          float* exp_sums, void* stream) {
  PA_TRY(decode_common(layout, q, num_reqs, num_q_heads, k_cache, v_cache, block_table,
                       bt_stride, seq_lens, max_seq_len, scale, k_scale, v_scale));
  if (partition_size <= 0 || partition_size % layout->block_size != 0)
    return PA_ERR_INVALID_ARG;
  const int64_t need = ((int64_t)max_seq_len + partition_size - 1) / partition_size;
  if (max_num_partitions < 1 || max_num_partitions < need) return PA_ERR_INVALID_ARG;
  if (num_reqs == 0) return PA_OK;
  if (!tmp_out || !max_logits || !exp_sums || !aligned16(tmp_out)) return PA_ERR_INVALID_ARG;
  pa::DecodeArgs a = decode_args(layout, q, num_reqs, num_q_heads, k_cache, v_cache,
                                 block_table, bt_stride, seq_lens, max_seq_len, scale,
                                 k_scale, v_scale, alibi_slopes);
  a.tmp_out = tmp_out;
  a.max_logits = max_logits;
  a.exp_sums = exp_sums;
  a.partition_size = partition_size;
  a.max_num_partitions = max_num_partitions;
  return hip_status(pa::launch_decode(a, true, (hipStream_t)stream));
}

int pa_decode_partitioned_range(const pa_kv_layout* layout, const void* q, int32_t num_reqs,
                                int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, int32_t bt_stride,
                                const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                const float* k_scale, const float* v_scale,
                                const float* alibi_slopes, int32_t partition_size,
                                int32_t max_num_partitions, int32_t part_begin,
                                int32_t part_end, float* tmp_out, float* max_logits,
                                float* exp_sums, void* stream) {
  PA_TRY(decode_common(layout, q, num_reqs, num_q_heads, k_cache, v_cache, block_table,
                       bt_stride, seq_lens, max_seq_len, scale, k_scale, v_scale));
  if (partition_size <= 0 || partition_size % layout->block_size != 0)
    return PA_ERR_INVALID_ARG;
  const int64_t need = ((int64_t)max_seq_len + partition_size - 1) / partition_size;
  if (max_num_partitions < 1 || max_num_partitions < need) return PA_ERR_INVALID_ARG;
  if (part_begin < 0 || part_end < part_begin || part_end > max_num_partitions)
    return PA_ERR_INVALID_ARG;
  if (num_reqs == 0 || part_end == part_begin) return PA_OK;
  if (!tmp_out || !max_logits || !exp_sums || !aligned16(tmp_out)) return PA_ERR_INVALID_ARG;
  pa::DecodeArgs a = decode_args(layout, q, num_reqs, num_q_heads, k_cache, v_cache,
                                 block_table, bt_stride, seq_lens, max_seq_len, scale,
                                 k_scale, v_scale, alibi_slopes);
  a.tmp_out = tmp_out;
  a.max_logits = max_logits;
  a.exp_sums = exp_sums;
  a.partition_size = partition_size;
  a.max_num_partitions = max_num_partitions;
  a.part_begin = part_begin;
  a.part_end = part_end;
  return hip_status(pa::launch_decode(a, true, (hipStream_t)stream));
}

int pa_decode_shared_prefix(const pa_kv_layout* layout, void* out, const void* q,
                            int32_t num_reqs, int32_t num_q_heads, const void* k_cache,
                            const void* v_cache, const int32_t* block_table, int32_t bt_stride,
                            const int32_t* seq_lens, int32_t max_seq_len, float scale,
                            const float* k_scale, const float* v_scale,
                            const float* alibi_slopes, int32_t shared_blocks,
                            int32_t partition_size, int32_t max_num_partitions, float* tmp_out,
                            float* max_logits, float* exp_sums, void* stream) {
  PA_TRY(decode_common(layout, q, num_reqs, num_q_heads, k_cache, v_cache, block_table,
                       bt_stride, seq_lens, max_seq_len, scale, k_scale, v_scale));
  if (partition_size <= 0 || partition_size % 64 != 0 || shared_blocks < 0)
    return PA_ERR_INVALID_ARG;
  const int64_t shared_tokens = (int64_t)shared_blocks * layout->block_size;
  if (shared_tokens % partition_size != 0 || shared_tokens > max_seq_len)
    return PA_ERR_INVALID_ARG;
  const int64_t need = ((int64_t)max_seq_len + partition_size - 1) / partition_size;
  if (max_num_partitions < 1 || max_num_partitions < need) return PA_ERR_INVALID_ARG;
  if (num_reqs == 0) return PA_OK;
  if (!out || !aligned16(out) || !tmp_out || !max_logits || !exp_sums || !aligned16(tmp_out))
    return PA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (shared_tokens > 0) {
    pa::PrefillArgs p;
    memset(&p, 0, sizeof(p));
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.seq_lens = seq_lens;
    p.block_table = block_table;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.alibi_slopes = alibi_slopes;
    p.num_reqs = num_reqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = layout->num_kv_heads;
    p.head_dim = layout->head_dim;
    p.cache_dtype = layout->cache_dtype;
    p.bt_stride = bt_stride;
    p.max_seq_len = max_seq_len;
    p.scale = scale;
    p.tmp_out = tmp_out;
    p.max_logits = max_logits;
    p.exp_sums = exp_sums;
    p.partition_size = partition_size;
    p.max_num_partitions = max_num_partitions;
    p.shared_tokens = (int32_t)shared_tokens;
    PA_TRY(hip_status(pa::launch_shared_prefix(p, st)));
  }
  // the private tails: one open-ended record per request (partition
  // first_tail, tokens shared_tokens .. seq_len), merged with the prefix's
  const int32_t first_tail = (int32_t)(shared_tokens / partition_size);
  if (first_tail < need) {
    pa::DecodeArgs a = decode_args(layout, q, num_reqs, num_q_heads, k_cache, v_cache,
                                   block_table, bt_stride, seq_lens, max_seq_len, scale,
                                   k_scale, v_scale, alibi_slopes);
    a.tmp_out = tmp_out;
    a.max_logits = max_logits;
    a.exp_sums = exp_sums;
    a.partition_size = partition_size;
    a.max_num_partitions = max_num_partitions;
    a.part_begin = first_tail;
    a.part_end = first_tail + 1;
    a.open_last = 1;
    PA_TRY(hip_status(pa::launch_decode(a, true, st)));
  }
  return hip_status(pa::launch_merge(out, tmp_out, max_logits, exp_sums, seq_lens, num_reqs,
                                     num_q_heads, layout->head_dim, partition_size,
                                     max_num_partitions, st, first_tail + 1));
}

int pa_merge_partitions(void* out, const float* tmp_out, const float* max_logits,
                        const float* exp_sums, const int32_t* seq_lens, int32_t num_reqs,
                        int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                        int32_t max_num_partitions, void* stream) {
  if (num_reqs < 0 || num_q_heads <= 0 || partition_size <= 0 || max_num_partitions < 1)
    return PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_reqs == 0) return PA_OK;
  if (!out || !tmp_out || !max_logits || !exp_sums || !seq_lens) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_merge(out, tmp_out, max_logits, exp_sums, seq_lens, num_reqs,
                                     num_q_heads, head_dim, partition_size,
                                     max_num_partitions, (hipStream_t)stream));
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static size_t split_workspace_bytes(int32_t num_reqs, int32_t num_q_heads, int32_t head_dim,
                                    int32_t max_num_partitions) {
  const size_t rows = (size_t)num_reqs * num_q_heads * max_num_partitions;
  return align256(rows * head_dim * 4) + 2 * align256(rows * 4);
}

int pa_decode_plan_for(const pa_kv_layout* layout, int32_t num_reqs, int32_t num_q_heads,
                       int32_t max_seq_len, pa_decode_plan* plan) {
  PA_TRY(check_layout(layout));
  PA_TRY(check_heads(layout, num_q_heads));
  if (num_reqs < 0 || max_seq_len < 0 || !plan) return PA_ERR_INVALID_ARG;
  const int64_t G = num_q_heads / layout->num_kv_heads;
  const int64_t units = (int64_t)num_reqs * layout->num_kv_heads * ((G + 7) / 8);
  const int64_t L = max_seq_len, w = G < 8 ? G : 8;
  memset(plan, 0, sizeof(*plan));
  plan->split = ((units <= 64 && L * w >= 7168) || (units > 64 && units < 256 && L * w >= 14336))
                    ? 1 : 0;
  const int64_t work = units * L;
  plan->partition_size = work <= (1 << 16) ? 256 : work <= (1 << 17) ? 512 : 1024;
  plan->max_num_partitions = (int32_t)std::max<int64_t>(
      1, (L + plan->partition_size - 1) / plan->partition_size);
  plan->workspace_bytes = plan->split ? split_workspace_bytes(num_reqs, num_q_heads,
                                                              layout->head_dim,
                                                              plan->max_num_partitions)
                                      : 0;
  return PA_OK;
}

}  // extern "C"

// The split path of a decode plan with its partials carved from `workspace`
// (checked by the callers).
static int decode_split_in(const pa_kv_layout* layout, void* out, const void* q,
                           int32_t num_reqs, int32_t num_q_heads, const void* k_cache,
                           const void* v_cache, const int32_t* block_table, int32_t bt_stride,
                           const int32_t* seq_lens, int32_t max_seq_len, float scale,
                           const float* k_scale, const float* v_scale,
                           const float* alibi_slopes, const pa_decode_plan* plan,
                           void* workspace, void* stream) {
  const size_t rows = (size_t)num_reqs * num_q_heads * plan->max_num_partitions;
  char* base = reinterpret_cast<char*>(workspace);
  float* tmp = reinterpret_cast<float*>(base);
  float* ml = reinterpret_cast<float*>(base + align256(rows * layout->head_dim * 4));
  float* es = reinterpret_cast<float*>(base + align256(rows * layout->head_dim * 4) +
                                       align256(rows * 4));
  PA_TRY(pa_decode_partitioned(layout, q, num_reqs, num_q_heads, k_cache, v_cache, block_table,
                               bt_stride, seq_lens, max_seq_len, scale, k_scale, v_scale,
                               alibi_slopes, plan->partition_size, plan->max_num_partitions, tmp,
                               ml, es, stream));
  return pa_merge_partitions(out, tmp, ml, es, seq_lens, num_reqs, num_q_heads,
                             layout->head_dim, plan->partition_size, plan->max_num_partitions,
                             stream);
}

// Device memory of pa_decode_auto_static: the split-KV partials of a plan
// live here instead of in a caller's workspace.  Every device the library
// runs on holds its own copy, for the life of the process.  In host code
// `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, once per device (scratch_address).
static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call made with that device current, then kept).
int scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode_auto(const pa_kv_layout* layout, void* out, const void* q, int32_t num_reqs,
                   int32_t num_q_heads, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                   int32_t max_seq_len, float scale, const float* k_scale, const float* v_scale,
                   const float* alibi_slopes, const pa_decode_plan* plan, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!plan) return PA_ERR_INVALID_ARG;
  if (!plan->split)
    return pa_decode(layout, out, q, num_reqs, num_q_heads, k_cache, v_cache, block_table,
                     bt_stride, seq_lens, max_seq_len, scale, k_scale, v_scale, alibi_slopes,
                     stream);
  PA_TRY(check_layout(layout));
  if (num_reqs == 0) return PA_OK;
  if (num_reqs < 0 || num_q_heads <= 0 || plan->max_num_partitions <= 0)
    return PA_ERR_INVALID_ARG;
  const size_t need = split_workspace_bytes(num_reqs, num_q_heads, layout->head_dim,
                                            plan->max_num_partitions);
  if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < need ||
      !out || !aligned16(out))
    return PA_ERR_INVALID_ARG;
  return decode_split_in(layout, out, q, num_reqs, num_q_heads, k_cache, v_cache, block_table,
                         bt_stride, seq_lens, max_seq_len, scale, k_scale, v_scale,
                         alibi_slopes, plan, workspace, stream);
}

int pa_decode_auto_static(const pa_kv_layout* layout, void* out, const void* q,
                          int32_t num_reqs, int32_t num_q_heads, const void* k_cache,
                          const void* v_cache, const int32_t* block_table, int32_t bt_stride,
                          const int32_t* seq_lens, int32_t max_seq_len, float scale,
                          const float* k_scale, const float* v_scale,
                          const float* alibi_slopes, const pa_decode_plan* plan, void* stream) {
  if (!plan) return PA_ERR_INVALID_ARG;
  if (!plan->split)
    return pa_decode(layout, out, q, num_reqs, num_q_heads, k_cache, v_cache, block_table,
                     bt_stride, seq_lens, max_seq_len, scale, k_scale, v_scale, alibi_slopes,
                     stream);
  PA_TRY(check_layout(layout));
  if (num_reqs == 0) return PA_OK;
  if (num_reqs < 0 || num_q_heads <= 0 || plan->max_num_partitions <= 0)
    return PA_ERR_INVALID_ARG;
  if (!out || !aligned16(out)) return PA_ERR_INVALID_ARG;
  const size_t need = split_workspace_bytes(num_reqs, num_q_heads, layout->head_dim,
                                            plan->max_num_partitions);
  if (need > (size_t)PA_STATIC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
  void* ws = nullptr;
  PA_TRY(scratch_address(&ws));
  return decode_split_in(layout, out, q, num_reqs, num_q_heads, k_cache, v_cache, block_table,
                         bt_stride, seq_lens, max_seq_len, scale, k_scale, v_scale,
                         alibi_slopes, plan, ws, stream);
}

int pa_prefill_varlen(const pa_kv_layout* layout, void* out, const void* q, int32_t num_tokens,
                      int32_t num_q_heads, const void* k_cache, const void* v_cache,
                      const int32_t* query_start_loc, const int32_t* seq_lens,
                      const int32_t* block_table, int32_t bt_stride, int32_t num_reqs,
                      int32_t max_query_len, int32_t max_seq_len, float scale,
                      const float* k_scale, const float* v_scale, const float* alibi_slopes,
                      void* stream) {
  PA_TRY(decode_common(layout, q, num_reqs, num_q_heads, k_cache, v_cache, block_table,
                       bt_stride, seq_lens, max_seq_len, scale, k_scale, v_scale));
  if (num_tokens < 0 || max_query_len < 0 || max_query_len > max_seq_len)
    return PA_ERR_INVALID_ARG;
  if (num_reqs == 0 || num_tokens == 0) return PA_OK;
  if (!out || !aligned16(out) || !query_start_loc) return PA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  // decode-like rows (q_len == 1): the decode kernel, one pass per KV head
  pa::DecodeArgs a = decode_args(layout, q, num_reqs, num_q_heads, k_cache, v_cache,
                                 block_table, bt_stride, seq_lens, max_seq_len, scale,
                                 k_scale, v_scale, alibi_slopes);
  a.out = out;
  a.query_start_loc = query_start_loc;
  pa::PrefillArgs p;
  memset(&p, 0, sizeof(p));
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.query_start_loc = query_start_loc;
  p.seq_lens = seq_lens;
  p.block_table = block_table;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.alibi_slopes = alibi_slopes;
  p.out = out;
  p.num_reqs = num_reqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = layout->num_kv_heads;
  p.head_dim = layout->head_dim;
  p.cache_dtype = layout->cache_dtype;
  p.bt_stride = bt_stride;
  p.num_tokens = num_tokens;
  p.max_query_len = max_query_len;
  p.max_seq_len = max_seq_len;
  p.scale = scale;
  // both kinds of rows in one launch where that applies, else the decode
  // rows and then the prefill rows
  if (pa::varlen_fused_applies(p)) return hip_status(pa::launch_varlen(p, a, st));
  PA_TRY(hip_status(pa::launch_decode(a, false, st)));
  if (max_query_len <= 1) return PA_OK;
  return hip_status(pa::launch_prefill(p, st));
}

int pa_debug_gather_kv(const pa_kv_layout* layout, void* k_out, void* v_out,
                       const void* k_cache, const void* v_cache, const int32_t* block_table,
                       int32_t bt_stride, const int32_t* seq_lens, const int32_t* cu_seq_lens,
                       int32_t num_reqs, int32_t max_seq_len, void* stream) {
  PA_TRY(check_layout(layout));
  if (num_reqs < 0 || max_seq_len < 0 || bt_stride <= 0) return PA_ERR_INVALID_ARG;
  if ((int64_t)max_seq_len > (int64_t)bt_stride * layout->block_size) return PA_ERR_INVALID_ARG;
  if (num_reqs == 0 || max_seq_len == 0) return PA_OK;
  if (!k_out || !v_out || !k_cache || !v_cache || !block_table || !seq_lens || !cu_seq_lens)
    return PA_ERR_INVALID_ARG;
  const int eb = layout->cache_dtype == PA_CACHE_BF16 ? 2 : 1;
  return hip_status(pa::launch_gather_kv(k_out, v_out, k_cache, v_cache, block_table,
                                         bt_stride, seq_lens, cu_seq_lens, num_reqs,
                                         max_seq_len, layout->num_kv_heads, layout->head_dim,
                                         eb, (hipStream_t)stream));
}

int pa_debug_fp8_to_f32(const uint8_t* codes, float* out, int32_t n, void* stream) {
  if (n < 0) return PA_ERR_INVALID_ARG;
  if (n == 0) return PA_OK;
  if (!codes || !out) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_fp8_to_f32(codes, out, n, (hipStream_t)stream));
}

int pa_debug_fp8_to_f16(const uint8_t* codes, uint16_t* out, int32_t n, void* stream) {
  if (n < 0) return PA_ERR_INVALID_ARG;
  if (n == 0) return PA_OK;
  if (!codes || !out) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_fp8_to_f16(codes, out, n, (hipStream_t)stream));
}

int pa_measure_read_stream(const void* src, size_t bytes, uint32_t* sink, int32_t work_groups,
                           void* stream) {
  if (bytes == 0) return PA_OK;
  if (!src || !sink || !aligned16(src) || bytes % 16 != 0) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_read_stream(src, (int64_t)bytes, sink, work_groups,
                                           (hipStream_t)stream));
}

int pa_validate_metadata(const int32_t* block_table, int32_t bt_stride,
                         const int32_t* query_start_loc, const int32_t* seq_lens,
                         int32_t num_reqs, const int64_t* slot_mapping, int32_t num_tokens,
                         int32_t num_blocks, int32_t block_size) {
  if (num_reqs < 0 || bt_stride <= 0 || num_blocks <= 0 || block_size <= 0 || num_tokens < 0)
    return PA_ERR_INVALID_ARG;
  if (num_reqs > 0 && (!block_table || !seq_lens)) return PA_ERR_INVALID_ARG;
  if (query_start_loc) {
    if (query_start_loc[0] != 0) return PA_ERR_METADATA;
    for (int r = 0; r < num_reqs; ++r)
      if (query_start_loc[r + 1] < query_start_loc[r]) return PA_ERR_METADATA;
  }
  for (int r = 0; r < num_reqs; ++r) {
    const int64_t n = seq_lens[r];
    if (n < 0 || n > (int64_t)bt_stride * block_size) return PA_ERR_METADATA;
    if (query_start_loc && query_start_loc[r + 1] - query_start_loc[r] > n) return PA_ERR_METADATA;
    const int64_t nb = (n + block_size - 1) / block_size;
    for (int64_t b = 0; b < nb; ++b) {
      const int32_t id = block_table[(int64_t)r * bt_stride + b];
      if (id < 0 || id >= num_blocks) return PA_ERR_METADATA;
    }
  }
  if (slot_mapping && num_tokens > 0) {
    const int64_t limit = (int64_t)num_blocks * block_size;
    std::vector<char> seen((size_t)limit, 0);
    for (int j = 0; j < num_tokens; ++j) {
      const int64_t s = slot_mapping[j];
      if (s < 0) continue;
      if (s >= limit || seen[(size_t)s]) return PA_ERR_METADATA;
      seen[(size_t)s] = 1;
    }
  }
  return PA_OK;
}

}  // extern "C"
