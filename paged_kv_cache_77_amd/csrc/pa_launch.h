// Kernel launchers of libpa (internal; the C ABI in pa_api.hip validates
// arguments and calls these).  Each returns a hipError_t from the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct DecodeArgs {
  const void* q;             // bf16 rows
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* query_start_loc;   // NULL: q/out row r is request r
  const float* k_scale;             // NULL for bf16 caches
  const float* v_scale;
  const float* alibi_slopes;        // fp32 [num_q_heads] or NULL (no bias)
  void* out;                        // bf16, final output (NULL in partitioned mode)
  const void* new_k;                // append mode: this step's K/V rows [R][Hkv][D] bf16,
  const void* new_v;                //   written at position seq_len - 1 before decoding
  int64_t* slot_out;                // append mode: each request's slot (or NULL)
  float* tmp_out;                   // partitioned mode only
  float* max_logits;
  float* exp_sums;
  int32_t num_reqs, num_q_heads, num_kv_heads, head_dim, cache_dtype;
  int32_t bt_stride;
  int32_t max_seq_len;
  int32_t partition_size;           // tokens per partition (partitioned mode)
  int32_t max_num_partitions;
  int32_t part_begin, part_end;     // partitioned mode: partitions written (end 0 = all)
  int32_t open_last;                // partition part_end - 1 runs to seq_len (a tail record)
  int32_t lpt;                      // set by the launcher: longest requests first
  int32_t lpt_half;                 // set by the launcher: > 0 pairs ranks (see decode_kernel)
  int32_t xcd_items;                // set by the launcher (split-KV): > 0 = 1-D grid of that many
  int32_t xcd_even, xcd_odd;        //   items, xcd_even per even XCD, xcd_odd per odd one
  float scale;
};

hipError_t launch_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                               int32_t bt_stride, const int32_t* query_start_loc,
                               const int32_t* seq_lens, int32_t num_reqs,
                               int32_t max_query_len_hint, hipStream_t stream);

hipError_t launch_reshape_and_cache(void* k_cache, void* v_cache, const void* key,
                                    const void* value, int32_t num_tokens,
                                    const int64_t* slot_mapping, int32_t num_kv_heads,
                                    int32_t head_dim, bool fp8, const float* k_scale,
                                    const float* v_scale, hipStream_t stream);

// Each request's newest token (position seq_len - 1) from key/value [R][Hkv][D]
// bf16 into the pools at its slot (quantised for FP8 pools); slot_out[r]
// gets the slot when given.  One work-group per request.
hipError_t launch_append_rows(void* k_cache, void* v_cache, const void* key, const void* value,
                              const int32_t* block_table, int32_t bt_stride,
                              const int32_t* seq_lens, int32_t num_reqs, int32_t num_kv_heads,
                              int32_t head_dim, int64_t* slot_out, bool fp8,
                              const float* k_scale, const float* v_scale, hipStream_t stream);

// Decode with the append: the newest token's K/V written first (in the
// decode kernel's own work-groups where the path allows, else one more
// launch before it).
hipError_t launch_decode_append(const DecodeArgs& args, hipStream_t stream);

hipError_t launch_reshape_and_cache_varlen(void* k_cache, void* v_cache, const void* key,
                                           const void* value, const int32_t* block_table,
                                           int32_t bt_stride, const int32_t* query_start_loc,
                                           const int32_t* seq_lens, int32_t num_reqs,
                                           int32_t num_tokens, int32_t num_kv_heads,
                                           int32_t head_dim, int64_t* slot_mapping, bool fp8,
                                           const float* k_scale, const float* v_scale,
                                           hipStream_t stream);

hipError_t launch_gather_kv(void* k_out, void* v_out, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            int32_t bt_stride, const int32_t* seq_lens,
                            const int32_t* cu_seq_lens, int32_t num_reqs,
                            int32_t max_seq_len, int32_t num_kv_heads, int32_t head_dim,
                            int32_t elem_bytes, hipStream_t stream);

hipError_t launch_fp8_to_f32(const uint8_t* codes, float* out, int32_t n,
                             hipStream_t stream);
// One streaming read of `bytes` at src (measurement support).
hipError_t launch_read_stream(const void* src, int64_t bytes, uint32_t* sink, int32_t work_groups,
                              hipStream_t stream);

hipError_t launch_fp8_to_f16(const uint8_t* codes, uint16_t* out, int32_t n,
                             hipStream_t stream);

// Decode: partitioned == false writes args.out directly (one pass per
// request and KV head); true writes the partials.
hipError_t launch_decode(const DecodeArgs& args, bool partitioned, hipStream_t stream);

// FP8-cache decode on the matrix cores (same outputs and partials as
// launch_decode); used by launch_decode for FP8 caches with G >= 4.
hipError_t launch_decode_mfma(const DecodeArgs& args, bool partitioned, hipStream_t stream);

// Work-balanced decode (output as launch_decode's single pass) and its
// workspace size in bytes; at most balanced_max_reqs() requests.
hipError_t launch_decode_balanced(const DecodeArgs& args, void* workspace, hipStream_t stream);
int64_t balanced_workspace_bytes(int num_reqs, int num_q_heads, int num_kv_heads, int head_dim);
int balanced_max_reqs();

// max_used > 0: at most that many partitions per request are merged (the
// last one may be an open-ended tail record); 0: ceil(seq_len / P).
hipError_t launch_merge(void* out, const float* tmp_out, const float* max_logits,
                        const float* exp_sums, const int32_t* seq_lens, int32_t num_reqs,
                        int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                        int32_t max_num_partitions, hipStream_t stream, int32_t max_used = 0);

struct PrefillArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* query_start_loc;
  const int32_t* seq_lens;
  const int32_t* block_table;
  const float* k_scale;
  const float* v_scale;
  const float* alibi_slopes;        // fp32 [num_q_heads] or NULL (no bias)
  void* out;
  int32_t num_reqs, num_q_heads, num_kv_heads, head_dim, cache_dtype;
  int32_t bt_stride;
  int32_t num_tokens;               // query rows in the batch
  int32_t max_query_len, max_seq_len;
  float scale;
  // shared-prefix decode (launch_shared_prefix): partials of the prefix's
  // partitions, as the split-KV decode writes them
  float* tmp_out;
  float* max_logits;
  float* exp_sums;
  int32_t partition_size, max_num_partitions;
  int32_t shared_tokens;            // prefix length (a multiple of partition_size)
};

// Rows of requests with q_len > 1 (the decode kernel takes the others).
hipError_t launch_prefill(const PrefillArgs& args, hipStream_t stream);

// Both kinds of rows of a varlen batch in one launch (prefill tiles and
// decode rows side by side on every compute unit); varlen_fused_applies
// says whether launch_varlen handles the batch (bf16 caches, GQA groups
// below 8, enough decode rows to fill the device).
bool varlen_fused_applies(const PrefillArgs& args);

// The shared prefix's partitions of a shared-prefix decode: every request's
// decode query against the key partitions [0, shared_tokens / P) of request
// 0's table, on the matrix cores, written as split-KV partials.
hipError_t launch_shared_prefix(const PrefillArgs& args, hipStream_t stream);
hipError_t launch_varlen(const PrefillArgs& prefill, const DecodeArgs& decode,
                         hipStream_t stream);

}  // namespace pa
