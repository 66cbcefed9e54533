// Cache write path and addressing helpers of libpa (gfx950):
//   slot mapping  -- "vLLM 深度解析（二）：PagedAttention 核心机制" §3.1
//                    (slot = physical_block * B + offset); "vllm 深度解析：
//                    一切从 PagedAttention 谈起" (_compute_slot_mappings_kernel)
//   scatter       -- same page 3: write_to_paged_cache / reshape_and_cache;
//                    FP8 caches store the E4M3FN code of x / scale (the
//                    inverse of the read side's code * scale, §3.2.1 of the
//                    first page)
//   debug gather  -- the read addressing of §3.1, exposed for bit-exact tests
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// One work-group per request; threads stride over the request's new tokens.
__global__ __launch_bounds__(256) void slot_mapping_kernel(
    int64_t* __restrict__ slot_mapping, const int32_t* __restrict__ block_table,
    int32_t bt_stride, const int32_t* __restrict__ query_start_loc,
    const int32_t* __restrict__ seq_lens) {
  const int r = blockIdx.x;
  const int lo = query_start_loc[r];
  const int hi = query_start_loc[r + 1];
  const int first_pos = seq_lens[r] - (hi - lo);
  const int32_t* row = block_table + (int64_t)r * bt_stride;
  for (int j = lo + (int)threadIdx.x; j < hi; j += blockDim.x) {
    const int pos = first_pos + (j - lo);
    const int logical = pos / kBlock;
    const int offset = pos - logical * kBlock;
    slot_mapping[j] = (int64_t)row[logical] * kBlock + offset;
  }
}

hipError_t launch_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                               int32_t bt_stride, const int32_t* query_start_loc,
                               const int32_t* seq_lens, int32_t num_reqs,
                               int32_t /*max_query_len_hint*/, hipStream_t stream) {
  if (num_reqs == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(num_reqs), dim3(256), 0, stream,
                     slot_mapping, block_table, bt_stride, query_start_loc, seq_lens);
  return hipGetLastError();
}

// One thread per 16-byte chunk of a (token, KV head) source row, K and V
// together.  Rows are head_dim bf16 = 8 or 16 chunks; a tile row in the pool
// holds the same head_dim elements in order, so chunk c of the source lands
// at chunk c of the pool row (16 bytes for bf16, 8 codes for FP8).
template <bool FP8>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    void* __restrict__ k_cache, void* __restrict__ v_cache,
    const uint4* __restrict__ key, const uint4* __restrict__ value,
    const int64_t* __restrict__ slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
    int32_t head_dim, const float* __restrict__ k_scale, const float* __restrict__ v_scale) {
  const int chunks = head_dim / 8;                     // 16-byte chunks per row
  const int64_t per_token = (int64_t)num_kv_heads * chunks;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= per_token * num_tokens) return;
  const int64_t j = i / per_token;
  const int rem = (int)(i - j * per_token);
  const int g = rem / chunks;
  const int c = rem - g * chunks;
  const int64_t slot = slot_mapping[j];
  if (slot < 0) return;                                // padding token
  const int64_t dst = slot_offset(slot, g, num_kv_heads, head_dim) / 8 + c;
  const float ks = FP8 ? *k_scale : 1.f, vs = FP8 ? *v_scale : 1.f;
  store_chunk<FP8>(k_cache, dst, key[i], ks);
  store_chunk<FP8>(v_cache, dst, value[i], vs);
}

// The newest token of every request (position seq_len - 1), all KV heads:
// one work-group per request, one thread per 16-byte source chunk.
template <bool FP8>
__global__ __launch_bounds__(256) void append_rows_kernel(
    void* __restrict__ k_cache, void* __restrict__ v_cache, const uint4* __restrict__ key,
    const uint4* __restrict__ value, const int32_t* __restrict__ block_table, int32_t bt_stride,
    const int32_t* __restrict__ seq_lens, int32_t num_kv_heads, int32_t head_dim,
    int64_t* __restrict__ slot_out, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale) {
  const int r = blockIdx.x;
  const int L = seq_lens[r];
  if (L <= 0) return;                                  // no token in this step
  const int pos = L - 1;
  const int64_t slot = (int64_t)block_table[(int64_t)r * bt_stride + pos / kBlock] * kBlock +
                       pos % kBlock;
  if (threadIdx.x == 0 && slot_out != nullptr) slot_out[r] = slot;
  const int chunks = head_dim / 8;
  const float ks = FP8 ? *k_scale : 1.f, vs = FP8 ? *v_scale : 1.f;
  for (int i = threadIdx.x; i < num_kv_heads * chunks; i += blockDim.x) {
    const int g = i / chunks, c = i - g * chunks;
    const int64_t dst = slot_offset(slot, g, num_kv_heads, head_dim) / 8 + c;
    const int64_t src = (int64_t)r * num_kv_heads * chunks + i;
    store_chunk<FP8>(k_cache, dst, key[src], ks);
    store_chunk<FP8>(v_cache, dst, value[src], vs);
  }
}

hipError_t launch_append_rows(void* k_cache, void* v_cache, const void* key, const void* value,
                              const int32_t* block_table, int32_t bt_stride,
                              const int32_t* seq_lens, int32_t num_reqs, int32_t num_kv_heads,
                              int32_t head_dim, int64_t* slot_out, bool fp8,
                              const float* k_scale, const float* v_scale, hipStream_t stream) {
  if (num_reqs == 0) return hipSuccess;
  if (fp8)
    hipLaunchKernelGGL(append_rows_kernel<true>, dim3(num_reqs), dim3(256), 0, stream, k_cache,
                       v_cache, (const uint4*)key, (const uint4*)value, block_table, bt_stride,
                       seq_lens, num_kv_heads, head_dim, slot_out, k_scale, v_scale);
  else
    hipLaunchKernelGGL(append_rows_kernel<false>, dim3(num_reqs), dim3(256), 0, stream, k_cache,
                       v_cache, (const uint4*)key, (const uint4*)value, block_table, bt_stride,
                       seq_lens, num_kv_heads, head_dim, slot_out, k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(void* k_cache, void* v_cache, const void* key,
                                    const void* value, int32_t num_tokens,
                                    const int64_t* slot_mapping, int32_t num_kv_heads,
                                    int32_t head_dim, bool fp8, const float* k_scale,
                                    const float* v_scale, hipStream_t stream) {
  const int64_t total = (int64_t)num_tokens * num_kv_heads * (head_dim / 8);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  if (fp8)
    hipLaunchKernelGGL(reshape_and_cache_kernel<true>, dim3((uint32_t)blocks), dim3(256), 0,
                       stream, k_cache, v_cache, (const uint4*)key, (const uint4*)value,
                       slot_mapping, num_tokens, num_kv_heads, head_dim, k_scale, v_scale);
  else
    hipLaunchKernelGGL(reshape_and_cache_kernel<false>, dim3((uint32_t)blocks), dim3(256), 0,
                       stream, k_cache, v_cache, (const uint4*)key, (const uint4*)value,
                       slot_mapping, num_tokens, num_kv_heads, head_dim, k_scale, v_scale);
  return hipGetLastError();
}

// Slot mapping and scatter in one launch: each thread copies one 16-byte
// chunk of a (token, KV head) row and derives the token's slot itself.  The
// request of token j is found by binary search over query_start_loc, staged
// in LDS when it fits.
constexpr int kQslLds = 2048;

template <bool FP8>
__global__ __launch_bounds__(256) void reshape_and_cache_varlen_kernel(
    void* __restrict__ k_cache, void* __restrict__ v_cache, const uint4* __restrict__ key,
    const uint4* __restrict__ value, const int32_t* __restrict__ block_table, int32_t bt_stride,
    const int32_t* __restrict__ query_start_loc, const int32_t* __restrict__ seq_lens,
    int32_t num_reqs, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
    int64_t* __restrict__ slot_mapping, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale) {
  __shared__ int32_t qsl[kQslLds];
  const bool in_lds = num_reqs + 1 <= kQslLds;
  if (in_lds) {
    for (int i = threadIdx.x; i <= num_reqs; i += blockDim.x) qsl[i] = query_start_loc[i];
    __syncthreads();
  }
  const int chunks = head_dim / 8;
  const int64_t per_token = (int64_t)num_kv_heads * chunks;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= per_token * num_tokens) return;
  const int j = (int)(i / per_token);
  const int rem = (int)(i - (int64_t)j * per_token);
  // largest r with query_start_loc[r] <= j (requests with q_len 0 are skipped)
  int lo = 0, hi = num_reqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int v = in_lds ? qsl[mid] : query_start_loc[mid];
    if (v <= j) lo = mid; else hi = mid - 1;
  }
  const int r = lo;
  const int q0 = in_lds ? qsl[r] : query_start_loc[r];
  const int q1 = in_lds ? qsl[r + 1] : query_start_loc[r + 1];
  const int pos = seq_lens[r] - (q1 - q0) + (j - q0);
  const int logical = pos / kBlock;
  const int64_t slot = (int64_t)block_table[(int64_t)r * bt_stride + logical] * kBlock +
                       (pos - logical * kBlock);
  if (slot_mapping != nullptr && rem == 0) slot_mapping[j] = slot;
  const int g = rem / chunks;
  const int c = rem - g * chunks;
  const int64_t dst = slot_offset(slot, g, num_kv_heads, head_dim) / 8 + c;
  const float ks = FP8 ? *k_scale : 1.f, vs = FP8 ? *v_scale : 1.f;
  store_chunk<FP8>(k_cache, dst, key[i], ks);
  store_chunk<FP8>(v_cache, dst, value[i], vs);
}

hipError_t launch_reshape_and_cache_varlen(void* k_cache, void* v_cache, const void* key,
                                           const void* value, const int32_t* block_table,
                                           int32_t bt_stride, const int32_t* query_start_loc,
                                           const int32_t* seq_lens, int32_t num_reqs,
                                           int32_t num_tokens, int32_t num_kv_heads,
                                           int32_t head_dim, int64_t* slot_mapping, bool fp8,
                                           const float* k_scale, const float* v_scale,
                                           hipStream_t stream) {
  const int64_t total = (int64_t)num_tokens * num_kv_heads * (head_dim / 8);
  if (total == 0 || num_reqs == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  if (fp8)
    hipLaunchKernelGGL(reshape_and_cache_varlen_kernel<true>, dim3((uint32_t)blocks), dim3(256),
                       0, stream, k_cache, v_cache, (const uint4*)key, (const uint4*)value,
                       block_table, bt_stride, query_start_loc, seq_lens, num_reqs, num_tokens,
                       num_kv_heads, head_dim, slot_mapping, k_scale, v_scale);
  else
    hipLaunchKernelGGL(reshape_and_cache_varlen_kernel<false>, dim3((uint32_t)blocks), dim3(256),
                       0, stream, k_cache, v_cache, (const uint4*)key, (const uint4*)value,
                       block_table, bt_stride, query_start_loc, seq_lens, num_reqs, num_tokens,
                       num_kv_heads, head_dim, slot_mapping, k_scale, v_scale);
  return hipGetLastError();
}

// grid (ceil(max_seq_len/16), num_kv_heads, num_reqs); one row per token of
// a block: threads copy 4-byte words of the row.
__global__ __launch_bounds__(256) void gather_kv_kernel(
    uint32_t* __restrict__ k_out, uint32_t* __restrict__ v_out,
    const uint32_t* __restrict__ k_cache, const uint32_t* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, int32_t bt_stride,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_seq_lens,
    int32_t num_kv_heads, int32_t head_dim, int32_t elem_bytes) {
  const int r = blockIdx.z, g = blockIdx.y, b = blockIdx.x;
  const int n = seq_lens[r];
  if (b * kBlock >= n) return;
  const int32_t phys = block_table[(int64_t)r * bt_stride + b];
  const int words = head_dim * elem_bytes / 4;        // 4-byte words per row
  const int64_t tile = tile_offset(phys, g, num_kv_heads, head_dim) * elem_bytes / 4;
  for (int i = threadIdx.x; i < kBlock * words; i += blockDim.x) {
    const int row = i / words, w = i - row * words;
    const int t = b * kBlock + row;
    if (t >= n) break;
    const int64_t dst = (((int64_t)cu_seq_lens[r] + t) * num_kv_heads + g) * words + w;
    k_out[dst] = k_cache[tile + (int64_t)row * words + w];
    v_out[dst] = v_cache[tile + (int64_t)row * words + w];
  }
}

hipError_t launch_gather_kv(void* k_out, void* v_out, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            int32_t bt_stride, const int32_t* seq_lens,
                            const int32_t* cu_seq_lens, int32_t num_reqs,
                            int32_t max_seq_len, int32_t num_kv_heads, int32_t head_dim,
                            int32_t elem_bytes, hipStream_t stream) {
  if (num_reqs == 0 || max_seq_len == 0) return hipSuccess;
  dim3 grid((max_seq_len + kBlock - 1) / kBlock, num_kv_heads, num_reqs);
  hipLaunchKernelGGL(gather_kv_kernel, grid, dim3(256), 0, stream, (uint32_t*)k_out,
                     (uint32_t*)v_out, (const uint32_t*)k_cache, (const uint32_t*)v_cache,
                     block_table, bt_stride, seq_lens, cu_seq_lens, num_kv_heads, head_dim,
                     elem_bytes);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fp8_to_f32_kernel(const uint8_t* __restrict__ codes,
                                                         float* __restrict__ out, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int base = i * 4;
  if (base >= n) return;
  uint32_t w = 0;
  for (int k = 0; k < 4; ++k)
    if (base + k < n) w |= (uint32_t)codes[base + k] << (8 * k);
  const f32x4_t v = fp8x4_to_f32(w);
  const float vals[4] = {v.x, v.y, v.z, v.w};
  for (int k = 0; k < 4; ++k)
    if (base + k < n) out[base + k] = vals[k];
}

hipError_t launch_fp8_to_f32(const uint8_t* codes, float* out, int32_t n,
                             hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int threads = (n + 3) / 4;
  hipLaunchKernelGGL(fp8_to_f32_kernel, dim3((threads + 255) / 256), dim3(256), 0, stream,
                     codes, out, n);
  return hipGetLastError();
}

}  // namespace pa

namespace pa {

// Four codes per thread through the FP8 -> f16 pair conversion of the decode
// kernel's V path (both halves of the word).
__global__ __launch_bounds__(256) void fp8_to_f16_kernel(const uint8_t* __restrict__ codes,
                                                         uint16_t* __restrict__ out, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int base = i * 4;
  if (base >= n) return;
  uint32_t w = 0;
  for (int k = 0; k < 4; ++k)
    if (base + k < n) w |= (uint32_t)codes[base + k] << (8 * k);
  const uint32_t lo = fp8x2_to_f16x2<false>(w), hi = fp8x2_to_f16x2<true>(w);
  const uint16_t vals[4] = {(uint16_t)(lo & 0xffffu), (uint16_t)(lo >> 16),
                            (uint16_t)(hi & 0xffffu), (uint16_t)(hi >> 16)};
  for (int k = 0; k < 4; ++k)
    if (base + k < n) out[base + k] = vals[k];
}

hipError_t launch_fp8_to_f16(const uint8_t* codes, uint16_t* out, int32_t n,
                             hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int threads = (n + 3) / 4;
  hipLaunchKernelGGL(fp8_to_f16_kernel, dim3((threads + 255) / 256), dim3(256), 0, stream,
                     codes, out, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Measurement support: one streaming read of a buffer (16-byte non-temporal
// loads, eight in flight per thread, grid-stride), the on-device read rate
// the attention kernels' HBM rates are compared with.  Nothing is written
// unless the XOR of a thread's data is 0xffffffff, which keeps the loads
// from being removed.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t xor4(const u32x4_t v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4_t* __restrict__ src,
                                                          int64_t n, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  constexpr int U = 8;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= xor4(v[u]);
  }
  for (; i < n; i += stride) acc ^= xor4(__builtin_nontemporal_load(src + i));
  if (acc == 0xffffffffu) sink[0] = acc;
}

hipError_t launch_read_stream(const void* src, int64_t bytes, uint32_t* sink, int32_t work_groups,
                              hipStream_t st) {
  const int64_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  int64_t per = work_groups;
  if (per <= 0) {                       // default: eight 4-wave work-groups per compute unit
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    per = (int64_t)(cus > 0 ? cus : 1) * 8;
  }
  const int64_t groups = per < (n + 255) / 256 ? per : (n + 255) / 256;
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)groups), dim3(256), 0, st,
                     reinterpret_cast<const u32x4_t*>(src), n, sink);
  return hipGetLastError();
}

}  // namespace pa
