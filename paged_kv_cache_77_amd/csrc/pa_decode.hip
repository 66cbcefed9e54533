// Single-query paged decode attention for gfx950.
//
// What is computed ("vLLM 深度解析（二）：PagedAttention 核心机制"):
//   §3.1   block_table[request][t // B] gives the physical block of token t;
//   §3.2.4 scores scale*<q, k> for the query heads sharing one KV head,
//          plus the optional ALiBi term slope_h * (t - seq_len + 1),
//          positions at or past seq_len excluded;
//   §3.2.8 V rows past the context never contribute (selected away, since
//          unwritten slots may hold NaN);
//   §2.2   the running state (m, l, A) makes the tiled result exact;
//   §3.2.7 / §3.3 the split-KV (V2) variant keeps per-partition max logit,
//          exp-sum and normalised output; §3.2.9 merges them.
//
// Kernels here: decode_kernel (single pass and split-KV, one work-group per
// (request, KV head, head chunk[, partition])), the work-balanced decode and
// its merge, the partition merge, and their launchers.  The wave-level
// machinery (lane layout, online softmax, tile streaming) is in
// pa_decode_wave.h.
#include "pa_decode_wave.h"

namespace pa {

// One work-group per (request, KV head, head chunk[, partition]).
// PART: false -> write the final bf16 output; true -> write the partition
// partials.
template <int D, int GC, bool FP8, int WAVES, bool PART, int PD>
__global__ __launch_bounds__(WAVES * 64, (decode_min_waves<GC, FP8, PART, WAVES>())) void decode_kernel(
    DecodeArgs a, int n_chunks) {
  __shared__ DecodeSmem<D, GC, FP8, WAVES> sm;

  // With a.lpt, blockIdx.z is a rank: the request with the rank-th longest
  // context (ties by index), so the hardware hands out the longest units
  // first and the short ones fill the tail (longest-processing-time order).
  // With a.lpt_half, the grid is at most two work-groups per compute unit:
  // requests z < lpt_half (one work-group per compute unit) take ranks z,
  // the rest ranks R - 1 - (z - lpt_half), so the work-group that joins a
  // compute unit later takes a short unit beside a long one.
  int r = blockIdx.z;
  int unit = blockIdx.y;
  int part_idx = blockIdx.x;
  if constexpr (PART) {
    // Split-KV over a grid of many rounds: every XCD gets the same number of
    // work-groups in dispatch order (slot L on XCD L % 8), but the odd XCDs
    // stream ~7% slower, so the items (partition, unit, request) are dealt
    // unevenly -- xcd_even to each even XCD, xcd_odd to each odd one, the odd
    // XCDs' surplus slots idle.
    if (a.xcd_items > 0) {
      const int L = blockIdx.x, x = L % 8, j = L / 8;
      int item;
      if ((x & 1) == 0) {
        item = j < a.xcd_even ? (x >> 1) * a.xcd_even + j : -1;
      } else {
        const int base = 4 * a.xcd_even + (x >> 1) * a.xcd_odd;
        item = (j < a.xcd_odd && base + j < a.xcd_items) ? base + j : -1;
      }
      if (item < 0) return;
      const int per_req = a.num_kv_heads * n_chunks;      // units per request
      const int nparts = a.xcd_items / (a.num_reqs * per_req);
      r = item / (per_req * nparts);
      const int rem = item - r * per_req * nparts;
      unit = rem / nparts;
      part_idx = rem - unit * nparts;
    }
  }
  if constexpr (!PART) {
    if (a.lpt) {
      const int R = a.num_reqs;
      const int z = blockIdx.z, hf = a.lpt_half;
      int32_t* len = sm.bt;                 // [R] context lengths
      int32_t* req_of = sm.bt + R;          // [R] request of each rank
      // (in a varlen batch only rows with q_len 1 are decode rows: the
      // others rank last, and their work-groups exit)
      for (int i = threadIdx.x; i < R; i += WAVES * kWave)
        len[i] = (a.query_start_loc == nullptr ||
                  a.query_start_loc[i + 1] - a.query_start_loc[i] == 1) ? a.seq_lens[i] : -1;
      __syncthreads();
      for (int j = threadIdx.x; j < R; j += WAVES * kWave) {
        const int lj = len[j];
        int rank = 0;
        for (int k = 0; k < R; ++k) {
          const int lk = len[k];
          rank += (lk > lj || (lk == lj && k < j)) ? 1 : 0;
        }
        req_of[rank] = j;
      }
      __syncthreads();
      // Work-groups reach the XCDs round-robin (slot L on XCD L % 8) and, in
      // the two-round grid, slots z and z + hf of an XCD share a compute
      // unit, which thus streams the pair of ranks (p, R - 1 - p).  On
      // MI355X the odd XCDs stream about 7% slower than the even ones on
      // equal work, so when the (KV head, chunk) units are exactly 8 (one
      // per XCD in grid order) the pairs are ranked by their token sum and
      // the heavier half goes to the even XCDs, the lighter half to the odd
      // ones: slot (XCD x, unit slot s = z % hf, round z / hf) takes pair
      // q = (x & 1) * hf/2 + s % (hf/2) in that order and the (KV head, chunk)
      // unit 2 (x >> 1) + s / (hf/2).  Each (rank, unit) is taken once.
      const bool xcd_weighted = PA_DECODE_XCD_WEIGHT && hf > 0 && R == 2 * hf && hf % 2 == 0 &&
                                gridDim.x == 1 && gridDim.y == 8;
      int target;
      if (xcd_weighted) {
        int32_t* psum = sm.bt + 2 * R;      // [hf] token sums of the rank pairs
        int32_t* pair_at = sm.bt + 2 * R + hf;   // [hf] pairs, heaviest first
        for (int p = threadIdx.x; p < hf; p += WAVES * kWave)
          psum[p] = len[req_of[p]] + len[req_of[R - 1 - p]];
        __syncthreads();
        for (int p = threadIdx.x; p < hf; p += WAVES * kWave) {
          int pos = 0;
          for (int k = 0; k < hf; ++k) pos += (psum[k] > psum[p] || (psum[k] == psum[p] && k < p));
          pair_at[pos] = p;
        }
        __syncthreads();
        const int x = blockIdx.y, half = hf / 2, sl = z % hf;
        const int pr = pair_at[(x & 1) * half + sl % half];
        target = z < hf ? pr : R - 1 - pr;
        unit = 2 * (x >> 1) + sl / half;
      } else {
        target = (hf > 0 && z >= hf) ? R - 1 - (z - hf) : z;
      }
      r = __builtin_amdgcn_readfirstlane(req_of[target]);
      unit = __builtin_amdgcn_readfirstlane(unit);
      __syncthreads();
    }
  }
  decode_unit<D, GC, FP8, WAVES, PART, PD>(a, sm, r, unit, part_idx, n_chunks);
}

// ---------------------------------------------------------------------------
// Work-balanced decode.  The items are the 16-token blocks of every unit
// (request r, KV head g, head chunk), units in order and blocks in order
// within a unit; with N items and W waves, wave k takes items
// [floor(kN/W), floor((k+1)N/W)).  A unit a wave covers entirely is written
// to the output directly.  Otherwise the wave leaves a partial record --
// slot 0 for a piece that does not start at the unit's first block (only the
// wave's first piece can), slot 1 for a piece that starts there but ends
// inside the unit (only its last piece can) -- and balanced_merge_kernel
// folds the pieces of each split unit with the merge of the split-KV page
// section (§3.2.9).  Every wave streams the same number of blocks, so no
// long request leaves the GPU idle at the end.
constexpr int kBalWaves = 4;               // waves per work-group
constexpr int kBalMaxReqs = 4096;          // requests whose prefix fits in LDS
constexpr int kBalMaxTotalWaves = 4096;    // waves the workspace is sized for
constexpr int kBalSegBlocks = 256;         // block-table entries per wave in LDS

struct BalancedLayout {
  // workspace: int32 prefix[R + 1] (256-byte aligned), then float records
  // [W][2][GC][D + 2]: m (natural log units) per head, l per head, O rows.
  static __host__ __device__ int64_t header_bytes(int num_reqs) {
    return ((int64_t)(num_reqs + 1) * 4 + 255) / 256 * 256;
  }
  static __host__ __device__ int64_t record_floats(int gc, int d) { return (int64_t)gc * (d + 2); }
};

__device__ __forceinline__ int64_t bal_bound(int64_t k, int64_t N, int64_t W) {
  return k * N / W;
}

// Number of blocks of every request, exclusive prefix into C[0..R] (LDS).
__device__ __forceinline__ void block_prefix(const int32_t* seq_lens, int R, int32_t* C,
                                             int32_t* scratch256) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (R + nt - 1) / nt;
  const int lo = min(R, tid * per), hi = min(R, lo + per);
  int32_t sum = 0;
  for (int r = lo; r < hi; ++r) sum += (seq_lens[r] + kBlock - 1) / kBlock;
  scratch256[tid] = sum;
  __syncthreads();
  for (int s = 1; s < nt; s <<= 1) {          // inclusive Hillis-Steele scan
    const int32_t v = tid >= s ? scratch256[tid - s] : 0;
    __syncthreads();
    scratch256[tid] += v;
    __syncthreads();
  }
  int32_t run = scratch256[tid] - sum;         // exclusive prefix of this chunk
  for (int r = lo; r < hi; ++r) {
    C[r] = run;
    run += (seq_lens[r] + kBlock - 1) / kBlock;
  }
  if (tid == nt - 1) C[R] = scratch256[nt - 1];
  __syncthreads();
}

template <int D, int GC, bool FP8, int PD>
__global__ __launch_bounds__(kBalWaves * 64) void decode_balanced_kernel(
    DecodeArgs a, int n_chunks, float* __restrict__ records, int32_t* __restrict__ prefix_out) {
  using Dec = WaveDecoder<D, GC, FP8>;
  __shared__ int32_t C[kBalMaxReqs + 1];
  __shared__ int32_t scan[kBalWaves * 64];
  __shared__ int32_t bt_l[kBalWaves][kBalSegBlocks];
  __shared__ float slab[kBalWaves][2][kBlock][Dec::GCP];

  const int R = a.num_reqs;
  block_prefix(a.seq_lens, R, C, scan);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= R; i += blockDim.x) prefix_out[i] = C[i];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);     // scalar wave index
  const int G = a.num_q_heads / a.num_kv_heads;
  const int U = a.num_kv_heads * n_chunks;                  // units per request
  // (LDS reads are per lane to the compiler: the wave-uniform values below
  // are made scalar, so the loop bounds and tile addresses stay uniform)
  const int64_t N = (int64_t)__builtin_amdgcn_readfirstlane(C[R]) * U;
  const int64_t W = (int64_t)gridDim.x * kBalWaves;
  const int64_t k = (int64_t)blockIdx.x * kBalWaves + w;
  const int64_t x_end = bal_bound(k + 1, N, W);
  int64_t x = bal_bound(k, N, W);
  const int64_t x_begin = x;
  int piece_b0 = 0;

  float qk_scale = a.scale * kLog2e;
  if constexpr (FP8) qk_scale *= *a.k_scale;
  Dec dec;
  dec.init(lane, qk_scale, a.alibi_slopes != nullptr);
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);
  const float vs = FP8 ? *a.v_scale : 1.f;
  const int rec = (int)BalancedLayout::record_floats(GC, D);

  while (x < x_end) {
    // unit containing item x: the largest r with C[r]*U <= x (requests with
    // no blocks share their C with the next one and are never picked)
    int lo = 0, hi = R - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)C[mid] * U <= x) lo = mid; else hi = mid - 1;
    }
    const int r = __builtin_amdgcn_readfirstlane(lo);
    const int cr = __builtin_amdgcn_readfirstlane(C[r]);
    const int nb = __builtin_amdgcn_readfirstlane(C[r + 1]) - cr;
    const int64_t local = x - (int64_t)cr * U;
    const int j = (int)(local / nb);
    const int b0 = (int)(local - (int64_t)j * nb);
    const int b1 = (int)min<int64_t>(nb, b0 + (x_end - x));
    const int g = j / n_chunks, hc = j - g * n_chunks;
    const int h0 = g * G + hc * GC, nh = min(GC, G - hc * GC);
    const int seq_len = a.seq_lens[r];
    const int32_t* bt_row = a.block_table + (int64_t)r * a.bt_stride;

    if (b0 == 0 || x == x_begin) {
      piece_b0 = b0;            // a new unit (or the wave's first piece)
      dec.load_q(reinterpret_cast<const uint16_t*>(a.q), r, a.num_q_heads, h0, nh);
      dec.set_query(a.alibi_slopes, h0, seq_len);
      dec.reset();
    }
    // at most kBalSegBlocks blocks per pass; the unit continues in the next pass
    const int ce = min(b1, b0 + kBalSegBlocks);
    {
      const int n = ce - b0;
      for (int i = lane; i < n; i += kWave) bt_l[w][i] = bt_row[b0 + i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      stream_blocks<PD>(
          dec, n, kbase, vbase, g, a.num_kv_heads, seq_len, &slab[w][0][0][0], &slab[w][1][0][0],
          [&](int it) { return __builtin_amdgcn_readfirstlane(bt_l[w][min(it, n - 1)]); },
          [&](int it) { return (b0 + it) * kBlock; });
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    if (ce < b1) {                            // more of this piece to come
      x += ce - b0;
      continue;
    }
    dec.finish();

    if (piece_b0 == 0 && b1 == nb) {                // the whole unit: write the output row
#pragma unroll
      for (int jj = 0; jj < GC; ++jj) {
        const float inv = vs / __builtin_bit_cast(float,
            __builtin_amdgcn_readlane(__builtin_bit_cast(int, dec.l_part), jj));
        if (jj < nh && lane < 16) {
          uint16_t* o = reinterpret_cast<uint16_t*>(a.out) +
                        ((int64_t)r * a.num_q_heads + h0 + jj) * D + dec.vcol;
#pragma unroll
          for (int e = 0; e < Dec::VE; ++e) o[e] = f32_to_bf16(dec.acc[jj][e] * inv);
        }
      }
    } else {                                  // a piece: partial record
      const int slot = piece_b0 != 0 ? 0 : 1;
      float* rp = records + (k * 2 + slot) * rec;
#pragma unroll
      for (int jj = 0; jj < GC; ++jj) {
        const float L = __builtin_bit_cast(float,
            __builtin_amdgcn_readlane(__builtin_bit_cast(int, dec.l_part), jj));
        const float M = __builtin_bit_cast(float,
            __builtin_amdgcn_readlane(__builtin_bit_cast(int, dec.m_run), jj));
        const float Mt = __builtin_bit_cast(float,
            __builtin_amdgcn_readlane(__builtin_bit_cast(int, dec.m_true), jj));
        const float inv = vs / L;
        if (lane == 0) {
          rp[jj] = Mt * kLn2;                               // m in natural-log units
          rp[GC + jj] = L * fast_exp2(M - Mt);             // l relative to it
        }
        if (lane < 16) {
#pragma unroll
          for (int e = 0; e < Dec::VE; ++e) rp[2 * GC + jj * D + dec.vcol + e] = dec.acc[jj][e] * inv;
        }
      }
    }
    x += b1 - b0;
  }
}

// Fold the pieces of every split unit.  One work-group per unit, one wave
// per head of the chunk: lanes first read the pieces' (m, l) in parallel,
// then every lane sums its D/64 output elements over the pieces.
template <int D, int GC>
__global__ __launch_bounds__(GC * 64) void balanced_merge_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ records,
    const int32_t* __restrict__ prefix, int32_t num_reqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t n_chunks, int32_t total_waves) {
  constexpr int E = D / 64;
  const int U = num_kv_heads * n_chunks;
  const int r = blockIdx.x / U, j = blockIdx.x - (blockIdx.x / U) * U;
  const int lane = threadIdx.x % 64, jj = threadIdx.x / 64;
  const int G = num_q_heads / num_kv_heads;
  const int g = j / n_chunks, hc = j - g * n_chunks;
  const int h0 = g * G + hc * GC, nh = min(GC, G - hc * GC);
  if (jj >= nh) return;
  const int nb = prefix[r + 1] - prefix[r];
  uint16_t* o = out + ((int64_t)r * num_q_heads + h0 + jj) * D;
  if (nb == 0) {                                    // empty context: zero row
    for (int i = lane; i < D; i += 64) o[i] = 0;
    return;
  }
  const int64_t N = (int64_t)prefix[num_reqs] * U;
  const int64_t W = total_waves;
  const int64_t S = (int64_t)prefix[r] * U + (int64_t)j * nb;
  const int64_t Eend = S + nb;
  // wave holding item x: the largest k with floor(kN/W) <= x
  auto wave_of = [&](int64_t xx) { return ((xx + 1) * W + N - 1) / N - 1; };
  const int64_t kf = wave_of(S), kl = wave_of(Eend - 1);
  if (kf == kl) return;                             // written whole by one wave
  const int rec = (int)BalancedLayout::record_floats(GC, D);
  const int npieces = (int)(kl - kf + 1);
  // pass 1: max of the pieces' m (lanes over pieces)
  float M = -INFINITY;
  for (int i = lane; i < npieces; i += 64) {
    const int64_t kk = kf + i;
    if (kk > kf && bal_bound(kk, N, W) == bal_bound(kk + 1, N, W)) continue;   // empty wave
    M = fmaxf(M, records[(kk * 2 + (kk == kf ? 1 : 0)) * rec + jj]);
  }
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) M = fmaxf(M, xor_lanes(M, s));
  // pass 2: weighted sum of the pieces' rows
  float L = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int i = 0; i < npieces; ++i) {
    const int64_t kk = kf + i;
    if (kk > kf && bal_bound(kk, N, W) == bal_bound(kk + 1, N, W)) continue;
    const float* rp = records + (kk * 2 + (kk == kf ? 1 : 0)) * rec;
    const float wgt = rp[GC + jj] * fast_exp2((rp[jj] - M) * kLog2e);
    L += wgt;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(wgt, rp[2 * GC + jj * D + lane * E + e], acc[e]);
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int e = 0; e < E; ++e) o[lane * E + e] = f32_to_bf16(acc[e] * inv);
}

// ---------------------------------------------------------------------------
// merge of partition partials ("vLLM 深度解析（二）：PagedAttention 核心机制"
// §3.2.9): one 256-thread work-group per (request, query head).  The
// partition weights l_j e^(m_j - m) go to LDS first; then groups of D/4
// threads each read one partition row with 16-byte loads, so 256/(D/4)
// partitions are in flight per step, and the groups are summed in LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeMaxParts = 2048;    // partitions held in LDS per pass

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ tmp_out,
    const float* __restrict__ max_logits, const float* __restrict__ exp_sums,
    const int32_t* __restrict__ seq_lens, int32_t num_q_heads, int32_t partition_size,
    int32_t max_num_partitions, int32_t max_used) {
  constexpr int TPR = D / 4;                    // threads per partition row
  constexpr int PG = kMergeThreads / TPR;       // partition rows per step
  __shared__ float wgt[kMergeMaxParts];
  __shared__ float red[kMergeThreads];
  __shared__ f32x4_t part[PG][TPR];
  const int r = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  int n = (seq_lens[r] + partition_size - 1) / partition_size;
  if (max_used > 0) n = min(n, max_used);      // the last record may be an open tail
  n = min(n, max_num_partitions);              // (a seq_len past the host bound stays in bounds)
  const int64_t base = ((int64_t)r * num_q_heads + h) * max_num_partitions;
  const int pg = tid / TPR, c = tid % TPR;

  // global max of the partition maxima
  float M = -INFINITY;
  for (int p = tid; p < n; p += kMergeThreads) M = fmaxf(M, max_logits[base + p]);
  red[tid] = M;
  __syncthreads();
  for (int s = kMergeThreads / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
    __syncthreads();
  }
  M = red[0];
  __syncthreads();

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int p0 = 0; p0 < n; p0 += kMergeMaxParts) {
    const int np = min(n - p0, kMergeMaxParts);
    float lsum = 0.f;
    for (int p = tid; p < np; p += kMergeThreads) {
      const float w = exp_sums[base + p0 + p] * fast_exp2((max_logits[base + p0 + p] - M) * kLog2e);
      wgt[p] = w;
      lsum += w;
    }
    red[tid] = lsum;
    __syncthreads();
    for (int s = kMergeThreads / 2; s > 0; s >>= 1) {
      if (tid < s) red[tid] += red[tid + s];
      __syncthreads();
    }
    L += red[0];
    const f32x4_t* rows = reinterpret_cast<const f32x4_t*>(tmp_out + (base + p0) * D);
#pragma unroll 4
    for (int p = pg; p < np; p += PG) {
      const f32x4_t v = rows[(int64_t)p * TPR + c];
      const float w = wgt[p];
      acc.x = fmaf(w, v.x, acc.x);
      acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z);
      acc.w = fmaf(w, v.w, acc.w);
    }
    __syncthreads();
  }
  part[pg][c] = acc;
  __syncthreads();
  if (pg == 0) {
    f32x4_t sum = part[0][c];
#pragma unroll
    for (int g = 1; g < PG; ++g) {
      sum.x += part[g][c].x; sum.y += part[g][c].y;
      sum.z += part[g][c].z; sum.w += part[g][c].w;
    }
    const float inv = n ? 1.f / L : 0.f;
    const uint32_t w0 = (uint32_t)f32_to_bf16(sum.x * inv) | ((uint32_t)f32_to_bf16(sum.y * inv) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16(sum.z * inv) | ((uint32_t)f32_to_bf16(sum.w * inv) << 16);
    *reinterpret_cast<uint2*>(out + ((int64_t)r * num_q_heads + h) * D + 4 * c) = make_uint2(w0, w1);
  }
}

// The same merge for short partition lists (at most kMergeFewParts per
// request): one wave per (request, query head), four per work-group.  Lane p
// holds partition p's weight l_p e^(m_p - m); every lane then sums its D/64
// output elements over the partitions.
constexpr int kMergeFewParts = 16;

template <int D>
__global__ __launch_bounds__(256) void merge_few_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ tmp_out,
    const float* __restrict__ max_logits, const float* __restrict__ exp_sums,
    const int32_t* __restrict__ seq_lens, int32_t num_reqs, int32_t num_q_heads,
    int32_t partition_size, int32_t max_num_partitions, int32_t max_used) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x % 64;
  const int64_t unit = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;     // r * Hq + h
  if (unit >= (int64_t)num_reqs * num_q_heads) return;
  const int r = (int)(unit / num_q_heads);
  int n = (seq_lens[r] + partition_size - 1) / partition_size;
  if (max_used > 0) n = min(n, max_used);      // the last record may be an open tail
  n = min(n, max_num_partitions);              // (a seq_len past the host bound stays in bounds)
  const int64_t base = unit * max_num_partitions;
  const float m = lane < n ? max_logits[base + lane] : -INFINITY;
  float M = m;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) M = fmaxf(M, xor_lanes(M, s));
  const float wgt = (lane < n && m != -INFINITY) ? exp_sums[base + lane] * fast_exp2((m - M) * kLog2e)
                                                 : 0.f;
  float L = wgt;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) L += xor_lanes(L, s);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int p = 0; p < n; ++p) {
    const float wp = __shfl(wgt, p, 64);
    if (wp != 0.f) {                           // (a partition with no key holds no row)
      const float* row = tmp_out + (base + p) * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(wp, row[e], acc[e]);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) out[unit * D + lane * E + e] = f32_to_bf16(acc[e] * inv);
}

// The same merge for 17..64 partitions: one wave per (request, query head),
// four per work-group, everything in flight at once.  Lane q holds partition
// q's weight l_q e^(m_q - m); every partition row is read up front, D/4
// lanes per row with 16-byte loads (64 / (D/4) rows per load instruction);
// each lane sums its rows with their weights (shuffled from the owning
// lanes), and the row groups are combined across lanes at the end.
constexpr int kMergeWaveParts = 64;
#ifndef PA_MERGE_WAVE
#define PA_MERGE_WAVE 1
#endif

template <int D>
__global__ __launch_bounds__(256) void merge_wave_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ tmp_out,
    const float* __restrict__ max_logits, const float* __restrict__ exp_sums,
    const int32_t* __restrict__ seq_lens, int32_t num_reqs, int32_t num_q_heads,
    int32_t partition_size, int32_t max_num_partitions, int32_t max_used) {
  constexpr int LPR = D / 4;                     // lanes per partition row
  constexpr int RPL = kWave / LPR;               // rows per load instruction
  constexpr int NL = kMergeWaveParts / RPL;      // load instructions per lane
  const int lane = threadIdx.x % kWave;
  const int64_t unit = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;     // r * Hq + h
  if (unit >= (int64_t)num_reqs * num_q_heads) return;
  const int r = (int)(unit / num_q_heads);
  int n = (seq_lens[r] + partition_size - 1) / partition_size;
  if (max_used > 0) n = min(n, max_used);        // the last record may be an open tail
  n = min(n, min(max_num_partitions, kMergeWaveParts));
  const int64_t base = unit * max_num_partitions;
  const int c = lane % LPR, grp = lane / LPR;
  f32x4_t v[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int p = i * RPL + grp;
    v[i] = p < n ? *reinterpret_cast<const f32x4_t*>(tmp_out + (base + p) * D + 4 * c)
                 : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float m = lane < n ? max_logits[base + lane] : -INFINITY;
  float M = m;
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) M = fmaxf(M, xor_lanes(M, s));
  const float wgt = (lane < n && m != -INFINITY) ? exp_sums[base + lane] * fast_exp2((m - M) * kLog2e)
                                                 : 0.f;
  float L = wgt;
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) L += xor_lanes(L, s);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const float wp = __shfl(wgt, i * RPL + grp, kWave);
    acc.x = fmaf(wp, v[i].x, acc.x);
    acc.y = fmaf(wp, v[i].y, acc.y);
    acc.z = fmaf(wp, v[i].z, acc.z);
    acc.w = fmaf(wp, v[i].w, acc.w);
  }
#pragma unroll
  for (int s = LPR; s < kWave; s <<= 1) {
    acc.x += xor_lanes(acc.x, s);
    acc.y += xor_lanes(acc.y, s);
    acc.z += xor_lanes(acc.z, s);
    acc.w += xor_lanes(acc.w, s);
  }
  if (lane < LPR) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const uint32_t w0 = (uint32_t)f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16);
    *reinterpret_cast<uint2*>(out + unit * D + 4 * c) = make_uint2(w0, w1);
  }
}

// ---------------------------------------------------------------------------
// dispatch

// Compute units of the current device (cached per device; 0 if unknown).
static int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev] = cus;
  }
  return cached[dev];
}

template <int D, int GC, bool FP8>
static hipError_t launch_decode_t(const DecodeArgs& a, bool partitioned, hipStream_t st) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int n_chunks = (G + GC - 1) / GC;
  constexpr int PD = PA_DECODE_PREFETCH;
  if (partitioned) {
    constexpr int WAVES = PA_DECODE_WAVES_SPLIT;
    int nparts = (a.max_seq_len + a.partition_size - 1) / a.partition_size;
    if (a.part_end > 0) nparts = min(nparts, a.part_end) - a.part_begin;
    if (nparts <= 0) return hipSuccess;
    dim3 grid(nparts, a.num_kv_heads * n_chunks, a.num_reqs);
    DecodeArgs b = a;
    b.xcd_items = 0;
    const int64_t items = (int64_t)grid.x * grid.y * grid.z;
    const int cus = device_cu_count();
    if (PA_DECODE_XCD_WEIGHT && cus > 0 && items >= 8 * (int64_t)cus && items < (1 << 28)) {
      // even : odd XCD shares 1.07 : 1 (measured streaming rates)
      const int64_t ne = (items * 107 + 4 * 207 - 1) / (4 * 207);
      const int64_t no = (items - 4 * ne + 3) / 4;
      b.xcd_items = (int32_t)items;
      b.xcd_even = (int32_t)ne;
      b.xcd_odd = (int32_t)no;
      grid = dim3((unsigned)(8 * std::max(ne, no)), 1, 1);
    }
    hipLaunchKernelGGL((decode_kernel<D, GC, FP8, WAVES, true, PD>), grid, dim3(WAVES * 64), 0, st,
                       b, n_chunks);
  } else {
    // Few work-groups: spread each context over more waves; many: more groups.
    dim3 grid(1, a.num_kv_heads * n_chunks, a.num_reqs);
    const int64_t groups = (int64_t)grid.y * grid.z;
    DecodeArgs b = a;
    // (the rank search costs O(num_reqs) per thread: kept to modest batches)
    b.lpt = (PA_DECODE_LPT && a.num_reqs <= kLptMaxReqs) ? 1 : 0;
    const int64_t min_len = groups < 384 ? PA_DECODE_WAVES_SINGLE_MIN_LEN
                                         : 2 * PA_DECODE_WAVES_SINGLE_MIN_LEN;
    const int cus = device_cu_count();
    if (b.lpt && cus > 0 && groups > cus && groups <= 2 * cus) {
      // one to two rounds: 4-wave work-groups, all resident at once (two per
      // compute unit), ranks paired long with short (measured on MI355X:
      // 64 requests x 8 KV heads, contexts U[512, 4096]: 0.111 vs 0.114 ms
      // with 8 waves in two rounds; 64 x 2048 tokens: 0.090 vs 0.096 ms)
      b.lpt_half = std::max(1, cus / (int)grid.y);
      constexpr int WAVES = PA_DECODE_WAVES_SPLIT;
      hipLaunchKernelGGL((decode_kernel<D, GC, FP8, WAVES, false, PD>), grid, dim3(WAVES * 64), 0,
                         st, b, n_chunks);
    } else if (groups < 768 && a.max_seq_len >= min_len) {
      constexpr int WAVES = PA_DECODE_WAVES_SINGLE;
      hipLaunchKernelGGL((decode_kernel<D, GC, FP8, WAVES, false, PD>), grid, dim3(WAVES * 64), 0,
                         st, b, n_chunks);
    } else {
      constexpr int WAVES = PA_DECODE_WAVES_SPLIT;
      hipLaunchKernelGGL((decode_kernel<D, GC, FP8, WAVES, false, PD>), grid, dim3(WAVES * 64), 0,
                         st, b, n_chunks);
    }
  }
  return hipGetLastError();
}

template <int D, int GC, bool FP8>
static hipError_t launch_balanced_t(const DecodeArgs& a, void* workspace, hipStream_t st) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int n_chunks = (G + GC - 1) / GC;
  constexpr int PD = PA_DECODE_PREFETCH;
  auto kern = decode_balanced_kernel<D, GC, FP8, PD>;
  // as many waves as fit on the device at once (one round, no tail)
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBalWaves * 64, 0);
  if (e != hipSuccess) return e;
  int groups = max(1, cus * max(1, per_cu));
  groups = min(groups, kBalMaxTotalWaves / kBalWaves);
  int32_t* prefix = reinterpret_cast<int32_t*>(workspace);
  float* records = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                            BalancedLayout::header_bytes(a.num_reqs));
  hipLaunchKernelGGL(kern, dim3(groups), dim3(kBalWaves * 64), 0, st, a, n_chunks, records, prefix);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int units = a.num_reqs * a.num_kv_heads * n_chunks;
  hipLaunchKernelGGL((balanced_merge_kernel<D, GC>), dim3(units), dim3(GC * 64), 0, st,
                     reinterpret_cast<uint16_t*>(a.out), records, prefix, a.num_reqs,
                     a.num_q_heads, a.num_kv_heads, n_chunks, groups * kBalWaves);
  return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t launch_decode_d(const DecodeArgs& a, int mode, void* ws, hipStream_t st) {
  const int G = a.num_q_heads / a.num_kv_heads;
#define PA_CASE(GCV)                                                              \
  case GCV:                                                                       \
    return mode == 2 ? launch_balanced_t<D, GCV, FP8>(a, ws, st)                  \
                     : launch_decode_t<D, GCV, FP8>(a, mode == 1, st);
  switch (G) {
    PA_CASE(1)
    PA_CASE(2)
    PA_CASE(3)
    PA_CASE(4)
    PA_CASE(5)
    PA_CASE(6)
    PA_CASE(7)
    default:                                                  // chunks of 8
      return mode == 2 ? launch_balanced_t<D, 8, FP8>(a, ws, st)
                       : launch_decode_t<D, 8, FP8>(a, mode == 1, st);
  }
#undef PA_CASE
}

static hipError_t launch_any(const DecodeArgs& a, int mode, void* ws, hipStream_t st) {
  if (a.num_reqs == 0) return hipSuccess;
  const bool fp8 = a.cache_dtype != 0;
  // FP8 caches with groups of 4+ query heads, bf16 ones with large groups:
  // the MFMA kernel (the vector-ALU kernel is the limit there, not memory)
  if (PA_DECODE_FP8_MFMA && fp8 && mode != 2 && a.num_q_heads / a.num_kv_heads >= 4)
    return launch_decode_mfma(a, mode == 1, st);
  if (PA_DECODE_BF16_MFMA_MIN_G > 0 && !fp8 && mode != 2 &&
      a.num_q_heads / a.num_kv_heads >= PA_DECODE_BF16_MFMA_MIN_G)
    return launch_decode_mfma(a, mode == 1, st);
  if (a.head_dim == 64)
    return fp8 ? launch_decode_d<64, true>(a, mode, ws, st)
               : launch_decode_d<64, false>(a, mode, ws, st);
  return fp8 ? launch_decode_d<128, true>(a, mode, ws, st)
             : launch_decode_d<128, false>(a, mode, ws, st);
}

hipError_t launch_decode(const DecodeArgs& a, bool partitioned, hipStream_t st) {
  return launch_any(a, partitioned ? 1 : 0, nullptr, st);
}

hipError_t launch_decode_append(const DecodeArgs& a, hipStream_t st) {
  if (a.num_reqs == 0) return hipSuccess;
  const bool fp8 = a.cache_dtype != 0;
  const int G = a.num_q_heads / a.num_kv_heads;
  // the vector-ALU single pass with one head chunk per KV head writes the
  // rows itself; the other paths get them from a launch before
  const bool in_kernel = !(PA_DECODE_FP8_MFMA && fp8 && G >= 4) &&
                         !(PA_DECODE_BF16_MFMA_MIN_G > 0 && !fp8 &&
                           G >= PA_DECODE_BF16_MFMA_MIN_G) &&
                         G <= 8;
  if (in_kernel) return launch_any(a, 0, nullptr, st);
  const hipError_t e = launch_append_rows(const_cast<void*>(a.k_cache),
                                          const_cast<void*>(a.v_cache), a.new_k, a.new_v,
                                          a.block_table, a.bt_stride, a.seq_lens, a.num_reqs,
                                          a.num_kv_heads, a.head_dim, a.slot_out, fp8, a.k_scale,
                                          a.v_scale, st);
  if (e != hipSuccess) return e;
  DecodeArgs b = a;
  b.new_k = b.new_v = nullptr;
  b.slot_out = nullptr;
  return launch_any(b, 0, nullptr, st);
}

hipError_t launch_decode_balanced(const DecodeArgs& a, void* workspace, hipStream_t st) {
  return launch_any(a, 2, workspace, st);
}

int64_t balanced_workspace_bytes(int num_reqs, int num_q_heads, int num_kv_heads, int head_dim) {
  const int G = num_q_heads / num_kv_heads;
  const int gc = G > 8 ? 8 : G;
  return BalancedLayout::header_bytes(num_reqs) +
         (int64_t)kBalMaxTotalWaves * 2 * BalancedLayout::record_floats(gc, head_dim) * 4;
}

int balanced_max_reqs() { return kBalMaxReqs; }

hipError_t launch_merge(void* out, const float* tmp_out, const float* max_logits,
                        const float* exp_sums, const int32_t* seq_lens, int32_t num_reqs,
                        int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                        int32_t max_num_partitions, hipStream_t st, int32_t max_used) {
  if (num_reqs == 0) return hipSuccess;
  const int parts = max_used > 0 ? std::min(max_used, max_num_partitions) : max_num_partitions;
  if (parts <= kMergeFewParts) {
    const int64_t units = (int64_t)num_reqs * num_q_heads;
    const dim3 g4((unsigned)((units + 3) / 4));
    if (head_dim == 64)
      hipLaunchKernelGGL(merge_few_kernel<64>, g4, dim3(256), 0, st, (uint16_t*)out, tmp_out,
                         max_logits, exp_sums, seq_lens, num_reqs, num_q_heads, partition_size,
                         max_num_partitions, max_used);
    else
      hipLaunchKernelGGL(merge_few_kernel<128>, g4, dim3(256), 0, st, (uint16_t*)out, tmp_out,
                         max_logits, exp_sums, seq_lens, num_reqs, num_q_heads, partition_size,
                         max_num_partitions, max_used);
    return hipGetLastError();
  }
  if (PA_MERGE_WAVE && parts <= kMergeWaveParts) {
    const int64_t units = (int64_t)num_reqs * num_q_heads;
    const dim3 g4((unsigned)((units + 3) / 4));
    if (head_dim == 64)
      hipLaunchKernelGGL(merge_wave_kernel<64>, g4, dim3(256), 0, st, (uint16_t*)out, tmp_out,
                         max_logits, exp_sums, seq_lens, num_reqs, num_q_heads, partition_size,
                         max_num_partitions, max_used);
    else
      hipLaunchKernelGGL(merge_wave_kernel<128>, g4, dim3(256), 0, st, (uint16_t*)out, tmp_out,
                         max_logits, exp_sums, seq_lens, num_reqs, num_q_heads, partition_size,
                         max_num_partitions, max_used);
    return hipGetLastError();
  }
  dim3 grid(num_q_heads, num_reqs);
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kMergeThreads), 0, st, (uint16_t*)out, tmp_out,
                       max_logits, exp_sums, seq_lens, num_q_heads, partition_size,
                       max_num_partitions, max_used);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kMergeThreads), 0, st, (uint16_t*)out, tmp_out,
                       max_logits, exp_sums, seq_lens, num_q_heads, partition_size,
                       max_num_partitions, max_used);
  return hipGetLastError();
}

}  // namespace pa
