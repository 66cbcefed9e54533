// Varlen chunked prefill over the paged cache, MFMA tiles for gfx950.
//
// What is computed ("第11章 分块预填充与混合批处理" §11.6; "vLLM 深度解析（二）：
// PagedAttention 核心机制" §2 and §5.2): request r owns query rows
// query_start_loc[r] .. query_start_loc[r+1]-1; row i sits at position
// seq_len - q_len + i and attends keys 0..position (causal), K/V read through
// block_table[r][t / 16].  With ALiBi slopes the score of key t for the query
// at position p gains slope_h * (t - p): the decode term of "vLLM 深度解析
// （二）" §3.2.4, slope_h * (t - seq_len + 1), is this for p = seq_len - 1.
// Tiles of keys are folded in with the running (m, l, A) state, so S and P
// never reach HBM (§2.1/§2.2 of the second page).
// Rows of requests with q_len <= 1 are left to the decode kernel.
//
// Work-group: (request, KV head, query tile, head chunk).  Its 4 waves share
// the staged K / V^T tiles: with group size G >= 4 each wave is one query
// head of the chunk over 32 queries; with G < 4 the waves cover the G heads
// times 4/G blocks of 32 queries.  Staging is done once per KV group.
// Per 64-key tile (4 cache blocks):
//   S^T[64 keys x 32 queries] = K . Q^T   (v_mfma_f32_32x32x16_bf16; keys on
//       the M side so each lane owns one query column: the softmax row
//       reductions are in-lane plus one swap with lane^32)
//   O^T[d x 32 queries] += V^T . P^T      (P^T comes straight from the S^T
//       accumulators: the MFMA contraction order over keys is permuted to the
//       order the accumulators hold them, and the V^T fragments are read
//       from LDS in that order)
// bf16 caches: each wave copies one 16-token block of K and of V straight
// from global memory into LDS (global_load_lds_dwordx4: no staging
// registers), both row-major with a 16-byte-chunk XOR swizzle; the V^T
// fragments of the PV products come from gfx950's transposing LDS read
// (ds_read_b64_tr_b16).  FP8 caches are converted to bf16 in registers on
// the way and stored in the same layout.  All tiles are double-buffered.
// P^T enters the PV products in bf16, and the softmax denominator sums those
// same rounded weights, so O stays an exact weighted average of V's rows.
#include <algorithm>

#include "pa_decode_wave.h"
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// LDS offset of a generic pointer to an LDS object (its low 32 bits)
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// v_mfma / ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane
// i receives element i % 4 of the 64-bit values addressed by lanes
// 4e + i / 4, e = 0..3 (a 4 x 4 transpose of 16-bit elements per group).
// Two of these reads form one 8-element MFMA operand (p0's elements first),
// kept as one vector so both land in the operand's registers.
__device__ __forceinline__ uint4 lds_read_tr16_pair(const void* p0, const void* p1) {
  const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p0);
  const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p1);
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(uint4, v);
}

constexpr int kBN = 64;         // keys per tile
constexpr int kWaves = 4;
constexpr int kQW = 32;         // queries per wave
constexpr int kMaxPrefillGroups = 4096;   // work-groups of one launch (a multiple of 8)
// Prefill and decode rows of a varlen batch in one launch where it applies
// (0: always the two launches, decode rows then prefill rows).
#ifndef PA_VARLEN_FUSED
#define PA_VARLEN_FUSED 1
#endif
// Tiles in flight per decode wave in the fused launch (its work-groups have
// 256 VGPRs per wave, the prefill role's budget).
#ifndef PA_VARLEN_DECODE_PREFETCH
#define PA_VARLEN_DECODE_PREFETCH 1
#endif
// Prefill items placed before the decode units in the fused launch, in
// multiples of the compute-unit count (measured on the mixed batch of 128
// decode rows and a 2048-token chunk: 2 -- every item first, decode units
// filling the slots the items free -- 0.775 ms; 1: 0.80; 0: 0.80; two
// launches: 0.82).
#ifndef PA_VARLEN_FIRST
#define PA_VARLEN_FIRST 2
#endif
// The fused launch hands out its decode rows longest first for batches of
// up to this many requests (each decode work-group ranks the rows' lengths
// in LDS, O(num_reqs) a thread; measured on the mixed batch of 128 decode
// rows and a 2048-token chunk: 0.606 vs 0.644 ms in request order).
constexpr int kVarlenLptMaxReqs = 256;

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int D>
struct PrefillSmem {
  uint4 k[2][kBN * D / 8];        // [key][16-byte chunk ^ k_swizzle(key)]
  uint4 vt[2][kBN * D / 8];       // [key][16-byte chunk ^ v_swizzle(key)] (read transposed)
};

// Position of 16-byte chunk c of tile row r is c ^ swizzle(r).  LDS has 64
// four-byte banks: a 256-byte line is 16 chunks, one row at head size 128,
// two rows at 64.
// K rows are read as 16-byte fragments, 16 consecutive keys at one chunk
// per 16 lanes: their chunks must fall in 16 different 4-bank groups, so
// the swizzle is a bijection on the key's position among 16 (the row's line
// half, r & 1, separates the two rows of a line at head size 64).
template <int D>
__device__ __forceinline__ int k_swizzle(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
// V rows are read by the transposing 64-bit reads: 32 lanes take 4
// consecutive rows x 4 consecutive chunks (64 bytes) at once, so each of the
// 4 rows must put its 4 chunks in a different 4-chunk group (with the
// key-only XOR of K all four rows land in one group: a 4-way bank conflict).
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3))
                  : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Work-group shape: hpw heads x qbw 32-query blocks (hpw * qbw == kWaves).
__host__ __device__ inline void prefill_shape(int G, int& hpw, int& qbw, int& nhc) {
  hpw = G < kWaves ? G : kWaves;                            // heads per work-group
  qbw = kWaves / hpw;                                       // 32-query blocks per work-group
  nhc = (G + kWaves - 1) / kWaves;                          // head chunks per KV head
}

// One work item: query tile `tile` (kQW * qbw queries) of request r, KV head
// group `unit` (KV head unit / nhc, head chunk unit % nhc).
// SHARED (the prefix part of pa_decode_shared_prefix): the decode queries of
// every request, flattened per KV head (query j = (request j / G, head
// g * G + j % G)), against key partition `r` of the prefix the requests
// share (request 0's table), tile `tile` = 128 flattened queries, `unit` = KV
// head; the result is that partition's (m, l, O) partials.  A query sits at
// position seq_len - 1 of its request, so the causal mask below is its
// context bound.
template <int D, bool FP8, bool ALIBI, bool SHARED = false>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, PrefillSmem<D>& sm, int r,
                                             int tile, int unit) {
  constexpr int CH = D / 8;               // 16-byte chunks per bf16 row
  constexpr int KSTEPS = D / 16;          // MFMA k-steps over d
  constexpr int DBLK = D / 32;            // 32-row d blocks of O^T

  // ---- this wave's part of the item
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  int hpw, qbw, nhc;
  prefill_shape(G, hpw, qbw, nhc);
  // the wave index is uniform: keep it (and all per-wave values) scalar
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int lq = lane % 32, lh = lane / 32;

  int g, seq_len, kt_begin, n_tiles, p_q, wave_pmin, wave_pmax, h;
  bool q_ok, wave_on;
  int64_t q_row;                           // query row of this lane (token index)
  const int32_t* bt_row;
  if constexpr (SHARED) {
    g = unit;
    const int nq = a.num_reqs * G;                          // flattened queries of the head
    const int j = (tile * kWaves + w) * kQW + lq;
    q_ok = j < nq;
    const int rq = q_ok ? j / G : 0;
    h = g * G + (q_ok ? j - rq * G : 0);
    q_row = rq;
    seq_len = a.shared_tokens;                              // keys of the prefix
    kt_begin = r * (a.partition_size / kBN);
    n_tiles = min((r + 1) * a.partition_size, seq_len) / kBN;
    p_q = q_ok ? a.seq_lens[rq] - 1 : -1;                   // context bound of the query
    int pmin = q_ok ? p_q : INT32_MAX, pmax = p_q;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      pmin = min(pmin, __shfl_xor(pmin, m, 64));
      pmax = max(pmax, __shfl_xor(pmax, m, 64));
    }
    wave_pmin = __builtin_amdgcn_readfirstlane(pmin);
    wave_pmax = __builtin_amdgcn_readfirstlane(pmax);
    wave_on = true;
    bt_row = a.block_table;                                 // the shared rows: request 0's
  } else {
    const int hc = unit - (unit / nhc) * nhc;
    g = unit / nhc;
    const int qlo = a.query_start_loc[r];
    const int q_len = a.query_start_loc[r + 1] - qlo;
    const int i0 = tile * kQW * qbw;                        // first query of the tile
    seq_len = a.seq_lens[r];
    const int pos0 = seq_len - q_len;                       // position of query 0
    const int hw = w % hpw, qbl = w / hpw;                  // head and query block of the wave
    wave_on = (qbl < qbw) && (hc * kWaves + hw < G);
    h = g * G + hc * kWaves + (wave_on ? hw : 0);
    const int wq0 = i0 + qbl * kQW;                         // first query of the wave
    const int qi = wq0 + lq;                                // query index in request
    q_ok = qi < q_len;
    q_row = qlo + (q_ok ? qi : 0);
    p_q = pos0 + qi;                                        // this lane's query position
    wave_pmin = pos0 + wq0;                                 // first query position of the wave
    wave_pmax = wave_on ? pos0 + min(wq0 + kQW, q_len) - 1 : -1;   // -1: no work
    const int kend = pos0 + min(i0 + kQW * qbw, q_len);     // keys the work-group needs
    kt_begin = 0;
    n_tiles = (kend + kBN - 1) / kBN;
    bt_row = a.block_table + (int64_t)r * a.bt_stride;
  }

  // ---- Q fragments (B operand of S^T = K Q^T): query lq, d = 16k + 8lh .. +8
  uint4 qf[KSTEPS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (q_row * Hq + h) * D;
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      const uint4 v = *reinterpret_cast<const uint4*>(qp + 16 * k + 8 * lh);
      qf[k] = q_ok ? v : make_uint4(0, 0, 0, 0);
    }
  }

  float qk_scale = a.scale * kLog2e;
  if constexpr (FP8) qk_scale *= *a.k_scale;
  // With ALiBi the scores are scaled and biased in place (then sc = 1);
  // otherwise the scale is applied inside the exponent (sc = qk_scale).
  const float slope = ALIBI ? a.alibi_slopes[h] * kLog2e : 0.f;
  const float sc = ALIBI ? 1.f : qk_scale;

  constexpr int EB = FP8 ? 1 : 2;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);

  // ---- FP8: global -> registers -> LDS staging of one 64-key tile (4
  // blocks).  Thread chunk i of K and of V is (key tid/CH + (256/CH) i, 8
  // elements at tid % CH), so rows stream contiguously; the LDS offsets are
  // loop-invariant and computed once.
  constexpr int NCH = kBN * CH / (kWaves * 64);             // chunks per thread per tensor
  const int kc_chunk = tid % CH;
  int k_key[NCH], k_lds[NCH], v_lds[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    k_key[i] = tid / CH + (kWaves * 64 / CH) * i;
    k_lds[i] = k_key[i] * CH + (kc_chunk ^ k_swizzle<D>(k_key[i]));
    v_lds[i] = k_key[i] * CH + (kc_chunk ^ v_swizzle<D>(k_key[i]));
  }
  // the raw codes stay in registers while the current tile is computed and
  // are converted to bf16 only when staged (converting at load time would
  // make the loop wait for the next tile's loads before computing)
  uint2 kraw[NCH], vraw[NCH];
  bool live[NCH];                                           // key of chunk i < seq_len
  auto cvt8 = [](uint2 raw) -> uint4 {                      // 8 codes -> 8 bf16
    const f32x4_t lo = fp8x4_to_f32(raw.x), hi = fp8x4_to_f32(raw.y);
    return make_uint4(pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w),
                      pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w));
  };
  const int64_t head_off = (int64_t)g * (kBlock * D);
  const int64_t blk_stride = (int64_t)Hkv * (kBlock * D);
  // block ids of tile kt's 4 blocks in lanes 0..3 (entries past the context
  // are not read); loaded one tile ahead of the data they address
  auto tile_bids = [&](int kt) -> int32_t {
    const int jb_lane = lane & 3;
    return (kt < n_tiles && kt * kBN + jb_lane * kBlock < seq_len) ? bt_row[kt * 4 + jb_lane] : 0;
  };
  auto fetch = [&](int kt, int32_t bid_vec) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int t = kt * kBN + k_key[i];
      const int jb = __builtin_amdgcn_readfirstlane(k_key[i] / kBlock);
      const int32_t bid = __builtin_amdgcn_readlane(bid_vec, jb);
      const uint8_t* p = kbase + (bid * blk_stride + head_off +
                                  (int64_t)((k_key[i] % kBlock) * D + kc_chunk * 8)) * EB;
      // (unconditional: a key past the context has block id 0, a valid
      // block; its codes are replaced by zeros when staged)
      live[i] = t < seq_len;
      kraw[i] = *reinterpret_cast<const uint2*>(p);
      vraw[i] = *reinterpret_cast<const uint2*>(vbase + (p - kbase));
    }
  };
  // ---- bf16: direct copies.  Wave w copies block w of tile kt (16 keys, the
  // tile's keys 16w .. 16w+15) of K and V; instruction j writes LDS chunks
  // 64j .. 64j+63 of the block, lane i chunk 64j + i, fetching the global
  // chunk that the swizzle puts there.  The block's address is wave-uniform
  // (scalar registers); each lane adds its 32-bit offset in the block.  (The
  // block id is a vector load made uniform when used: a scalar load would
  // share the LDS reads' wait counter and, returning out of order, force
  // full waits on it.)
  auto block_id = [&](int kt) -> int32_t {                  // wave-uniform
    return kt * kBN + kBlock * w < seq_len ? bt_row[kt * 4 + w] : -1;
  };

  uint32_t dma_k[D / 32], dma_v[D / 32];                    // lane byte offsets in a block
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    const int P = 64 * j + lane;
    const int key = P / CH;                                 // key in the block
    dma_k[j] = (uint32_t)((key * D + ((P % CH) ^ k_swizzle<D>(kBlock * w + key)) * 8) * EB);
    dma_v[j] = (uint32_t)((key * D + ((P % CH) ^ v_swizzle<D>(kBlock * w + key)) * 8) * EB);
  }
  auto dma = [&](int kt, int32_t bid_v, int buf) {
    (void)kt;
    const int32_t bid = __builtin_amdgcn_readfirstlane(bid_v);
    if (bid < 0) return;                                    // block past the context
    const int64_t base = ((int64_t)bid * blk_stride + head_off) * EB;
    const uint8_t* kblk = kbase + base;
    const uint8_t* vblk = vbase + base;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const int slot = kBlock * CH * w + 64 * j;
      // (destinations as plain LDS offsets: the copies' completion is
      // awaited explicitly before the barrier that publishes the buffer,
      // and the compiler then adds no wait before reads of the other one)
      __builtin_amdgcn_global_load_lds((const void*)(kblk + dma_k[j]),
                                       (lds_void_t*)(uintptr_t)lds_offset(&sm.k[buf][slot]),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vblk + dma_v[j]),
                                       (lds_void_t*)(uintptr_t)lds_offset(&sm.vt[buf][slot]),
                                       16, 0, 0);
    }
  };
  // once this wave's copies have landed: zero the V rows of its block past
  // the context (unwritten slots may hold NaN, and P = 0 times NaN is NaN;
  // K rows there are masked by select)
  auto zero_tail = [&](int kt, int buf) {
    const int t0 = kt * kBN + kBlock * w;
    if (t0 + kBlock <= seq_len) return;                     // wave-uniform
    uint4* vl = &sm.vt[buf][kBlock * CH * w];
    for (int idx = lane; idx < kBlock * CH; idx += 64)
      if (t0 + idx / CH >= seq_len) vl[idx] = make_uint4(0, 0, 0, 0);
  };
  auto wait_copies = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // FP8: K and V rows, converted to bf16, in the same swizzled row-major
  // layout the bf16 copies produce (V^T fragments then come from the
  // transposing LDS reads, as for bf16 caches)
  auto stage = [&](int buf) {
    uint4* kl = &sm.k[buf][0];
    uint4* vl = &sm.vt[buf][0];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      kl[k_lds[i]] = live[i] ? cvt8(kraw[i]) : make_uint4(0, 0, 0, 0);
      vl[v_lds[i]] = live[i] ? cvt8(vraw[i]) : make_uint4(0, 0, 0, 0);
    }
  };

  // ---- running state of this lane's query (keys split between lane halves);
  // m_run is in scaled log2 units, scores s are raw dot products (times sc).
  float m_run = -INFINITY, l_run = 0.f;
  float m_true = -INFINITY;                 // exact max (partials of SHARED)
  f32x16_t oacc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[b][v] = 0.f;

  // Byte offsets in a V buffer of this lane's transposing reads, k-step 0:
  // the V^T fragment of d block db (d = 32db + lane % 32) over keys
  // 16ks + 4lh + 8(t/4) + t%4 for element t -- the order of P^T's k-step
  // (b, s') = (ks/2, ks%2) -- comes from rows 4lh + gi/4 + 8hp (+16ks) of
  // row-major V: lane gi of 16-lane group Gr addresses elements
  // 32db + 16(Gr&1) + 4(gi%4) .. +3 of that row, and the transpose hands lane
  // gi those rows' element 32db + 16(Gr&1) + gi.  Constant over the tiles.
  uint32_t vt_off[DBLK][2];
  {
    const int Gr = lane / 16, gi = lane % 16;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        const int r = 4 * lh + gi / 4 + 8 * hp;
        const int e0 = 32 * db + 16 * (Gr & 1) + 4 * (gi % 4);
        vt_off[db][hp] = 16 * (r * CH + ((e0 / 8) ^ v_swizzle<D>(r))) + 2 * (e0 % 8);
      }
  }

  int32_t bid_next = -1;                     // the block id of tile kt + 1
  if constexpr (FP8) {
    fetch(kt_begin, tile_bids(kt_begin));
    bid_next = tile_bids(kt_begin + 1);
    stage(0);
  } else {
    if (kt_begin + 1 < n_tiles) bid_next = block_id(kt_begin + 1);
    dma(kt_begin, block_id(kt_begin), 0);
    wait_copies();
    zero_tail(kt_begin, 0);
  }
  __syncthreads();

  for (int kt = kt_begin; kt < n_tiles; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    const bool more = kt + 1 < n_tiles;
    if constexpr (FP8) {
      if (more) {
        fetch(kt + 1, bid_next);
        bid_next = tile_bids(kt + 2);
      }
    }
    const int k0 = kt * kBN;
    const bool compute = k0 <= wave_pmax;       // some key of the tile is visible to the wave
    f32x16_t s[2];
    if (compute) {
      // -- S^T = K Q^T for the two 32-key halves of the tile
      // (the two halves' MFMA chains interleaved: consecutive MFMAs are
      // independent while the next K fragments are read)
      // (K fragments read one k-step ahead of their products, two pairs
      // in flight)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[b][v] = 0.f;
      auto kread = [&](int k, int b) -> uint4 {
        const int key = 32 * b + lq;
        return sm.k[buf][key * CH + ((2 * k + lh) ^ k_swizzle<D>(key))];
      };
      uint4 kf[2][2];
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int b = 0; b < 2; ++b) kf[k][b] = kread(k, b);
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {
#pragma unroll
        for (int b = 0; b < 2; ++b) s[b] = mfma32(kf[k & 1][b], qf[k], s[b]);
        if (k + 2 < KSTEPS) {
#pragma unroll
          for (int b = 0; b < 2; ++b) kf[k & 1][b] = kread(k + 2, b);
        }
      }
      // keep that order: 4 reads, then (2 products, 2 reads) per k-step
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int k = 0; k + 2 < KSTEPS; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    // bf16: the next tile's copy, issued by every wave (each copies its own
    // block) after this tile's QK products: while a copy is in flight the
    // compiler waits for all outstanding LDS reads at once, which the QK
    // fragment reads, one k-step ahead, cannot afford
    if constexpr (!FP8) {
      if (more) {
        dma(kt + 1, bid_next, buf ^ 1);
        if (kt + 2 < n_tiles) bid_next = block_id(kt + 2);
      }
    }
    if (compute) {
      // -- ALiBi: s <- s * qk_scale + slope * (t - p_q)
      if constexpr (ALIBI) {
        const float bias0 = slope * (float)(k0 + 4 * lh - p_q);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            s[b][v] = fmaf(s[b][v], qk_scale,
                           fmaf(slope, (float)(32 * b + 8 * (v / 4) + (v % 4)), bias0));
      }
      // -- causal mask by select (diagonal tiles only), tile max
      if (k0 + kBN - 1 > wave_pmin) {
        // key k0 + c (c = 32b + 8(v/4) + 4lh + v%4) is visible iff c <= p_q - k0
        const int lim = p_q - k0 - 4 * lh;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            s[b][v] = (32 * b + 8 * (v / 4) + (v % 4) <= lim) ? s[b][v] : -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s[b][v]);
      tmax = max_xor32(tmax) * sc;
      if constexpr (SHARED) m_true = fmaxf(m_true, tmax);
      // -- lazy rescale: move the max only when it grows by more than 2^8.
      // Key 0 is visible to every query, so m_run is finite after tile 0.
      if (tmax > m_run + 8.0f) {
        const float alpha = fast_exp2(m_run - tmax);         // 0 on the first tile
        m_run = tmax;
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < DBLK; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[b][v] *= alpha;
      }
      // -- P^T as bf16 B operands: k-step (b, s') takes accumulator rows
      // 8s'..8s'+7.  The row sum l takes the same bf16-rounded weights that
      // multiply V, so O = sum(p~ v) / sum(p~) is an exact weighted average:
      // a rounding (2^-9 relative per weight) moves O by at most 2^-9 times
      // the spread of v about O, and a one-hot row gives its v exactly.
      // (Summing the unrounded p instead leaves a bias of the same order
      // times |v|, which took peaked rows past the tolerance.)
      uint4 pf[4];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            p[e] = fast_exp2(fmaf(s[b][8 * sp + e], sc, -m_run));   // -inf -> 0
          uint32_t hw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hw[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
            l_run = dot2_bf16(hw[e], 0x3f803f80u, l_run);   // + both rounded weights
          }
          pf[2 * b + sp] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        }
      // -- O^T += V^T P^T
      {
        // V^T fragments by two transposing reads each (offsets vt_off;
        // k-step ks reads 16 rows further down)
        const char* vbuf = reinterpret_cast<const char*>(&sm.vt[buf][0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {             // (d blocks' chains interleaved)
#pragma unroll
          for (int db = 0; db < DBLK; ++db) {
            const uint4 vf = lds_read_tr16_pair(vbuf + vt_off[db][0] + ks * (16 * D * 2),
                                                vbuf + vt_off[db][1] + ks * (16 * D * 2));
            oacc[db] = mfma32(vf, pf[ks], oacc[db]);
          }
        }
      }
    }
    if (more) {
      if constexpr (FP8) {
        stage(buf ^ 1);
      } else {
        wait_copies();
        zero_tail(kt + 1, buf ^ 1);
      }
    }
    __syncthreads();
  }

  // ---- finalize: l over both lane halves, O = A / l, write bf16 rows (or
  // the partition's partials: max logit in natural-log units, exp-sum
  // relative to it, O normalised -- the split-KV record of P1 §3.2.7)
  const float l_tot = sum_xor32(l_run);
  if constexpr (SHARED) {
    if (q_ok) {
      const bool any = l_tot > 0.f;          // false: no key of the partition is visible
      float inv = any ? 1.f / l_tot : 0.f;
      if constexpr (FP8) inv *= *a.v_scale;
      const int64_t idx = (q_row * Hq + h) * a.max_num_partitions + r;
      float* op = a.tmp_out + idx * D;
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 32 * db + 8 * i + 4 * lh;
          // (select, not a product: with no key the accumulators hold NaN)
          *reinterpret_cast<f32x4_t*>(op + d) =
              any ? f32x4_t{oacc[db][4 * i + 0] * inv, oacc[db][4 * i + 1] * inv,
                            oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv}
                  : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      if (lh == 0) {
        a.max_logits[idx] = any ? m_true * kLn2 : -INFINITY;
        a.exp_sums[idx] = any ? l_tot * fast_exp2(m_run - m_true) : 0.f;
      }
    }
    return;
  }
  if (q_ok && wave_on) {
    float inv = 1.f / l_tot;
    if constexpr (FP8) inv *= *a.v_scale;
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (q_row * Hq + h) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * db + 8 * i + 4 * lh;
        const uint32_t w0 = (uint32_t)f32_to_bf16(oacc[db][4 * i + 0] * inv) |
                            ((uint32_t)f32_to_bf16(oacc[db][4 * i + 1] * inv) << 16);
        const uint32_t w1 = (uint32_t)f32_to_bf16(oacc[db][4 * i + 2] * inv) |
                            ((uint32_t)f32_to_bf16(oacc[db][4 * i + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + d) = make_uint2(w0, w1);
      }
  }
}

// The work items are the query tiles of the requests with q_len > 1, in
// request order, times the KV-head groups: item k is flattened tile k / U of
// KV-head group k % U (U = num_kv_heads * nhc).  Wave 0 of a work-group finds
// the request holding a flattened tile by a running prefix over the
// requests' tile counts, 64 requests per step.  Work-groups take items
// blockIdx.x, blockIdx.x + gridDim.x, ...; the grid is sized by a bound on
// the tile count (decode rows cost no work-groups).
// With direct != 0 (few requests) the grid is (tiles * U, num_reqs) instead:
// one item per work-group, request blockIdx.y, no search.
// Work items k = first, first + stride, ... (k < num_items) of one
// work-group; with snake, its j-th item is j * stride + first for even j and
// (j + 1) * stride - 1 - first for odd j (persistent workers then pair the
// long query tiles of a causal chunk with the short ones).
// With DIRECT, the work-group's one item is (request blockIdx.y, tile
// blockIdx.x / U, group blockIdx.x % U) instead.
template <int D, bool FP8, bool ALIBI, bool DIRECT = false>
__device__ __forceinline__ void prefill_items(const PrefillArgs& a, PrefillSmem<D>& sm,
                                              int* sched, int64_t first, int64_t stride,
                                              int64_t num_items, bool snake) {
  int hpw, qbw, nhc;
  prefill_shape(a.num_q_heads / a.num_kv_heads, hpw, qbw, nhc);
  const int U = a.num_kv_heads * nhc;
  const int QT = kQW * qbw;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int64_t j = 0;; ++j) {
    const int64_t k = (snake && (j & 1)) ? (j + 1) * stride - 1 - first : j * stride + first;
    if constexpr (DIRECT) {
      const int r = blockIdx.y, tile = blockIdx.x / U;
      const int q_len = a.query_start_loc[r + 1] - a.query_start_loc[r];
      if (j > 0 || q_len <= 1 || tile * QT >= q_len) break;
      prefill_item<D, FP8, ALIBI>(a, sm, r, tile, blockIdx.x % U);
      continue;
    }
    if (k >= num_items) break;
    const int64_t kt = k / U;
    if (w == 0) {
      int64_t base = 0;
      int found_r = -1, found_t = 0;
      for (int r0 = 0; r0 < a.num_reqs && found_r < 0; r0 += 64) {
        const int rr = r0 + lane;
        int nt = 0;
        if (rr < a.num_reqs) {
          const int ql = a.query_start_loc[rr + 1] - a.query_start_loc[rr];
          nt = ql > 1 ? (ql + QT - 1) / QT : 0;
        }
        int incl = nt;                                       // inclusive prefix in the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int v = __shfl_up(incl, off, 64);
          if (lane >= off) incl += v;
        }
        const int excl = incl - nt;
        const bool mine = nt > 0 && kt >= base + excl && kt < base + incl;
        const uint64_t m = __builtin_amdgcn_ballot_w64(mine);
        if (m != 0) {
          const int src = __builtin_ctzll(m);
          found_r = r0 + src;
          found_t = (int)(kt - base - __shfl(excl, src, 64));
        }
        base += __shfl(incl, 63, 64);
      }
      if (lane == 0) {
        sched[0] = found_r;
        sched[1] = found_t;
      }
    }
    __syncthreads();
    // uniform across the work-group: keep them scalar
    const int r = __builtin_amdgcn_readfirstlane(sched[0]);
    const int tile = __builtin_amdgcn_readfirstlane(sched[1]);
    __syncthreads();
    if (r < 0) break;            // past the last tile (later items are larger still)
    prefill_item<D, FP8, ALIBI>(a, sm, r, tile, (int)(k % U));
    __syncthreads();
  }
}

// The work items are the query tiles of the requests with q_len > 1, in
// request order, times the KV-head groups: item k is flattened tile k / U of
// KV-head group k % U (U = num_kv_heads * nhc).  Wave 0 of a work-group finds
// the request holding a flattened tile by a running prefix over the
// requests' tile counts, 64 requests per step.  Work-groups take items
// blockIdx.x, blockIdx.x + gridDim.x, ...; the grid is sized by a bound on
// the tile count (decode rows cost no work-groups).
// With direct != 0 (few requests) the grid is (tiles * U, num_reqs) instead:
// one item per work-group, request blockIdx.y, no search.
template <int D, bool FP8, bool ALIBI, bool DIRECT>
__global__ __launch_bounds__(kWaves * 64, 2) void prefill_kernel(PrefillArgs a,
                                                                 int64_t num_items) {
  __shared__ PrefillSmem<D> sm;
  __shared__ int sched[2];
  prefill_items<D, FP8, ALIBI, DIRECT>(a, sm, sched, blockIdx.x, gridDim.x, num_items, false);
}

// Shared-prefix partials: work-group (query block of 128 flattened decode
// queries, key partition, KV head).
template <int D, bool FP8, bool ALIBI>
__global__ __launch_bounds__(kWaves * 64, 2) void shared_prefix_kernel(PrefillArgs a) {
  __shared__ PrefillSmem<D> sm;
  prefill_item<D, FP8, ALIBI, true>(a, sm, blockIdx.y, blockIdx.x, blockIdx.z);
}

// Prefill tiles and decode rows of one varlen batch in one launch (bf16
// caches, vector-ALU decode).  The grid is three runs of work-groups, handed
// out in order: n_first prefill items (one each), then the n_dec (decode
// row, KV head x head chunk) units, longest rows first (with a.lpt), then
// the remaining prefill items.  Free slots of the compute units are
// refilled from the next run as work-groups finish, so the MFMA/LDS-bound
// prefill and the HBM-bound decode share the compute units instead of
// running one after the other, and the decode rows that start last are the
// short ones.
template <int D, bool ALIBI, int GC>
__global__ __launch_bounds__(kWaves * 64, 2) void varlen_kernel(PrefillArgs p, DecodeArgs a,
                                                                int64_t num_items, int n_first,
                                                                int n_dec, int n_chunks) {
  __shared__ union {
    PrefillSmem<D> pf;
    DecodeSmem<D, GC, false, kWaves> dc;
  } sm;
  __shared__ int sched[2];
  const int b = blockIdx.x;
  if (b < n_first || b >= n_first + n_dec) {
    const int64_t item = b < n_first ? b : (int64_t)b - n_dec;
    prefill_items<D, false, ALIBI>(p, sm.pf, sched, item, num_items, num_items, false);
    return;
  }
  const int u = b - n_first;
  const int U = a.num_kv_heads * n_chunks;
  int r = u / U;
  if (a.lpt) {
    // longest decode rows first: unit u takes the (u / U)-th longest row
    // with q_len 1 (ties by index; the other rows rank last and exit)
    const int R = a.num_reqs;
    int32_t* key = sm.dc.bt;
    for (int i = threadIdx.x; i < R; i += kWaves * 64)
      key[i] = a.query_start_loc[i + 1] - a.query_start_loc[i] == 1 ? a.seq_lens[i] : -1;
    __syncthreads();
    for (int j = threadIdx.x; j < R; j += kWaves * 64) {
      const int kj = key[j];
      int rank = 0;
      for (int k = 0; k < R; ++k) rank += (key[k] > kj || (key[k] == kj && k < j)) ? 1 : 0;
      if (rank == r) sched[0] = j;
    }
    __syncthreads();
    r = __builtin_amdgcn_readfirstlane(sched[0]);
    __syncthreads();
  }
  decode_unit<D, GC, false, kWaves, false, PA_VARLEN_DECODE_PREFETCH>(a, sm.dc, r, u % U, 0,
                                                                      n_chunks);
}

// Compute units of the current device (cached per device; 0 if unknown).
static int cu_count() {
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

// Prefill items of a launch: an upper bound on the query tiles of the
// requests with q_len > 1, times the KV-head groups.  Tiles <= sum over the
// prefill requests of (q_len / QT + 1) <= T / QT + #prefill requests, with
// #prefill requests <= min(num_reqs, T / 2) and each tile count <=
// ceil(max_query_len / QT).
static int64_t prefill_item_bound(const PrefillArgs& a) {
  int hpw, qbw, nhc;
  prefill_shape(a.num_q_heads / a.num_kv_heads, hpw, qbw, nhc);
  const int QT = kQW * qbw;
  const int64_t T = a.num_tokens;
  const int64_t per_req = (a.max_query_len + QT - 1) / QT;
  const int64_t nreq_bound = std::min<int64_t>(a.num_reqs, T / 2);
  const int64_t tiles = std::min<int64_t>((T + QT - 1) / QT + nreq_bound, per_req * nreq_bound);
  return tiles * a.num_kv_heads * nhc;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.num_reqs == 0 || a.max_query_len <= 1) return hipSuccess;
  int hpw, qbw, nhc;
  prefill_shape(a.num_q_heads / a.num_kv_heads, hpw, qbw, nhc);
  const int QT = kQW * qbw;
  const int64_t per_req = (a.max_query_len + QT - 1) / QT;
  const int64_t num_items = prefill_item_bound(a);
  if (num_items == 0) return hipSuccess;
  // few requests: the direct grid wastes at most a few work-groups
  const int direct = a.num_reqs <= 4 ? 1 : 0;
  dim3 grid((unsigned)std::min<int64_t>(num_items, kMaxPrefillGroups));
  if (direct) grid = dim3((unsigned)(per_req * a.num_kv_heads * nhc), a.num_reqs);
  const bool fp8 = a.cache_dtype != 0;
  const bool alibi = a.alibi_slopes != nullptr;
#define PA_PREFILL(DV, F8, AL)                                                              \
  do {                                                                                      \
    if (direct)                                                                             \
      hipLaunchKernelGGL((prefill_kernel<DV, F8, AL, true>), grid, dim3(kWaves * 64), 0, st, a, \
                         num_items);                                                        \
    else                                                                                    \
      hipLaunchKernelGGL((prefill_kernel<DV, F8, AL, false>), grid, dim3(kWaves * 64), 0, st,   \
                         a, num_items);                                                     \
  } while (0)
  if (a.head_dim == 64) {
    if (fp8) {
      if (alibi) PA_PREFILL(64, true, true); else PA_PREFILL(64, true, false);
    } else {
      if (alibi) PA_PREFILL(64, false, true); else PA_PREFILL(64, false, false);
    }
  } else {
    if (fp8) {
      if (alibi) PA_PREFILL(128, true, true); else PA_PREFILL(128, true, false);
    } else {
      if (alibi) PA_PREFILL(128, false, true); else PA_PREFILL(128, false, false);
    }
  }
#undef PA_PREFILL
  return hipGetLastError();
}

hipError_t launch_shared_prefix(const PrefillArgs& a, hipStream_t st) {
  if (a.num_reqs == 0 || a.shared_tokens <= 0) return hipSuccess;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t nq = (int64_t)a.num_reqs * G;
  const dim3 grid((unsigned)((nq + kWaves * kQW - 1) / (kWaves * kQW)),
                  (unsigned)(a.shared_tokens / a.partition_size), (unsigned)a.num_kv_heads);
  const bool fp8 = a.cache_dtype != 0;
  const bool alibi = a.alibi_slopes != nullptr;
#define PA_SHARED(DV, F8, AL) \
  hipLaunchKernelGGL((shared_prefix_kernel<DV, F8, AL>), grid, dim3(kWaves * 64), 0, st, a)
  if (a.head_dim == 64) {
    if (fp8) {
      if (alibi) PA_SHARED(64, true, true); else PA_SHARED(64, true, false);
    } else {
      if (alibi) PA_SHARED(64, false, true); else PA_SHARED(64, false, false);
    }
  } else {
    if (fp8) {
      if (alibi) PA_SHARED(128, true, true); else PA_SHARED(128, true, false);
    } else {
      if (alibi) PA_SHARED(128, false, true); else PA_SHARED(128, false, false);
    }
  }
#undef PA_SHARED
  return hipGetLastError();
}

bool varlen_fused_applies(const PrefillArgs& p) {
  if (!PA_VARLEN_FUSED || p.cache_dtype != 0 || p.max_query_len <= 1 || p.num_reqs < 2)
    return false;
  const int G = p.num_q_heads / p.num_kv_heads;
  if (G >= 8) return false;                     // decode rows on the matrix cores
  const int cus = cu_count();
  // at least one round of decode work-groups besides the prefill rows
  return cus > 0 && (int64_t)(p.num_reqs - 1) * p.num_kv_heads >= cus;
}

template <int D, int GC>
static hipError_t launch_varlen_t(const PrefillArgs& p, const DecodeArgs& a, hipStream_t st) {
  const int64_t num_items = prefill_item_bound(p);
  const int n_first = (int)std::min<int64_t>(num_items, (int64_t)PA_VARLEN_FIRST * cu_count());
  const int n_chunks = 1;                       // GC == G here (G < 8)
  const int n_dec = a.num_reqs * a.num_kv_heads * n_chunks;
  const int64_t groups = num_items + n_dec;
  if (p.alibi_slopes)
    hipLaunchKernelGGL((varlen_kernel<D, true, GC>), dim3((unsigned)groups), dim3(kWaves * 64), 0,
                       st, p, a, num_items, n_first, n_dec, n_chunks);
  else
    hipLaunchKernelGGL((varlen_kernel<D, false, GC>), dim3((unsigned)groups), dim3(kWaves * 64), 0,
                       st, p, a, num_items, n_first, n_dec, n_chunks);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_varlen_d(const PrefillArgs& p, const DecodeArgs& a, hipStream_t st) {
  switch (p.num_q_heads / p.num_kv_heads) {
    case 1: return launch_varlen_t<D, 1>(p, a, st);
    case 2: return launch_varlen_t<D, 2>(p, a, st);
    case 3: return launch_varlen_t<D, 3>(p, a, st);
    case 4: return launch_varlen_t<D, 4>(p, a, st);
    case 5: return launch_varlen_t<D, 5>(p, a, st);
    case 6: return launch_varlen_t<D, 6>(p, a, st);
    default: return launch_varlen_t<D, 7>(p, a, st);
  }
}

hipError_t launch_varlen(const PrefillArgs& p, const DecodeArgs& a, hipStream_t st) {
  DecodeArgs b = a;
  b.lpt = a.num_reqs <= kVarlenLptMaxReqs ? 1 : 0;
  return p.head_dim == 64 ? launch_varlen_d<64>(p, b, st) : launch_varlen_d<128>(p, b, st);
}

}  // namespace pa
