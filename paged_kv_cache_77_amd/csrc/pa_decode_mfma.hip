// Paged decode on the matrix cores (gfx950): FP8 caches, and bf16 caches
// with large GQA groups.
//
// Same result as decode_kernel ("vLLM 深度解析（二）：PagedAttention 核心机制"
// §3.2: block-table walk, scaled q.k of the query heads sharing a KV head,
// masked tail, softmax, PV; §2.2: the running (m, l, A) state; §3.2.7 for the
// split-KV partials).  Where the vector ALU, not memory, is the limit (FP8
// caches: four conversions per code; bf16 caches: work per token that grows
// with the group) the two products of a 16-token block run as MFMAs with the
// GQA group's query heads on the N side (16 per chunk; unused columns are
// zero queries):
//
//   S^T[16 tokens x 16 heads]  = K . Q^T   v_mfma_f32_16x16x32_{f16,bf16},
//       D/32 steps; lane l supplies K row (token) l%16, d = (D/4)(l/16) + 8s
//       .. +8 for step s, so its D/4 contiguous elements are one load; Q^T
//       is permuted alike.  The accumulator leaves lane l with tokens
//       4(l/16)+i of head l%16.
//   O^T[D x 16 heads] += V^T . P^T          v_mfma_f32_16x16x16_{f16,bf16},
//       D/16 steps; P^T is the lane's own four probabilities, V^T row m of
//       d-block db is d = (D/16)m + db, so lane l loads D/16 contiguous
//       elements of each of its four tokens and shuffles them into pairs
//       (exact).  The accumulator leaves lane l with d = (D/4)(l/16) +
//       (D/16)i + db of head l%16 -- the same head as its softmax state.
//
// FP8: codes convert exactly to f16; q enters as f16 after a per-head power
// of two (exact for bf16 values in range, see load_q); probabilities are f16
// for the PV product (relative error <= 2^-11 per weight).  bf16: K, V and q
// enter unchanged; probabilities are split into two bf16 terms (about 16
// significant bits).  l and the max stay fp32; softmax in log2 units with
// the lazy running max of decode_kernel.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int kMHeads = 16;       // query heads per chunk (the MFMA N side)
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif
constexpr int kMWaves = PA_MFMA_WAVES;
#ifndef PA_MFMA_LPT_MAX
#define PA_MFMA_LPT_MAX 128
#endif
constexpr int kMaxLptReqs = PA_MFMA_LPT_MAX;   // longest-first order up to this batch
constexpr int kMBtChunk = 1024;
constexpr float kMTau = 8.0f;
#ifndef PA_MFMA_PREFETCH
#define PA_MFMA_PREFETCH 2
#endif
constexpr int kMPrefetch = PA_MFMA_PREFETCH;   // tiles in flight per wave
#ifndef PA_MFMA_PREFETCH_BF16
#define PA_MFMA_PREFETCH_BF16 2
#endif
constexpr int kMPrefetchB = PA_MFMA_PREFETCH_BF16;   // bf16 tiles are twice the bytes
#ifndef PA_MFMA_MINW_BF16
#define PA_MFMA_MINW_BF16 1
#endif
// FP8 work-groups fit 4 per CU at 128 VGPRs with 2 tiles in flight (the
// whole shared-prefix grid resident at once: 4% faster than 3 per CU with a
// 3-tile ring; a 3-tile ring at 128 VGPRs spills, and so would ALiBi, which
// gets 3 per CU)
#ifndef PA_MFMA_MINW_FP8
#define PA_MFMA_MINW_FP8 4
#endif

template <int D>
struct MfmaDecodeSmem {
  int32_t bt[kMBtChunk];
  float m[kMWaves][kMHeads];
  float mt[kMWaves][kMHeads];
  float l[kMWaves][kMHeads];
  float acc[kMWaves][kMHeads][D];
  int32_t sched;
};

template <int D>
struct MTile {
  uint4 k[D / 64];               // D/4 codes of one K row (16 bytes each)
  uint32_t v[4][D / 64];         // D/16 codes of each of four V rows
};

template <int D>
__device__ __forceinline__ void mload(MTile<D>& t, const uint8_t* kbase, const uint8_t* vbase,
                                      int32_t phys, int g, int num_kv_heads, int lane) {
  const int64_t off = tile_offset(phys, g, num_kv_heads, D);      // bytes (1 per code)
  const int row = lane % 16, grp = lane / 16;
  const uint8_t* kp = kbase + off + row * D + (D / 4) * grp;
#pragma unroll
  for (int c = 0; c < D / 64; ++c) t.k[c] = *reinterpret_cast<const uint4*>(kp + 16 * c);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint8_t* vp = vbase + off + (4 * grp + e) * D + (D / 16) * row;
    if constexpr (D / 64 == 2) {
      const uint2 w = *reinterpret_cast<const uint2*>(vp);
      t.v[e][0] = w.x;
      t.v[e][1] = w.y;
    } else {
      t.v[e][0] = *reinterpret_cast<const uint32_t*>(vp);
    }
  }
}

template <int D, bool ALIBI>
struct MfmaDecoder {
  static constexpr int KS = D / 32;       // QK steps
  static constexpr int DB = D / 16;       // PV d-blocks
  int lane, col, grp;
  float qk_scale;                         // per lane: head col's scale (log2 units)
  float alibi;
  int pos_q;
  uint32_t qf[KS][4];                     // Q^T operand: 8 f16 per step
  float m_run, m_true, l_part;            // head col (replicated in the 4 lane groups)
  f32x4_t oacc[DB];                       // MFMA accumulators, used in place

  __device__ __forceinline__ void init(int lane_) {
    lane = lane_;
    col = lane % 16;
    grp = lane / 16;
    alibi = 0.f;
    pos_q = 0;
  }

  // q of row row_q, heads h0 .. h0+nh-1 (column col; others zero), as f16
  // scaled by a power of two 2^e per head (max |q| of the head lands in
  // [2^14, 2^15), where f16 holds every bf16 value exactly; only elements
  // below 2^-17 of the head's largest could round, far under the fp32
  // rounding of the dot product).  The scores are scaled back by 2^-e.
  __device__ __forceinline__ void load_q(const uint16_t* q, int64_t row_q, int num_q_heads,
                                         int h0, int nh, const float* slopes, int seq_len,
                                         float scale_log2) {
    const bool real = col < nh;
    const uint16_t* qh = q + (row_q * num_q_heads + h0 + (real ? col : 0)) * D + (D / 4) * grp;
    uint32_t raw[KS][4];
    float amax = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 v = *reinterpret_cast<const uint4*>(qh + 8 * s);
      raw[s][0] = real ? v.x : 0u;
      raw[s][1] = real ? v.y : 0u;
      raw[s][2] = real ? v.z : 0u;
      raw[s][3] = real ? v.w : 0u;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        amax = fmaxf(amax, fmaxf(fabsf(bf16lo(raw[s][u])), fabsf(bf16hi(raw[s][u]))));
    }
    amax = max_xor16(amax);
    amax = max_xor32(amax);      // max |q| of head col
    // exponent e with amax * 2^e in [2^14, 2^15); 0 for an all-zero head
    int e = 0;
    if (amax > 0.f && amax < INFINITY) e = 14 - (int)((__float_as_uint(amax) >> 23) & 0xff) + 127;
    const float up = __uint_as_float((uint32_t)(127 + max(-126, min(127, e))) << 23);
    const float down = __uint_as_float((uint32_t)(127 + max(-126, min(127, -e))) << 23);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        qf[s][u] = pack_f16x2(bf16lo(raw[s][u]) * up, bf16hi(raw[s][u]) * up);
    qk_scale = scale_log2 * down;
    pos_q = seq_len - 1;
    if constexpr (ALIBI) alibi = real ? slopes[h0 + col] * kLog2e : 0.f;
  }

  __device__ __forceinline__ void reset() {
    m_run = -INFINITY;
    m_true = -INFINITY;
    l_part = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) oacc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  __device__ __forceinline__ void compute(const MTile<D>& t, int tok0, int t_end) {
    // -- S^T = K Q^T (codes to exact f16 pairs)
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const uint4 raw = t.k[st / 2];
      const uint32_t w0 = (st & 1) ? raw.z : raw.x;
      const uint32_t w1 = (st & 1) ? raw.w : raw.y;
      const uint4 kb = make_uint4(fp8x2_to_f16x2<false>(w0), fp8x2_to_f16x2<true>(w0),
                                  fp8x2_to_f16x2<false>(w1), fp8x2_to_f16x2<true>(w1));
      const uint4 qb = make_uint4(qf[st][0], qf[st][1], qf[st][2], qf[st][3]);
      s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, kb),
                                                 __builtin_bit_cast(f16x8_t, qb), s, 0, 0, 0);
    }
    const bool full = tok0 + kBlock <= t_end;      // uniform
    // -- scaled scores of tokens tok0 + 4grp + i (past the context: -inf)
    float x[4];
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tok0 + 4 * grp + i;
      float xv = s[i] * qk_scale;
      if constexpr (ALIBI) xv = fmaf(alibi, (float)(tok - pos_q), xv);
      x[i] = (full || tok < t_end) ? xv : -INFINITY;
      bm = fmaxf(bm, x[i]);
    }
    bm = max_xor16(bm);
    bm = max_xor32(bm);            // max over the head's 16 tokens
    m_true = fmaxf(m_true, bm);
    const bool grow = bm > m_run + kMTau;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // wave-uniform and rare: move the max
      const float m_new = grow ? bm : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) oacc[b] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(x[i] - m_run);             // exp2(-inf) = 0 for masked tokens
      l_part += p[i];
    }
    const uint2 pt = make_uint2(pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]));
    // -- O^T += V^T P^T; in a partial block the rows past the context are
    // zeroed (they may hold NaN, and 0 * NaN would poison the sum)
    uint32_t w[4][D / 64];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int c = 0; c < D / 64; ++c) w[e][c] = t.v[e][c];
    if (!full) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool live = tok0 + 4 * grp + e < t_end;
#pragma unroll
        for (int c = 0; c < D / 64; ++c) w[e][c] = live ? w[e][c] : 0u;
      }
    }
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      // bytes j of the four rows' words, gathered per d-block db = 4c + j
      const uint32_t a01 = perm_bytes(w[1][c], w[0][c], 0x05010400u);  // t0b0 t1b0 t0b1 t1b1
      const uint32_t b01 = perm_bytes(w[1][c], w[0][c], 0x07030602u);  // t0b2 t1b2 t0b3 t1b3
      const uint32_t a23 = perm_bytes(w[3][c], w[2][c], 0x05010400u);
      const uint32_t b23 = perm_bytes(w[3][c], w[2][c], 0x07030602u);
      const uint32_t xs[4] = {perm_bytes(a23, a01, 0x05040100u), perm_bytes(a23, a01, 0x07060302u),
                              perm_bytes(b23, b01, 0x05040100u), perm_bytes(b23, b01, 0x07060302u)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 vt = make_uint2(fp8x2_to_f16x2<false>(xs[j]), fp8x2_to_f16x2<true>(xs[j]));
        const int b = 4 * c + j;
        oacc[b] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, vt),
                                                        __builtin_bit_cast(f16x4_t, pt), oacc[b],
                                                        0, 0, 0);
      }
    }
  }

  // l over the four lane groups (every lane of a head then holds it)
  __device__ __forceinline__ void finish() {
    l_part = sum_xor16(l_part);
    l_part = sum_xor32(l_part);
  }
};

// ---------------------------------------------------------------------------
// bf16 caches: the same two products with bf16 operands.  K rows need no
// conversion; V^T pairs are 16-bit shuffles; P^T is split into a bf16 high
// part and a bf16 remainder (two MFMAs), so the probabilities keep ~16
// significant bits -- bf16 alone (8 bits) would cost more accuracy than the
// output's own rounding allows on peaked softmaxes.
template <int D>
struct MTileB {
  uint4 k[D / 32];               // D/4 bf16 of one K row (8 per step)
  uint32_t v[4][D / 32];         // D/16 bf16 of each of four V rows
};

// (plain loads: each load instruction covers part of every cache line of
// the tile, so streaming loads, which do not keep the line, re-fetch it)
template <int D>
__device__ __forceinline__ void mloadB(MTileB<D>& t, const uint8_t* kbase, const uint8_t* vbase,
                                       int32_t phys, int g, int num_kv_heads, int lane) {
  const int64_t off = tile_offset(phys, g, num_kv_heads, D) * 2;     // bytes
  const int row = lane % 16, grp = lane / 16;
  const uint8_t* kp = kbase + off + (row * D + (D / 4) * grp) * 2;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) t.k[c] = *reinterpret_cast<const uint4*>(kp + 16 * c);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint8_t* vp = vbase + off + ((4 * grp + e) * D + (D / 16) * row) * 2;
    if constexpr (D / 32 == 4) {
      const uint4 w = *reinterpret_cast<const uint4*>(vp);
      t.v[e][0] = w.x; t.v[e][1] = w.y; t.v[e][2] = w.z; t.v[e][3] = w.w;
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(vp);
      t.v[e][0] = w.x; t.v[e][1] = w.y;
    }
  }
}

template <int D, bool ALIBI>
struct MfmaDecoderB {
  static constexpr int KS = D / 32;
  static constexpr int DB = D / 16;
  int lane, col, grp;
  float qk_scale, alibi;
  int pos_q;
  uint32_t qf[KS][4];
  float m_run, m_true, l_part;
  f32x4_t oacc[DB];

  __device__ __forceinline__ void init(int lane_) {
    lane = lane_;
    col = lane % 16;
    grp = lane / 16;
    alibi = 0.f;
    pos_q = 0;
  }

  __device__ __forceinline__ void load_q(const uint16_t* q, int64_t row_q, int num_q_heads,
                                         int h0, int nh, const float* slopes, int seq_len,
                                         float scale_log2) {
    const bool real = col < nh;
    const uint16_t* qh = q + (row_q * num_q_heads + h0 + (real ? col : 0)) * D + (D / 4) * grp;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 v = *reinterpret_cast<const uint4*>(qh + 8 * s);
      qf[s][0] = real ? v.x : 0u;
      qf[s][1] = real ? v.y : 0u;
      qf[s][2] = real ? v.z : 0u;
      qf[s][3] = real ? v.w : 0u;
    }
    qk_scale = scale_log2;
    pos_q = seq_len - 1;
    if constexpr (ALIBI) alibi = real ? slopes[h0 + col] * kLog2e : 0.f;
  }

  __device__ __forceinline__ void reset() {
    m_run = -INFINITY;
    m_true = -INFINITY;
    l_part = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) oacc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  __device__ __forceinline__ void compute(const MTileB<D>& t, int tok0, int t_end) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const uint4 qb = make_uint4(qf[st][0], qf[st][1], qf[st][2], qf[st][3]);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, t.k[st]),
                                                  __builtin_bit_cast(bf16x8_t, qb), s, 0, 0, 0);
    }
    const bool full = tok0 + kBlock <= t_end;
    float x[4];
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tok0 + 4 * grp + i;
      float xv = s[i] * qk_scale;
      if constexpr (ALIBI) xv = fmaf(alibi, (float)(tok - pos_q), xv);
      x[i] = (full || tok < t_end) ? xv : -INFINITY;
      bm = fmaxf(bm, x[i]);
    }
    bm = max_xor16(bm);
    bm = max_xor32(bm);
    m_true = fmaxf(m_true, bm);
    const bool grow = bm > m_run + kMTau;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? bm : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) oacc[b] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(x[i] - m_run);
      l_part += p[i];
    }
    // P^T = high + remainder, both bf16
    const uint32_t h01 = pack_bf16x2(p[0], p[1]), h23 = pack_bf16x2(p[2], p[3]);
    const uint32_t l01 = pack_bf16x2(p[0] - bf16lo(h01), p[1] - bf16hi(h01));
    const uint32_t l23 = pack_bf16x2(p[2] - bf16lo(h23), p[3] - bf16hi(h23));
    const uint2 ph = make_uint2(h01, h23), pl = make_uint2(l01, l23);
    uint32_t w[4][D / 32];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int c = 0; c < D / 32; ++c) w[e][c] = t.v[e][c];
    if (!full) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool live = tok0 + 4 * grp + e < t_end;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) w[e][c] = live ? w[e][c] : 0u;
      }
    }
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      // element b of the four rows: 16-bit half b%2 of word b/2
      const uint32_t sel = (b & 1) ? 0x07060302u : 0x05040100u;
      const uint2 vt = make_uint2(perm_bytes(w[1][b / 2], w[0][b / 2], sel),
                                  perm_bytes(w[3][b / 2], w[2][b / 2], sel));
      oacc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, vt),
                                                          __builtin_bit_cast(bf16x4_t, ph),
                                                          oacc[b], 0, 0, 0);
      oacc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, vt),
                                                          __builtin_bit_cast(bf16x4_t, pl),
                                                          oacc[b], 0, 0, 0);
    }
  }

  __device__ __forceinline__ void finish() {
    l_part = sum_xor16(l_part);
    l_part = sum_xor32(l_part);
  }
};

// Path selection for the kernel: tile type, loader, decoder, cache scales.
template <int D, bool ALIBI, bool FP8>
struct MPath;
template <int D, bool ALIBI>
struct MPath<D, ALIBI, true> {
  using Tile = MTile<D>;
  using Dec = MfmaDecoder<D, ALIBI>;
  static constexpr int kPrefetch = kMPrefetch;
  static __device__ __forceinline__ void load(Tile& t, const uint8_t* kb, const uint8_t* vb,
                                              int32_t phys, int g, int hkv, int lane) {
    mload<D>(t, kb, vb, phys, g, hkv, lane);
  }
};
template <int D, bool ALIBI>
struct MPath<D, ALIBI, false> {
  using Tile = MTileB<D>;
  using Dec = MfmaDecoderB<D, ALIBI>;
  static constexpr int kPrefetch = kMPrefetchB;
  static __device__ __forceinline__ void load(Tile& t, const uint8_t* kb, const uint8_t* vb,
                                              int32_t phys, int g, int hkv, int lane) {
    mloadB<D>(t, kb, vb, phys, g, hkv, lane);
  }
};

// One work-group per (request, KV head, 16-head chunk[, partition]); wave w
// takes every kMWaves-th block of the range.
template <int D, bool PART, bool ALIBI, bool FP8>
__global__ __launch_bounds__(kMWaves * 64, FP8 ? (ALIBI ? 3 : PA_MFMA_MINW_FP8) : PA_MFMA_MINW_BF16) void decode_mfma_kernel(
    DecodeArgs a, int n_chunks) {
  using Path = MPath<D, ALIBI, FP8>;
  using Dec = typename Path::Dec;
  __shared__ MfmaDecodeSmem<D> sm;
  // With a.lpt, blockIdx.z is a rank: the request with the rank-th longest
  // context (ties by index), so the longest units are handed out first.
  int r = blockIdx.z;
  if constexpr (!PART) {
    if (a.lpt) {
      const int R = a.num_reqs;
      // (in a varlen batch only rows with q_len 1 are decode rows: the
      // others rank last, and their work-groups exit)
      for (int i = threadIdx.x; i < R; i += kMWaves * kWave)
        sm.bt[i] = (a.query_start_loc == nullptr ||
                    a.query_start_loc[i + 1] - a.query_start_loc[i] == 1) ? a.seq_lens[i] : -1;
      __syncthreads();
      for (int j = threadIdx.x; j < R; j += kMWaves * kWave) {
        const int lj = sm.bt[j];
        int rank = 0;
        for (int k = 0; k < R; ++k) {
          const int lk = sm.bt[k];
          rank += (lk > lj || (lk == lj && k < j)) ? 1 : 0;
        }
        if (rank == (int)blockIdx.z) sm.sched = j;
      }
      __syncthreads();
      r = __builtin_amdgcn_readfirstlane(sm.sched);
      __syncthreads();
    }
  }
  const int g = blockIdx.y / n_chunks;
  const int hc = blockIdx.y - g * n_chunks;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int h0 = g * G + hc * kMHeads;
  const int nh = min(kMHeads, G - hc * kMHeads);

  int row_q = r;
  if (a.query_start_loc != nullptr) {
    const int lo = a.query_start_loc[r];
    if (a.query_start_loc[r + 1] - lo != 1) return;   // not a decode row
    row_q = lo;
  }
  const int seq_len = a.seq_lens[r];
  const int part = a.part_begin + (int)blockIdx.x;
  int t_begin = 0, t_end = seq_len;
  if constexpr (PART) {
    t_begin = part * a.partition_size;
    if (t_begin >= seq_len) return;
    t_end = (a.open_last && part == a.part_end - 1) ? seq_len
                                                    : min(seq_len, t_begin + a.partition_size);
  }
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;

  if (t_end <= t_begin) {                           // empty context: zero row
    if constexpr (!PART) {
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
      for (int i = tid; i < nh * D; i += kMWaves * kWave)
        out[((int64_t)row_q * a.num_q_heads + h0 + i / D) * D + (i % D)] = 0;
    }
    return;
  }

  Dec dec;
  dec.init(lane);
  dec.load_q(reinterpret_cast<const uint16_t*>(a.q), row_q, a.num_q_heads, h0, nh,
             a.alibi_slopes, seq_len, a.scale * kLog2e * (FP8 ? *a.k_scale : 1.f));
  dec.reset();

  const int first_block = t_begin / kBlock;
  const int last_block = (t_end - 1) / kBlock;
  const int32_t* bt_row = a.block_table + (int64_t)r * a.bt_stride;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);

  for (int cb = first_block; cb <= last_block; cb += kMBtChunk) {
    const int nb = min(last_block + 1 - cb, kMBtChunk);
    __syncthreads();
    for (int i = tid; i < nb; i += kMWaves * kWave) sm.bt[i] = bt_row[cb + i];
    __syncthreads();
    const int n = nb > w ? (nb - w + kMWaves - 1) / kMWaves : 0;
    if (n > 0) {
      // PF tiles in flight while one is computed (a ring of
      // registers, indices fixed by unrolling); the index of a prefetch is
      // clamped so every load is unconditional
      auto phys = [&](int it) {
        return __builtin_amdgcn_readfirstlane(sm.bt[w + min(it, n - 1) * kMWaves]);
      };
      constexpr int PF = Path::kPrefetch;
      constexpr int NR = PF + 1;
      typename Path::Tile ring[NR];
#pragma unroll
      for (int j = 0; j < PF; ++j)
        Path::load(ring[j], kbase, vbase, phys(j), g, a.num_kv_heads, lane);
      for (int it = 0; it < n; it += NR) {
#pragma unroll
        for (int j = 0; j < NR; ++j) {
          if (it + j >= n) break;
          Path::load(ring[(j + PF) % NR], kbase, vbase, phys(it + j + PF), g,
                     a.num_kv_heads, lane);
          dec.compute(ring[j], (cb + w + (it + j) * kMWaves) * kBlock, t_end);
        }
      }
    }
  }
  dec.finish();
  if (lane < kMHeads) {
    sm.m[w][lane] = dec.m_run;
    sm.mt[w][lane] = dec.m_true;
    sm.l[w][lane] = dec.l_part;
  }
#pragma unroll
  for (int b = 0; b < Dec::DB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sm.acc[w][dec.col][(D / 4) * dec.grp + (D / 16) * i + b] = dec.oacc[b][i];
  __syncthreads();

  // ---- combine the waves and write (as decode_kernel)
  const float vs = FP8 ? *a.v_scale : 1.f;
  for (int i = tid; i < kMHeads * D; i += kMWaves * kWave) {
    const int j = i / D, dd = i - j * D;
    if (j >= nh) continue;
    float M = -INFINITY, Mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < kMWaves; ++u) {
      M = fmaxf(M, sm.m[u][j]);
      Mt = fmaxf(Mt, sm.mt[u][j]);
    }
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int u = 0; u < kMWaves; ++u) {
      const float wgt = (sm.m[u][j] == -INFINITY) ? 0.f : fast_exp2(sm.m[u][j] - M);
      L += sm.l[u][j] * wgt;
      O += sm.acc[u][j][dd] * wgt;
    }
    O = O / L * vs;
    const int h = h0 + j;
    if constexpr (PART) {
      const int64_t idx = ((int64_t)r * a.num_q_heads + h) * a.max_num_partitions + part;
      a.tmp_out[idx * D + dd] = O;
      if (dd == 0) {
        a.max_logits[idx] = Mt * kLn2;
        a.exp_sums[idx] = L * fast_exp2(M - Mt);
      }
    } else {
      reinterpret_cast<uint16_t*>(a.out)[((int64_t)row_q * a.num_q_heads + h) * D + dd] =
          f32_to_bf16(O);
    }
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, bool partitioned, hipStream_t st) {
  if (a.num_reqs == 0) return hipSuccess;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int n_chunks = (G + kMHeads - 1) / kMHeads;
  dim3 grid(1, a.num_kv_heads * n_chunks, a.num_reqs);
  if (partitioned) {
    int nparts = (a.max_seq_len + a.partition_size - 1) / a.partition_size;
    if (a.part_end > 0) nparts = min(nparts, a.part_end) - a.part_begin;
    if (nparts <= 0) return hipSuccess;
    grid.x = nparts;
  }
  const bool fp8 = a.cache_dtype != 0;
  DecodeArgs b = a;
  // (rank search: O(num_reqs) per thread, so modest batches only; the
  // rank buffer is the block-table staging array)
  static_assert(kMaxLptReqs <= kMBtChunk, "rank buffer");
  b.lpt = (!partitioned && a.num_reqs <= kMaxLptReqs) ? 1 : 0;
#define PA_MFMA(DV, PT, AL) \
  do {                                                                                        \
    if (fp8)                                                                                  \
      hipLaunchKernelGGL((decode_mfma_kernel<DV, PT, AL, true>), grid, dim3(kMWaves * 64), 0, \
                         st, b, n_chunks);                                                    \
    else                                                                                      \
      hipLaunchKernelGGL((decode_mfma_kernel<DV, PT, AL, false>), grid, dim3(kMWaves * 64), 0, \
                         st, b, n_chunks);                                                    \
  } while (0)
#define PA_MFMA_AL(DV, PT) \
  do { if (a.alibi_slopes) PA_MFMA(DV, PT, true); else PA_MFMA(DV, PT, false); } while (0)
  if (a.head_dim == 64) {
    if (partitioned) PA_MFMA_AL(64, true); else PA_MFMA_AL(64, false);
  } else {
    if (partitioned) PA_MFMA_AL(128, true); else PA_MFMA_AL(128, false);
  }
#undef PA_MFMA_AL
#undef PA_MFMA
  return hipGetLastError();
}

}  // namespace pa
