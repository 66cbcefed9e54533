// The wave-level decode machinery shared by the decode kernels and the
// fused varlen kernel: tile loads, the per-wave online-softmax state, the
// block streaming loop and the per-unit work of a work-group.
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
// Work decomposition (differs from the pages' CUDA kernel, which runs one
// CTA per query head and re-reads K/V for every head of a group):
//   one work-group per (request, KV head, head chunk[, partition]); each of
//   its waves walks every WAVES-th 16-token block of the range, so each K/V
//   byte is read once for the whole GQA group.
//
// Lane layout for one (block, KV head) tile of 16 rows x D elements:
//   K: LPR lanes per row (4 or 8), each holding KE = D/LPR elements in
//      16-byte chunks c, c+LPR, ... so one load instruction covers whole
//      64/128-byte row segments; dot products use v_dot2_f32_bf16 and an
//      LPR-lane DPP butterfly.  Lane c of a row owns query head c of the
//      chunk for the softmax (exp, running max, exp-sum).
//   V: 16 lanes per row, rows rg, rg+4, rg+8, rg+12 (rg = lane/16), each lane
//      holding D/16 contiguous elements; accumulators acc[head][D/16].
//   p moves from K lanes to V lanes through a per-wave LDS slab.  FP8 caches
//   take a cheaper PV: each K lane stores its two rows' p (rows r, r + 8) as
//   one f16 pair, V lanes interleave the codes of rows r and r + 8, convert
//   them to exact f16 pairs and accumulate with v_dot2_f32_f16 (two tokens
//   per instruction), halving the vector-ALU work of PV.
//
// Online softmax in log2 units (scores pre-multiplied by log2 e) with a lazy
// running max: the max of head h only moves when a score exceeds it by more
// than kTau, so after the first blocks the rescale branch is rarely taken;
// every p = 2^(x - m) stays <= 2^kTau and the final A / l is unchanged.
#pragma once

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr float kTau = 8.0f;

// Waves per work-group for the single-pass and split-KV launches (measured on
// MI355X: the single pass gains from spreading a long context over more
// waves, split-KV partitions from more work-groups), and the prefetch depth
// (tiles in flight while one is computed; 2 measured no better than 1).
#ifndef PA_DECODE_WAVES_SINGLE
#define PA_DECODE_WAVES_SINGLE 8
#endif
// ... and only for contexts long enough to give the extra waves blocks:
// max_seq_len >= this, twice this from 384 work-groups on (measured on
// MI355X: at 512 groups and 256..1024-token contexts 4 waves are up to 30%
// faster; with few groups 8 waves win from 1024 tokens).
#ifndef PA_DECODE_WAVES_SINGLE_MIN_LEN
#define PA_DECODE_WAVES_SINGLE_MIN_LEN 1024
#endif
#ifndef PA_DECODE_WAVES_SPLIT
#define PA_DECODE_WAVES_SPLIT 4
#endif
#ifndef PA_DECODE_PREFETCH
#define PA_DECODE_PREFETCH 1
#endif
// Minimum waves per SIMD the 8-wave single-pass decode kernel is compiled for
// (caps its VGPRs): bf16 kernels with up to 4 heads per chunk fit 3 waves per
// SIMD (168 VGPRs) without spilling (measured 1% faster on the batched
// workload); the 4-wave and split-KV variants measured slower with the cap.
#ifndef PA_DECODE_MIN_WAVES_EU
#define PA_DECODE_MIN_WAVES_EU 3
#endif
// Longest-first order of the single pass's work-groups (0 disables), used for
// batches of up to kLptMaxReqs requests.
// Two-round single pass with exactly 8 (KV head, chunk) units: heavier
// work-group pairs on the even XCDs (see decode_kernel).
#ifndef PA_DECODE_XCD_WEIGHT
#define PA_DECODE_XCD_WEIGHT 1
#endif
#ifndef PA_DECODE_LPT
#define PA_DECODE_LPT 1
#endif
constexpr int kLptMaxReqs = 128;
// Streaming (non-temporal) K/V loads for bf16 caches (FP8 ones are the
// shared-prefix case, which lives on L2 hits).
#ifndef PA_DECODE_NT_BF16
#define PA_DECODE_NT_BF16 1
#endif
// FP8 decode on the matrix cores for G >= 4 (0: always the vector-ALU kernel).
#ifndef PA_DECODE_FP8_MFMA
#define PA_DECODE_FP8_MFMA 1
#endif
// bf16 caches on the matrix cores from this GQA group size up (0: never).
// Below it the vector-ALU kernel is as fast: its work per token grows with
// the group, the matrix-core kernel's does not up to 16 heads.
#ifndef PA_DECODE_BF16_MFMA_MIN_G
#define PA_DECODE_BF16_MFMA_MIN_G 8
#endif
template <int GC, bool FP8, bool PART, int WAVES>
constexpr int decode_min_waves() {
  return (!FP8 && !PART && GC <= 4 && WAVES == 8) ? PA_DECODE_MIN_WAVES_EU : 1;
}

template <int D, int GC, bool FP8>
struct DecodeShape {
  static constexpr int EB = FP8 ? 1 : 2;                    // bytes per element
  static constexpr int LPR = 8;                             // K lanes per row
  static constexpr int RK = LPR / 4;                        // K rows per lane
  static constexpr int KE = D / LPR;                        // K elements per lane-row
  static constexpr int KBYTES = KE * EB;                    // K bytes per lane-row
  static constexpr int KCHB = KBYTES < 16 ? KBYTES : 16;    // bytes per K load
  static constexpr int KCH = KBYTES / KCHB;                 // K loads per lane-row
  static constexpr int KW = KCHB / 4;                       // words per K load
  static constexpr int QW = KE / 2;                         // q words (bf16 pairs) per head
  static constexpr int VE = D / 16;                         // V elements per lane-row
  static constexpr int VW = VE * EB / 4;                    // words per V load
  static constexpr int GCP = GC <= 4 ? 4 : 8;               // p slab row stride
  static_assert(LPR >= GC, "one softmax head per K lane");
  static_assert(KBYTES % KCHB == 0 && KCHB % 4 == 0, "K chunking");
  static_assert(VW >= 1 && VW <= 4, "V load width");
};

template <int N>
struct Words {
  uint32_t w[N];
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// NT: non-temporal (streaming) loads, for data that is read once
template <int N, bool NT = false>
__device__ __forceinline__ Words<N> load_words(const uint8_t* p) {
  Words<N> r;
  if constexpr (NT && N == 4) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (NT && N == 2) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    r.w[0] = v.x; r.w[1] = v.y;
  } else if constexpr (NT) {
    r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  } else if constexpr (N == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (N == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
  return r;
}

// Word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format
// (required by the untyped buffer loads), no swizzle, no index stride.
constexpr int kRsrcWord3 = 0x00020000;

// N words at byte offset `off` of a buffer resource (out-of-range lanes read 0)
template <int N, int AUX>
__device__ __forceinline__ Words<N> rsrc_words(__amdgpu_buffer_rsrc_t r, int off) {
  Words<N> w;
  if constexpr (N == 4) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    w.w[0] = v.x; w.w[1] = v.y; w.w[2] = v.z; w.w[3] = v.w;
  } else if constexpr (N == 2) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
    w.w[0] = v.x; w.w[1] = v.y;
  } else {
    w.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
  }
  return w;
}

constexpr int kBtChunk = 1024;   // block-table entries staged in LDS at a time

// ---------------------------------------------------------------------------
// One wave's decode state over a run of 16-token blocks of one (request, KV
// head, head chunk) unit: q in registers, the online-softmax state and the
// PV accumulators.  The kernels below differ only in how they hand out
// blocks to waves and what they do with the finished state.
template <int D, int GC, bool FP8>
struct WaveDecoder {
  using S = DecodeShape<D, GC, FP8>;
  static constexpr int EB = S::EB, LPR = S::LPR, RK = S::RK, KCH = S::KCH, KW = S::KW,
                       KCHB = S::KCHB, QW = S::QW, VE = S::VE, VW = S::VW, GCP = S::GCP;
  static constexpr bool kStream = PA_DECODE_NT_BF16 && !FP8;
  struct Tile {
    Words<KW> k[RK][KCH];
    Words<VW> v[4];
  };

  int lane, kc, krow0, vrg, vcol;
  int nh;                        // real heads of the current unit's chunk
  float qk_scale;
  bool has_alibi;                // uniform: ALiBi slopes given
  float alibi;                   // slope of head kc, log2 units (0 without ALiBi)
  int pos_q;                     // position of the query (seq_len - 1)
  uint32_t qreg[GC][QW];
  float m_run, m_true, l_part;   // lazy max (log2 units), exact max, exp-sum: head kc
  float acc[GC][VE];

  __device__ __forceinline__ void init(int lane_, float qk_scale_, bool has_alibi_) {
    lane = lane_;
    kc = lane % LPR;             // K lane within its row
    krow0 = lane / LPR;          // first K row; rows krow0 + (64/LPR)*i
    vrg = lane / 16;             // V row group; rows vrg + 4*i
    vcol = (lane % 16) * VE;     // first V element of this lane
    qk_scale = qk_scale_;
    has_alibi = has_alibi_;
    alibi = 0.f;
    pos_q = 0;
  }

  // ALiBi slope of this lane's head (call after load_q) and the query position
  __device__ __forceinline__ void set_query(const float* slopes, int h0, int seq_len) {
    pos_q = seq_len - 1;
    if (has_alibi) alibi = kc < nh ? slopes[h0 + kc] * kLog2e : 0.f;
  }

  // q of query row `row_q`, heads h0 .. h0+nh-1, at this lane's K positions
  __device__ __forceinline__ void load_q(const uint16_t* q, int64_t row_q, int num_q_heads,
                                         int h0, int nh_) {
    nh = nh_;
    constexpr int CE = KCHB / EB;            // elements per K chunk
#pragma unroll
    for (int j = 0; j < GC; ++j) {
      const bool real = j < nh;
      const uint16_t* qh = q + (row_q * num_q_heads + h0 + (real ? j : 0)) * D;
#pragma unroll
      for (int k = 0; k < KCH; ++k) {
        const int e0 = (kc + LPR * k) * CE;
#pragma unroll
        for (int u = 0; u < CE / 2; ++u) {
          const uint32_t v = *reinterpret_cast<const uint32_t*>(qh + e0 + 2 * u);
          qreg[j][k * (CE / 2) + u] = real ? v : 0u;
        }
      }
    }
  }

  __device__ __forceinline__ void reset() {
    m_run = -INFINITY;
    m_true = -INFINITY;
    l_part = 0.f;
#pragma unroll
    for (int j = 0; j < GC; ++j)
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[j][e] = 0.f;
  }

  __device__ __forceinline__ void load_tile(Tile& t, const uint8_t* kbase, const uint8_t* vbase,
                                            int32_t phys, int g, int num_kv_heads) const {
    const int64_t off = tile_offset(phys, g, num_kv_heads, D) * EB;
    const uint8_t* kt = kbase + off;
    const uint8_t* vt = vbase + off;
#pragma unroll
    for (int i = 0; i < RK; ++i)
#pragma unroll
      for (int k = 0; k < KCH; ++k)
        t.k[i][k] = load_words<KW, kStream>(kt + (krow0 + (64 / LPR) * i) * (D * EB) +
                                            (kc + LPR * k) * KCHB);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      t.v[i] = load_words<VW, kStream>(vt + ((vrg + 4 * i) * D + vcol) * EB);
  }

  // The same tile through buffer resources spanning just this tile: with
  // live == false the resources have zero length, so every lane's load
  // returns 0 without touching memory (a prefetch past the wave's last
  // block costs no traffic, and the load stays unconditional, which keeps
  // the compiler's wait counts exact).
  __device__ __forceinline__ void load_tile_rsrc(Tile& t, const uint8_t* kbase,
                                                 const uint8_t* vbase, int32_t phys, int g,
                                                 int num_kv_heads, bool live) const {
    constexpr int kTileBytes = kBlock * D * EB;
    constexpr int kAux = kStream ? 2 : 0;           // cache policy: nt (streaming)
    // the tile address and length are wave-uniform by construction; made
    // scalar here so the resources live in SGPRs whatever the caller's
    // control flow lets the compiler prove
    const int64_t off0 = tile_offset(phys, g, num_kv_heads, D) * EB;
    const int64_t off =
        (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(off0 >> 32)) << 32) |
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)off0));
    const int nrec = __builtin_amdgcn_readfirstlane(live ? kTileBytes : 0);
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + off), (short)0, nrec, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + off), (short)0, nrec, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < RK; ++i)
#pragma unroll
      for (int k = 0; k < KCH; ++k)
        t.k[i][k] = rsrc_words<KW, kAux>(kr, (krow0 + (64 / LPR) * i) * (D * EB) +
                                                 (kc + LPR * k) * KCHB);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      t.v[i] = rsrc_words<VW, kAux>(vr, ((vrg + 4 * i) * D + vcol) * EB);
  }

  // Fold one block (tokens tok0 .. tok0+15, those >= t_end excluded) into
  // the state.  `slab` is this wave's [16][GCP] float LDS buffer.
  __device__ __forceinline__ void compute(const Tile& t, int tok0, int t_end, float* slab) {
    // -- scores of the chunk's heads for this lane's K rows
    float s[RK][GC];
#pragma unroll
    for (int i = 0; i < RK; ++i) {
#pragma unroll
      for (int j = 0; j < GC; ++j) s[i][j] = 0.f;
#pragma unroll
      for (int k = 0; k < KCH; ++k) {
#pragma unroll
        for (int u = 0; u < KW; ++u) {
          if constexpr (FP8) {
            const f32x4_t f = fp8x4_to_f32(t.k[i][k].w[u]);
            const uint32_t p01 = pack_bf16x2(f.x, f.y);
            const uint32_t p23 = pack_bf16x2(f.z, f.w);
            const int qi = (k * KW + u) * 2;
#pragma unroll
            for (int j = 0; j < GC; ++j) {
              s[i][j] = dot2_bf16(qreg[j][qi], p01, s[i][j]);
              s[i][j] = dot2_bf16(qreg[j][qi + 1], p23, s[i][j]);
            }
          } else {
            const int qi = k * KW + u;
#pragma unroll
            for (int j = 0; j < GC; ++j) s[i][j] = dot2_bf16(qreg[j][qi], t.k[i][k].w[u], s[i][j]);
          }
        }
      }
      // sum over the LPR lanes of the row
#pragma unroll
      for (int j = 0; j < GC; ++j) {
        float x = s[i][j];
        x += dpp<kQuadXor1>(x);
        x += dpp<kQuadXor2>(x);
        if constexpr (LPR == 8) x += dpp<0x141>(x);   // row_half_mirror: other quad
        s[i][j] = x;
      }
    }
    // -- this lane's head (kc): scaled scores, masked by select
    float x[RK];
    bool any_big = false;
#pragma unroll
    for (int i = 0; i < RK; ++i) {
      float sv = s[i][0];
#pragma unroll
      for (int j = 1; j < GC; ++j) sv = (kc == j) ? s[i][j] : sv;
      const int tok = tok0 + krow0 + (64 / LPR) * i;
      const bool valid = (kc < nh) && (tok < t_end);
      float xv = sv * qk_scale;
      if (has_alibi) xv = fmaf(alibi, (float)(tok - pos_q), xv);
      x[i] = valid ? xv : -INFINITY;
      m_true = fmaxf(m_true, x[i]);
      any_big |= x[i] > m_run + kTau;
    }
    if (__builtin_amdgcn_ballot_w64(any_big) != 0) {      // wave-uniform branch
      float bm = x[0];
#pragma unroll
      for (int i = 1; i < RK; ++i) bm = fmaxf(bm, x[i]);
      // max over all rows of head kc: lanes with equal kc
      if constexpr (LPR == 4) bm = fmaxf(bm, dpp<kRowRor4>(bm));
      bm = fmaxf(bm, dpp<kRowRor8>(bm));
      bm = max_xor16(bm);
      bm = max_xor32(bm);
      const float m_new = fmaxf(m_run, bm);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int j = 0; j < GC; ++j) {
        const float aj = __builtin_bit_cast(float,
            __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), j));
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[j][e] *= aj;
      }
    }
    // -- probabilities to the LDS slab: fp32 [16 rows][GCP] for bf16 caches;
    // for FP8 caches one f16 pair per (row pair, head): rows krow0 and
    // krow0 + 8 (this lane's two K rows) share a word, [8 pairs][GCP].
    if constexpr (FP8) {
      static_assert(RK == 2 && 64 / LPR == 8, "row pairs (r, r + 8)");
      float pr[RK];
#pragma unroll
      for (int i = 0; i < RK; ++i) {
        pr[i] = (x[i] == -INFINITY) ? 0.f : fast_exp2(x[i] - m_run);
        l_part += pr[i];
      }
      if (kc < GC) reinterpret_cast<uint32_t*>(slab)[krow0 * GCP + kc] = pack_f16x2(pr[0], pr[1]);
    } else {
#pragma unroll
      for (int i = 0; i < RK; ++i) {
        const float p = (x[i] == -INFINITY) ? 0.f : fast_exp2(x[i] - m_run);
        l_part += p;
        if (kc < GC) slab[(krow0 + (64 / LPR) * i) * GCP + kc] = p;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // -- PV: this lane's 4 V rows
    const bool full = tok0 + kBlock <= t_end;
    if constexpr (FP8) {
      // Rows (vrg + 4ip, vrg + 4ip + 8) in pairs: their codes are interleaved
      // byte-wise, converted to f16 pairs (exact) and multiplied with the f16
      // p pairs by v_dot2_f32_f16, two tokens per instruction.
#pragma unroll
      for (int ip = 0; ip < 2; ++ip) {
        const int ra = vrg + 4 * ip;
        uint32_t pp[GCP];
#pragma unroll
        for (int q4 = 0; q4 < GCP / 4; ++q4) {
          const uint4 p4 = *reinterpret_cast<const uint4*>(
              &reinterpret_cast<const uint32_t*>(slab)[ra * GCP + q4 * 4]);
          pp[q4 * 4 + 0] = p4.x; pp[q4 * 4 + 1] = p4.y;
          pp[q4 * 4 + 2] = p4.z; pp[q4 * 4 + 3] = p4.w;
        }
        Words<VW> wa = t.v[ip], wb = t.v[ip + 2];
        if (!full) {
          if (tok0 + ra >= t_end) {
#pragma unroll
            for (int u = 0; u < VW; ++u) wa.w[u] = 0u;     // past the context: exclude
          }
          if (tok0 + ra + 8 >= t_end) {
#pragma unroll
            for (int u = 0; u < VW; ++u) wb.w[u] = 0u;
          }
        }
        uint32_t hv[VE];                 // f16 pairs (v[ra][e], v[ra + 8][e])
#pragma unroll
        for (int u = 0; u < VW; ++u) {
          const uint32_t x01 = perm_bytes(wb.w[u], wa.w[u], 0x05010400u);   // a0 b0 a1 b1
          const uint32_t x23 = perm_bytes(wb.w[u], wa.w[u], 0x07030602u);   // a2 b2 a3 b3
          hv[4 * u + 0] = fp8x2_to_f16x2<false>(x01);
          hv[4 * u + 1] = fp8x2_to_f16x2<true>(x01);
          hv[4 * u + 2] = fp8x2_to_f16x2<false>(x23);
          hv[4 * u + 3] = fp8x2_to_f16x2<true>(x23);
        }
#pragma unroll
        for (int j = 0; j < GC; ++j)
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[j][e] = dot2_f16(pp[j], hv[e], acc[j][e]);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vr = vrg + 4 * i;
      float pv[GCP];
#pragma unroll
      for (int q4 = 0; q4 < GCP / 4; ++q4) {
        const f32x4_t p4 = *reinterpret_cast<const f32x4_t*>(&slab[vr * GCP + q4 * 4]);
        pv[q4 * 4 + 0] = p4.x; pv[q4 * 4 + 1] = p4.y;
        pv[q4 * 4 + 2] = p4.z; pv[q4 * 4 + 3] = p4.w;
      }
      Words<VW> vw = t.v[i];
      if (!full && tok0 + vr >= t_end) {
#pragma unroll
        for (int u = 0; u < VW; ++u) vw.w[u] = 0u;     // past the context: exclude
      }
      float vf[VE];
      if constexpr (FP8) {
#pragma unroll
        for (int u = 0; u < VW; ++u) {
          const f32x4_t f = fp8x4_to_f32(vw.w[u]);
          vf[4 * u + 0] = f.x; vf[4 * u + 1] = f.y; vf[4 * u + 2] = f.z; vf[4 * u + 3] = f.w;
        }
      } else {
#pragma unroll
        for (int u = 0; u < VW; ++u) {
          vf[2 * u] = bf16lo(vw.w[u]);
          vf[2 * u + 1] = bf16hi(vw.w[u]);
        }
      }
#pragma unroll
      for (int j = 0; j < GC; ++j)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[j][e] = fmaf(pv[j], vf[e], acc[j][e]);
    }
  }

  // Reduce the lane partials: afterwards lane j < GC holds head j's m_run,
  // m_true and l_part, and lanes 0..15 hold acc[j][vcol + e] summed over rows.
  __device__ __forceinline__ void finish() {
    float l = l_part, mt = m_true;
    if constexpr (LPR == 4) {
      l += dpp<kRowRor4>(l);
      mt = fmaxf(mt, dpp<kRowRor4>(mt));
    }
    l += dpp<kRowRor8>(l);
    mt = fmaxf(mt, dpp<kRowRor8>(mt));
    l = sum_xor16(l);
    mt = max_xor16(mt);
    l = sum_xor32(l);
    mt = max_xor32(mt);
    l_part = l;
    m_true = mt;
#pragma unroll
    for (int j = 0; j < GC; ++j)
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        float v = acc[j][e];
        v = sum_xor16(v);
        v = sum_xor32(v);
        acc[j][e] = v;
      }
  }
};

// Stream n blocks through the decoder with PD tiles in flight.  phys_of(it)
// must accept it >= n (clamped by the caller): the prefetch is issued
// unconditionally, so the compiler's wait counts stay exact, and a prefetch
// past the last block is a zero-length buffer load that moves no data.
template <int PD, class Dec, class PhysFn, class TokFn>
__device__ __forceinline__ void stream_blocks(Dec& dec, int n, const uint8_t* kbase,
                                              const uint8_t* vbase, int g, int num_kv_heads,
                                              int t_end, float* slab0, float* slab1,
                                              PhysFn phys_of, TokFn tok0_of) {
  using Tile = typename Dec::Tile;
  if constexpr (PD == 1) {
    Tile ta, tb;
    dec.load_tile_rsrc(ta, kbase, vbase, phys_of(0), g, num_kv_heads, true);
    int32_t pn = phys_of(1);
    for (int it = 0; it < n; it += 2) {
      dec.load_tile_rsrc(tb, kbase, vbase, pn, g, num_kv_heads, it + 1 < n);
      pn = phys_of(it + 2);
      dec.compute(ta, tok0_of(it), t_end, slab0);
      if (it + 1 >= n) break;
      dec.load_tile_rsrc(ta, kbase, vbase, pn, g, num_kv_heads, it + 2 < n);
      pn = phys_of(it + 3);
      dec.compute(tb, tok0_of(it + 1), t_end, slab1);
    }
  } else {                                  // two tiles in flight while computing
    Tile t0, t1, t2;
    dec.load_tile_rsrc(t0, kbase, vbase, phys_of(0), g, num_kv_heads, true);
    dec.load_tile_rsrc(t1, kbase, vbase, phys_of(1), g, num_kv_heads, 1 < n);
    int32_t pn = phys_of(2);
    for (int it = 0; it < n; it += 3) {
      dec.load_tile_rsrc(t2, kbase, vbase, pn, g, num_kv_heads, it + 2 < n);
      pn = phys_of(it + 3);
      dec.compute(t0, tok0_of(it), t_end, (it & 1) ? slab1 : slab0);
      if (it + 1 >= n) break;
      dec.load_tile_rsrc(t0, kbase, vbase, pn, g, num_kv_heads, it + 3 < n);
      pn = phys_of(it + 4);
      dec.compute(t1, tok0_of(it + 1), t_end, (it & 1) ? slab0 : slab1);
      if (it + 2 >= n) break;
      dec.load_tile_rsrc(t1, kbase, vbase, pn, g, num_kv_heads, it + 4 < n);
      pn = phys_of(it + 5);
      dec.compute(t2, tok0_of(it + 2), t_end, (it & 1) ? slab1 : slab0);
    }
  }
}

template <int D, int GC, bool FP8, int WAVES>
struct DecodeSmem {
  using S = DecodeShape<D, GC, FP8>;
  int32_t bt[kBtChunk];           // block-table chunk (first: the requests' lengths)
  int32_t sched;
  float p[WAVES][2][kBlock][S::GCP];
  float m[WAVES][8];
  float mt[WAVES][8];
  float l[WAVES][8];
  float acc[WAVES][GC][D];
};

// The work of one (request r, KV head x head chunk `unit`[, partition
// part_idx]) unit, by the work-group's WAVES waves: walk its blocks, combine
// the waves' states in LDS, write the bf16 output row (or the partials).
// Rows of varlen batches come from query_start_loc when given (rows whose
// q_len is not 1 are left alone).
template <int D, int GC, bool FP8, int WAVES, bool PART, int PD>
__device__ __forceinline__ void decode_unit(const DecodeArgs& a, DecodeSmem<D, GC, FP8, WAVES>& sm,
                                            int r, int unit, int part_idx, int n_chunks) {
  using Dec = WaveDecoder<D, GC, FP8>;
  const int g = unit / n_chunks;
  const int hc = unit - g * n_chunks;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int h0 = g * G + hc * GC;                 // first query head of the chunk
  const int nh = min(GC, G - hc * GC);            // real heads in the chunk

  // query / output row of this request
  int row_q = r;
  if (a.query_start_loc != nullptr) {
    const int lo = a.query_start_loc[r];
    if (a.query_start_loc[r + 1] - lo != 1) return;   // not a decode row
    row_q = lo;
  }
  const int seq_len = a.seq_lens[r];
  int t_begin = 0, t_end = seq_len;
  const int part = a.part_begin + part_idx;     // partition index (PART)
  if constexpr (PART) {
    t_begin = part * a.partition_size;
    if (t_begin >= seq_len) return;
    t_end = (a.open_last && part == a.part_end - 1) ? seq_len
                                                    : min(seq_len, t_begin + a.partition_size);
  }

  const int tid = threadIdx.x;
  // wave index, scalar: the compiler then knows every per-wave count and
  // loop bound below is wave-uniform (no exec-masked loop control)
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;

  if (t_end <= t_begin) {                         // empty context: zero row
    if constexpr (!PART) {
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
      for (int i = tid; i < nh * D; i += WAVES * kWave)
        out[((int64_t)row_q * a.num_q_heads + h0 + i / D) * D + (i % D)] = 0;
    }
    return;
  }

  if constexpr (!PART) {
    // append mode (one head chunk per KV head): this work-group writes its KV
    // head's row of the request's newest token (position seq_len - 1,
    // P3's slot formula) and is the only one to read that head's tiles of
    // the request, so a block-level release and barrier order the write
    // before the loads below
    if (a.new_k != nullptr) {
      const int pos = seq_len - 1;
      const int64_t slot =
          (int64_t)a.block_table[(int64_t)r * a.bt_stride + pos / kBlock] * kBlock + pos % kBlock;
      constexpr int CHK = D / 8;                  // 16-byte source chunks per row
      if (tid < 2 * CHK) {
        const bool is_v = tid >= CHK;
        const int c = tid - (is_v ? CHK : 0);
        const uint4 src = reinterpret_cast<const uint4*>(is_v ? a.new_v : a.new_k)
            [((int64_t)r * a.num_kv_heads + g) * CHK + c];
        const float qs = FP8 ? *(is_v ? a.v_scale : a.k_scale) : 1.f;
        store_chunk<FP8>(const_cast<void*>(is_v ? a.v_cache : a.k_cache),
                         slot_offset(slot, g, a.num_kv_heads, D) / 8 + c, src, qs);
      }
      if (g == 0 && tid == 0 && a.slot_out != nullptr) a.slot_out[r] = slot;
      __threadfence_block();
      __syncthreads();
    }
  }

  float qk_scale = a.scale * kLog2e;
  if constexpr (FP8) qk_scale *= *a.k_scale;
  Dec dec;
  dec.init(lane, qk_scale, a.alibi_slopes != nullptr);
  dec.load_q(reinterpret_cast<const uint16_t*>(a.q), row_q, a.num_q_heads, h0, nh);
  dec.set_query(a.alibi_slopes, h0, seq_len);
  dec.reset();

  const int first_block = t_begin / kBlock;
  const int last_block = (t_end - 1) / kBlock;
  const int32_t* bt_row = a.block_table + (int64_t)r * a.bt_stride;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);

  // Walk the range in chunks of kBtChunk blocks whose block-table entries are
  // staged in LDS; wave w takes every WAVES-th block of a chunk.
  for (int cb = first_block; cb <= last_block; cb += kBtChunk) {
    const int nb = min(last_block + 1 - cb, kBtChunk);
    __syncthreads();
    for (int i = tid; i < nb; i += WAVES * kWave) sm.bt[i] = bt_row[cb + i];
    __syncthreads();
    const int n = nb > w ? (nb - w + WAVES - 1) / WAVES : 0;   // this wave's blocks
    if (n > 0) {
      stream_blocks<PD>(
          dec, n, kbase, vbase, g, a.num_kv_heads, t_end, &sm.p[w][0][0][0], &sm.p[w][1][0][0],
          [&](int it) {
            return __builtin_amdgcn_readfirstlane(sm.bt[w + min(it, n - 1) * WAVES]);
          },
          [&](int it) { return (cb + w + it * WAVES) * kBlock; });
    }
  }

  dec.finish();
  if (lane < GC) {                    // lane j: row 0, kc == j
    sm.m[w][lane] = dec.m_run;
    sm.mt[w][lane] = dec.m_true;
    sm.l[w][lane] = dec.l_part;
  }
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < GC; ++j)
#pragma unroll
      for (int e = 0; e < Dec::VE; ++e) sm.acc[w][j][dec.vcol + e] = dec.acc[j][e];
  }
  __syncthreads();

  // ---- combine the waves and write
  const float vs = FP8 ? *a.v_scale : 1.f;
  for (int i = tid; i < GC * D; i += WAVES * kWave) {
    const int j = i / D, dd = i - j * D;
    if (j >= nh) continue;
    float M = -INFINITY, Mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < WAVES; ++u) {
      M = fmaxf(M, sm.m[u][j]);
      Mt = fmaxf(Mt, sm.mt[u][j]);
    }
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int u = 0; u < WAVES; ++u) {
      const float wgt = (sm.m[u][j] == -INFINITY) ? 0.f : fast_exp2(sm.m[u][j] - M);
      L += sm.l[u][j] * wgt;
      O += sm.acc[u][j][dd] * wgt;
    }
    O = O / L * vs;
    const int h = h0 + j;
    if constexpr (PART) {
      const int64_t idx = ((int64_t)r * a.num_q_heads + h) * a.max_num_partitions + part;
      a.tmp_out[idx * D + dd] = O;
      if (dd == 0) {       // re-based on the exact max: (m, l) as the pages define them
        a.max_logits[idx] = Mt * kLn2;
        a.exp_sums[idx] = L * fast_exp2(M - Mt);
      }
    } else {
      reinterpret_cast<uint16_t*>(a.out)[((int64_t)row_q * a.num_q_heads + h) * D + dd] =
          f32_to_bf16(O);
    }
  }
}

}  // namespace pa
