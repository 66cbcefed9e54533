// Single-query paged decode attention for gfx950.
//
// What is computed ("vLLM 深度解析（二）：PagedAttention 核心机制"):
//   §3.1   block_table[request][t // B] gives the physical block of token t;
//   §3.2.4 scores scale*<q, k> for the query heads sharing one KV head,
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
//   p moves from K lanes to V lanes through a per-wave LDS slab.
//
// Online softmax in log2 units (scores pre-multiplied by log2 e) with a lazy
// running max: the max of head h only moves when a score exceeds it by more
// than kTau, so after the first blocks the rescale branch is rarely taken;
// every p = 2^(x - m) stays <= 2^kTau and the final A / l is unchanged.
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
#ifndef PA_DECODE_WAVES_SPLIT
#define PA_DECODE_WAVES_SPLIT 4
#endif
#ifndef PA_DECODE_PREFETCH
#define PA_DECODE_PREFETCH 1
#endif

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

template <int N>
__device__ __forceinline__ Words<N> load_words(const uint8_t* p) {
  Words<N> r;
  if constexpr (N == 4) {
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

constexpr int kBtChunk = 1024;   // block-table entries staged in LDS at a time

template <int D, int GC, bool FP8, int WAVES>
struct DecodeSmem {
  using S = DecodeShape<D, GC, FP8>;
  int32_t bt[kBtChunk];
  float p[WAVES][2][kBlock][S::GCP];
  float m[WAVES][8];
  float mt[WAVES][8];
  float l[WAVES][8];
  float acc[WAVES][GC][D];
};

// PART: false -> write the final bf16 output; true -> write the partition
// partials.  QSL: q/out rows come from query_start_loc (varlen decode rows).
template <int D, int GC, bool FP8, int WAVES, bool PART, int PD>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(DecodeArgs a, int n_chunks) {
  using S = DecodeShape<D, GC, FP8>;
  constexpr int EB = S::EB, LPR = S::LPR, RK = S::RK, KCH = S::KCH, KW = S::KW,
                KCHB = S::KCHB, QW = S::QW, VE = S::VE, VW = S::VW;
  __shared__ DecodeSmem<D, GC, FP8, WAVES> sm;

  const int r = blockIdx.z;
  const int g = blockIdx.y / n_chunks;
  const int hc = blockIdx.y - g * n_chunks;
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
  if constexpr (PART) {
    t_begin = blockIdx.x * a.partition_size;
    if (t_begin >= seq_len) return;
    t_end = min(seq_len, t_begin + a.partition_size);
  }

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = tid % kWave;

  if (t_end <= t_begin) {                         // empty context: zero row
    if constexpr (!PART) {
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
      for (int i = tid; i < nh * D; i += WAVES * kWave)
        out[((int64_t)row_q * a.num_q_heads + h0 + i / D) * D + (i % D)] = 0;
    }
    return;
  }

  // ---- per-lane roles
  const int kc = lane % LPR;                      // K lane within its row
  const int krow0 = lane / LPR;                   // first K row; rows krow0 + (64/LPR)*i
  const int vrg = lane / 16;                      // V row group; rows vrg + 4*i
  const int vcol = (lane % 16) * VE;              // first V element of this lane

  // ---- q for the chunk's heads, in this lane's K element positions
  uint32_t qreg[GC][QW];
  {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
#pragma unroll
    for (int j = 0; j < GC; ++j) {
      const bool real = j < nh;
      const uint16_t* qh = q + ((int64_t)row_q * a.num_q_heads + h0 + (real ? j : 0)) * D;
#pragma unroll
      for (int k = 0; k < KCH; ++k) {
        // elements of chunk (kc + LPR*k): KCHB/EB of them
        constexpr int CE = KCHB / EB;
        const int e0 = (kc + LPR * k) * CE;
#pragma unroll
        for (int u = 0; u < CE / 2; ++u) {
          const uint32_t v = *reinterpret_cast<const uint32_t*>(qh + e0 + 2 * u);
          qreg[j][k * (CE / 2) + u] = real ? v : 0u;
        }
      }
    }
  }

  float qk_scale = a.scale * kLog2e;
  if constexpr (FP8) qk_scale *= *a.k_scale;

  // ---- block range of the work-group
  const int first_block = t_begin / kBlock;
  const int last_block = (t_end - 1) / kBlock;
  const int32_t* bt_row = a.block_table + (int64_t)r * a.bt_stride;

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);
  const int Hkv = a.num_kv_heads;

  float m_run = -INFINITY;       // lazy running max (log2 units) of head kc
  float m_true = -INFINITY;      // exact max of this lane's scores of head kc
  float l_part = 0.f;            // exp-sum of head kc over this lane's rows
  float acc[GC][VE];
#pragma unroll
  for (int j = 0; j < GC; ++j)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[j][e] = 0.f;

  struct Tile {
    Words<KW> k[RK][KCH];
    Words<VW> v[4];
  };

  auto load_tile = [&](Tile& t, int32_t phys) {
    const int64_t off = tile_offset(phys, g, Hkv, D) * EB;
    const uint8_t* kt = kbase + off;
    const uint8_t* vt = vbase + off;
#pragma unroll
    for (int i = 0; i < RK; ++i)
#pragma unroll
      for (int k = 0; k < KCH; ++k)
        t.k[i][k] = load_words<KW>(kt + (krow0 + (64 / LPR) * i) * (D * EB) +
                                   (kc + LPR * k) * KCHB);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      t.v[i] = load_words<VW>(vt + ((vrg + 4 * i) * D + vcol) * EB);
  };

  auto compute = [&](Tile& t, int tok0, int buf) {
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
      x[i] = valid ? sv * qk_scale : -INFINITY;
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
      bm = fmaxf(bm, xor_lanes(bm, 16));
      bm = fmaxf(bm, xor_lanes(bm, 32));
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
    // -- probabilities to the LDS slab
    float* slab = &sm.p[w][buf][0][0];
#pragma unroll
    for (int i = 0; i < RK; ++i) {
      const float p = (x[i] == -INFINITY) ? 0.f : fast_exp2(x[i] - m_run);
      l_part += p;
      if (kc < GC) slab[(krow0 + (64 / LPR) * i) * S::GCP + kc] = p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // -- PV: this lane's 4 V rows
    const bool full = tok0 + kBlock <= t_end;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vr = vrg + 4 * i;
      float pv[S::GCP];
#pragma unroll
      for (int q4 = 0; q4 < S::GCP / 4; ++q4) {
        const f32x4_t p4 = *reinterpret_cast<const f32x4_t*>(&slab[vr * S::GCP + q4 * 4]);
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
  };

  // Walk the range in chunks of kBtChunk blocks whose block-table entries are
  // staged in LDS.  Within a chunk each wave double-buffers its tiles; the
  // prefetch is unconditional (the index is clamped to the wave's last block,
  // a repeat read that hits in L2) so every iteration has the same loads in
  // flight and the compiler's wait counts stay exact.
  for (int cb = first_block; cb <= last_block; cb += kBtChunk) {
    const int nb = min(last_block + 1 - cb, kBtChunk);
    __syncthreads();
    for (int i = tid; i < nb; i += WAVES * kWave) sm.bt[i] = bt_row[cb + i];
    __syncthreads();
    const int n = nb > w ? (nb - w + WAVES - 1) / WAVES : 0;   // this wave's blocks
    if (n > 0) {
      auto phys_of = [&](int it) {
        return __builtin_amdgcn_readfirstlane(sm.bt[w + min(it, n - 1) * WAVES]);
      };
      auto tok0_of = [&](int it) { return (cb + w + it * WAVES) * kBlock; };
      if constexpr (PD == 1) {
        Tile ta, tb;
        load_tile(ta, phys_of(0));
        int32_t pn = phys_of(1);
        for (int it = 0; it < n; it += 2) {
          load_tile(tb, pn);
          pn = phys_of(it + 2);
          compute(ta, tok0_of(it), 0);
          if (it + 1 >= n) break;
          load_tile(ta, pn);
          pn = phys_of(it + 3);
          compute(tb, tok0_of(it + 1), 1);
        }
      } else {                                  // two tiles in flight while computing
        Tile t0, t1, t2;
        load_tile(t0, phys_of(0));
        load_tile(t1, phys_of(1));
        int32_t pn = phys_of(2);
        for (int it = 0; it < n; it += 3) {
          load_tile(t2, pn);
          pn = phys_of(it + 3);
          compute(t0, tok0_of(it), it & 1);
          if (it + 1 >= n) break;
          load_tile(t0, pn);
          pn = phys_of(it + 4);
          compute(t1, tok0_of(it + 1), (it + 1) & 1);
          if (it + 2 >= n) break;
          load_tile(t1, pn);
          pn = phys_of(it + 5);
          compute(t2, tok0_of(it + 2), it & 1);
        }
      }
    }
  }

  // ---- wave totals: l over the rows of head kc, acc over the 4 row groups
  {
    float l = l_part, mt = m_true;
    if constexpr (LPR == 4) {
      l += dpp<kRowRor4>(l);
      mt = fmaxf(mt, dpp<kRowRor4>(mt));
    }
    l += dpp<kRowRor8>(l);
    mt = fmaxf(mt, dpp<kRowRor8>(mt));
    l += xor_lanes(l, 16);
    mt = fmaxf(mt, xor_lanes(mt, 16));
    l += xor_lanes(l, 32);
    mt = fmaxf(mt, xor_lanes(mt, 32));
    l_part = l;
    m_true = mt;
#pragma unroll
    for (int j = 0; j < GC; ++j)
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        float v = acc[j][e];
        v += xor_lanes(v, 16);
        v += xor_lanes(v, 32);
        acc[j][e] = v;
      }
  }
  if (lane < GC) {                    // lane j: row 0, kc == j
    sm.m[w][lane] = m_run;
    sm.mt[w][lane] = m_true;
    sm.l[w][lane] = l_part;
  }
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < GC; ++j)
#pragma unroll
      for (int e = 0; e < VE; ++e) sm.acc[w][j][vcol + e] = acc[j][e];
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
      const int64_t idx = ((int64_t)r * a.num_q_heads + h) * a.max_num_partitions + blockIdx.x;
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
    int32_t max_num_partitions) {
  constexpr int TPR = D / 4;                    // threads per partition row
  constexpr int PG = kMergeThreads / TPR;       // partition rows per step
  __shared__ float wgt[kMergeMaxParts];
  __shared__ float red[kMergeThreads];
  __shared__ f32x4_t part[PG][TPR];
  const int r = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  const int n = (seq_lens[r] + partition_size - 1) / partition_size;
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

// ---------------------------------------------------------------------------
// dispatch

template <int D, int GC, bool FP8>
static hipError_t launch_decode_t(const DecodeArgs& a, bool partitioned, hipStream_t st) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int n_chunks = (G + GC - 1) / GC;
  constexpr int PD = PA_DECODE_PREFETCH;
  if (partitioned) {
    constexpr int WAVES = PA_DECODE_WAVES_SPLIT;
    const int nparts = (a.max_seq_len + a.partition_size - 1) / a.partition_size;
    if (nparts == 0) return hipSuccess;
    dim3 grid(nparts, a.num_kv_heads * n_chunks, a.num_reqs);
    hipLaunchKernelGGL((decode_kernel<D, GC, FP8, WAVES, true, PD>), grid, dim3(WAVES * 64), 0, st,
                       a, n_chunks);
  } else {
    // Few work-groups: spread each context over more waves; many: more groups.
    dim3 grid(1, a.num_kv_heads * n_chunks, a.num_reqs);
    const int64_t groups = (int64_t)grid.y * grid.z;
    if (groups < 768) {
      constexpr int WAVES = PA_DECODE_WAVES_SINGLE;
      hipLaunchKernelGGL((decode_kernel<D, GC, FP8, WAVES, false, PD>), grid, dim3(WAVES * 64), 0,
                         st, a, n_chunks);
    } else {
      constexpr int WAVES = PA_DECODE_WAVES_SPLIT;
      hipLaunchKernelGGL((decode_kernel<D, GC, FP8, WAVES, false, PD>), grid, dim3(WAVES * 64), 0,
                         st, a, n_chunks);
    }
  }
  return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t launch_decode_d(const DecodeArgs& a, bool partitioned, hipStream_t st) {
  const int G = a.num_q_heads / a.num_kv_heads;
  switch (G) {
    case 1: return launch_decode_t<D, 1, FP8>(a, partitioned, st);
    case 2: return launch_decode_t<D, 2, FP8>(a, partitioned, st);
    case 3: return launch_decode_t<D, 3, FP8>(a, partitioned, st);
    case 4: return launch_decode_t<D, 4, FP8>(a, partitioned, st);
    case 5: return launch_decode_t<D, 5, FP8>(a, partitioned, st);
    case 6: return launch_decode_t<D, 6, FP8>(a, partitioned, st);
    case 7: return launch_decode_t<D, 7, FP8>(a, partitioned, st);
    default: return launch_decode_t<D, 8, FP8>(a, partitioned, st);   // chunks of 8
  }
}

hipError_t launch_decode(const DecodeArgs& a, bool partitioned, hipStream_t st) {
  if (a.num_reqs == 0) return hipSuccess;
  const bool fp8 = a.cache_dtype != 0;
  if (a.head_dim == 64)
    return fp8 ? launch_decode_d<64, true>(a, partitioned, st)
               : launch_decode_d<64, false>(a, partitioned, st);
  return fp8 ? launch_decode_d<128, true>(a, partitioned, st)
             : launch_decode_d<128, false>(a, partitioned, st);
}

hipError_t launch_merge(void* out, const float* tmp_out, const float* max_logits,
                        const float* exp_sums, const int32_t* seq_lens, int32_t num_reqs,
                        int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                        int32_t max_num_partitions, hipStream_t st) {
  if (num_reqs == 0) return hipSuccess;
  dim3 grid(num_q_heads, num_reqs);
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kMergeThreads), 0, st, (uint16_t*)out, tmp_out,
                       max_logits, exp_sums, seq_lens, num_q_heads, partition_size,
                       max_num_partitions);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kMergeThreads), 0, st, (uint16_t*)out, tmp_out,
                       max_logits, exp_sums, seq_lens, num_q_heads, partition_size,
                       max_num_partitions);
  return hipGetLastError();
}

}  // namespace pa
