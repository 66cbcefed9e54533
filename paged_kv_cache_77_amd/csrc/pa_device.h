// Device helpers shared by the gfx950 kernels of libpa.
//
// Cache tiles: pool[num_blocks][num_kv_heads][16][head_dim]; one
// (block, KV head) tile is 16 rows of head_dim contiguous elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;   // tokens per cache block
constexpr int kWave = 64;    // CDNA wavefront

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// addressing (logical token -> physical tile): used by every kernel that
// reads the cache and by the debug gather, so tests of the gather exercise
// the kernels' own arithmetic.

// Element offset of the (physical block, KV head) tile.  int64: pools exceed
// 2^31 elements.
__device__ __forceinline__ int64_t tile_offset(int32_t phys, int g, int num_kv_heads,
                                               int head_dim) {
  return ((int64_t)phys * num_kv_heads + g) * (int64_t)(kBlock * head_dim);
}

// Element offset of cache slot `slot` (block slot/16, row slot%16), KV head g.
__device__ __forceinline__ int64_t slot_offset(int64_t slot, int g, int num_kv_heads,
                                               int head_dim) {
  const int64_t blk = slot / kBlock;
  const int row = (int)(slot - blk * kBlock);
  return tile_offset((int32_t)blk, g, num_kv_heads, head_dim) + (int64_t)row * head_dim;
}

// ---------------------------------------------------------------------------
// conversions

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Four OCP E4M3FN codes packed in a word -> four floats (gfx950 hardware
// conversion; its results for all 256 codes are checked by a GPU test).
__device__ __forceinline__ f32x4_t fp8x4_to_f32(uint32_t w) {
  f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  return f32x4_t{lo.x, lo.y, hi.x, hi.y};
}

// fp32 -> OCP E4M3FN code: round to nearest even, |y| >= 448 saturates to
// +-448 (the format has no infinity), NaN -> S.1111.111, sign kept.  Integer
// arithmetic on the fp32 bits: normal results round the 23-bit mantissa to 3
// bits (a carry moves into the exponent); results below 2^-6 are multiples
// of 2^-9, found by rounding |y| * 512 (exact) to an integer.
__device__ __forceinline__ uint32_t f32_to_fp8_e4m3fn(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t a = bits & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;                   // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;                  // >= 448, inf: saturate
  if (a >= 0x3c800000u) {                                     // >= 2^-6: normal
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));                          // rebias 127 -> 7
  }
  return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
}

// x / s for fp32 x, s, correctly rounded: the quotient is formed in fp64
// (IEEE division) and rounded once more to fp32; with 53 >= 2*24 + 2 bits the
// double rounding cannot change the result.
__device__ __forceinline__ float div_rn(float x, float s) {
  return (float)((double)x / (double)s);
}

// Two floats -> packed bf16 pair (exact for values representable in bf16,
// such as decoded FP8).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two OCP E4M3FN codes (bytes 0,1 of w when hi is false, bytes 2,3 when
// true) -> an f16 pair, low half from the lower byte.  Exact: every finite
// E4M3FN value is an f16 value (scale operand 1.0).
template <bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHi));
}

// Two floats -> f16 pair (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                c, false);
}

// Byte shuffle of two words: result byte i = byte sel_i of the 8 bytes
// {lo[0..3], hi[0..3]} (selector values 0..7).
__device__ __forceinline__ uint32_t perm_bytes(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// ---------------------------------------------------------------------------
// Store 8 source elements (one 16-byte chunk of bf16) at chunk index `dst`
// of the pool: a bit copy for bf16 pools, 8 quantised codes for FP8 pools.
template <bool FP8>
__device__ __forceinline__ void store_chunk(void* pool, int64_t dst, const uint4& src,
                                            float scale) {
  if constexpr (!FP8) {
    reinterpret_cast<uint4*>(pool)[dst] = src;
  } else {
    const uint32_t w[4] = {src.x, src.y, src.z, src.w};
    uint32_t c[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (e & 1) ? bf16hi(w[e / 2]) : bf16lo(w[e / 2]);
      c[e / 4] |= f32_to_fp8_e4m3fn(div_rn(x, scale)) << (8 * (e % 4));
    }
    reinterpret_cast<uint2*>(pool)[dst] = make_uint2(c[0], c[1]);
  }
}

// cross-lane moves (DPP within 16-lane rows; ds_bpermute across rows)

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;   // rotate right by 4 within 16 lanes
constexpr int kRowRor8 = 0x128;   // rotate right by 8 within 16 lanes (== xor 8)

__device__ __forceinline__ float xor_lanes(float x, int m) { return __shfl_xor(x, m, kWave); }

// All-reduce of x with lane (l ^ 32) or (l ^ 16) on the vector ALU.
// v_permlane32_swap a, b exchanges lanes 32-63 of a with lanes 0-31 of b, so
// afterwards a = [a lanes 0-31, b lanes 0-31] and b = [a lanes 32-63,
// b lanes 32-63] (v_permlane16_swap the same with 16-lane rows: a = rows
// a0 b0 a2 b2, b = a1 b1 a3 b3; checked on gfx950).  With a = b = x every
// lane ends with x of both partners in {a, b}, in a lane-dependent order --
// hence only commutative reductions here.  No LDS crossbar traffic, unlike
// ds_bpermute.  Written as asm with both registers read-write: through the
// compiler builtin, ROCm 7.2's backend reads the first result in place of
// the second when both inputs carry the same value.  The s_nop gives the
// two wait states a VALU write needs before a permlane reads it.
template <bool ROW16>
__device__ __forceinline__ void swap_halves(float x, float& r0, float& r1) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  if constexpr (ROW16)
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  else
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  r0 = __builtin_bit_cast(float, a);
  r1 = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float sum_xor32(float x) {
  float r0, r1;
  swap_halves<false>(x, r0, r1);
  return r0 + r1;
}
__device__ __forceinline__ float max_xor32(float x) {
  float r0, r1;
  swap_halves<false>(x, r0, r1);
  return fmaxf(r0, r1);
}
__device__ __forceinline__ float sum_xor16(float x) {
  float r0, r1;
  swap_halves<true>(x, r0, r1);
  return r0 + r1;
}
__device__ __forceinline__ float max_xor16(float x) {
  float r0, r1;
  swap_halves<true>(x, r0, r1);
  return fmaxf(r0, r1);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace pa
