// common.h -- device helpers shared by the NVFP4 KV-cache kernels (gfx950).
//
// Format facts used here ("NVIDIA解説: NVFP4 KV Cacheで長コンテキストLLM推論を
// 最適化", section E2M1 + 2レベルスケーリング): E2M1 element codes, one E4M3
// scale per 16 elements, one FP32 scale per tensor.  The E4M3 variant is OCP
// E4M3FN (bias 7, largest finite 448), which is also gfx950's FP8 format.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kD = 128;        // head dimension
constexpr int kPage = 16;      // tokens per page
constexpr int kBlock = 16;     // elements per micro-block
constexpr int kNBlk = kD / kBlock;
constexpr int kSlab = kPage * kD / 2;        // code bytes per (page, head): 1024
constexpr int kScaleSlab = kPage * kNBlk;    // scale bytes per (page, head): 128
constexpr int kMxBlock = 32;                  // MXFP4 elements per block
constexpr int kMxNBlk = kD / kMxBlock;
constexpr int kMxScaleSlab = kPage * kMxNBlk; // MXFP4 scale bytes per (page, head): 64

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16 / 8 bytes read or written once: loads and stores with the non-temporal
// hint (the lines are not kept for reuse)
__device__ __forceinline__ uint4 load_once16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_once8(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(static_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void store_once16(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, static_cast<u32x4*>(p));
}

// ------------------------------------------------------------ E4M3 decode

// Exact value of a non-negative E4M3FN byte (sign ignored; 0x7F never used).
__device__ __forceinline__ float e4m3_to_float(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  if (e == 0u) return (float)m * 0x1p-9f;
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// The value of a block scale code the encoders produced (0 .. 0x7E, never
// the NaN pattern) with the hardware conversion: one instruction, no branch.
// The scale operand 1.0 leaves the value unchanged.
__device__ __forceinline__ float e4m3_code_value(uint32_t code) {
  return __builtin_amdgcn_cvt_scalef32_f32_fp8(code, 1.0f, 0);
}

// Two E4M3 bytes (byte 0 and byte 1 of `w` when hi == false, bytes 2, 3 when
// true) to two exact halves.  The conversion's scale operand only applies a
// power of two; 1.0 leaves the values unchanged.
__device__ __forceinline__ halfx2 e4m3x2_to_half(uint32_t w, bool hi) {
  fp16x2 h = hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(halfx2, h);
}

// Two E2M1 codes (low nibble -> element 0, high nibble -> element 1) of byte
// `sel` of `w` to two exact halves.
template <int SEL>
__device__ __forceinline__ halfx2 e2m1x2_to_half(uint32_t w) {
  fp16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
  return __builtin_bit_cast(halfx2, h);
}

// Two E2M1 codes of byte SEL of `w` times the power of two `scale` (an FP32
// 2^k, or 0), as two halves; exact while the products lie in FP16's range.
template <int SEL>
__device__ __forceinline__ halfx2 e2m1x2_to_half_scaled(uint32_t w, float scale) {
  fp16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, SEL);
  return __builtin_bit_cast(halfx2, h);
}

// ------------------------------------------------------ block scale (E4M3)

// Nearest E4M3FN code to the exact quotient amax / (6 s_t), ties to the even
// code, clamped to 448 (0x7E).  six_st = 6 * (double)s_t is exact.  The double
// quotient q = RN(amax / six_st) cannot cross or land on an E4M3 midpoint
// unless the exact quotient does: amax has 24 significant bits and
// six_st * midpoint at most 2 + 24 + 5, so a non-zero distance from a midpoint
// is at least ~2^-31 relative, far above double rounding (2^-53).
__device__ __forceinline__ uint32_t block_scale_code(float amax, double six_st) {
  double q = (double)amax / six_st;
  if (!(q < 448.0)) return 0x7Eu;                 // also catches NaN / inf
  if (q < 0x1p-6) return (uint32_t)rint(q * 512.0);   // subnormal spacing 2^-9
  int e = ilogb(q);                                 // -6 .. 8
  double r = rint(ldexp(q, 3 - e));                 // 8 .. 16, nearest-even
  return (uint32_t)((e + 6) * 8 + (int)r);
}

// The same code, fast path first.  q = amax * inv6 (inv6 = 1/(6 s_t) rounded
// to FP32) is within 2^-23 relative of the exact quotient, so q (1 - 2^-20)
// and q (1 + 2^-20) bracket it; the hardware FP32 -> E4M3 conversion rounds
// to nearest even and is monotone, so when the two brackets convert to the
// same code that code is the exact answer.  Quotients of 448 and above clamp
// to 0x7E; anything else (a bracket straddling a midpoint or 448, or a
// quotient far below the E4M3 range where FP32 loses precision) takes the
// exact double path.
__device__ __forceinline__ uint32_t block_scale_code_fast(float amax, float inv6, double six_st) {
  const float q = amax * inv6;
  const float lo = q * (1.0f - 0x1p-20f), hi = q * (1.0f + 0x1p-20f);
  if (lo >= 448.0f) return 0x7Eu;
  if (hi < 448.0f && q >= 0x1p-100f) {
    const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, 0, false);
    if ((w & 0xFFu) == ((w >> 8) & 0xFFu)) return w & 0xFFu;
  }
  if (amax == 0.0f) return 0u;
  return block_scale_code(amax, six_st);
}

// ------------------------------------------------------- element codes

// Magnitude code (0..7) of |x| for exact step d = s_block * s_t (double):
// the nearest E2M1 value to |x| / d, ties to the even code, clamped to 6.
// Thresholds d * {1/4, 3/4, 5/4, 7/4, 5/2, 7/2, 5} are exact in double.
__device__ __forceinline__ uint32_t e2m1_mag_exact(float x, double d) {
  double ax = fabs((double)x);
  uint32_t m = 0;
  m += ax > d * 0.25;
  m += ax >= d * 0.75;
  m += ax > d * 1.25;
  m += ax >= d * 1.75;
  m += ax > d * 2.5;
  m += ax >= d * 3.5;
  m += ax > d * 5.0;
  return m;
}

// Eight element codes of one half-block, packed as nibbles (element j in bits
// 4j..4j+3).  Fast path: the hardware FP32->E2M1 conversion rounds to nearest
// even (and saturates at 6) for every FP32 input; x * y_lo and x * y_hi
// bracket the exact quotient x / d, so when both conversions agree the exact
// code is that value (the rounding is monotone); an element where they
// disagree is decided exactly at its one candidate midpoint.  When d is
// outside the range where the FP32 bracket holds, the lane redoes its eight
// elements with exact double thresholds.
__device__ __forceinline__ uint32_t encode8(const float x[8], uint32_t sb_code, float s_t) {
  // the midpoint decision below needs |x| - p rounded on its own: a fused
  // |x| - a * s_t would compare a different residual with e
#pragma clang fp contract(off)
  auto signs = [&]() {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= (__float_as_uint(x[j]) >> 31) << (4 * j + 3);
    return w;
  };
  if (sb_code == 0u) return signs();                // zero scale: magnitude 0
  // d = s_block * s_t in FP32 (2^-24 relative) and its hardware reciprocal
  // (1 ulp) give y within ~2^-22 of 1/d; the brackets are 2^-20 wide
  const float df = e4m3_code_value(sb_code) * s_t;
  const bool fast = df >= 0x1p-100f && df <= 0x1p100f;
  uint32_t lo = 0, hi = 0;
  if (fast) {
    const float y = __builtin_amdgcn_rcpf(df);
    const float y_lo = y * (1.0f - 0x1p-20f);
    const float y_hi = y * (1.0f + 0x1p-20f);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x[0] * y_lo, x[1] * y_lo, 1.0f, 0);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x[2] * y_lo, x[3] * y_lo, 1.0f, 1);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x[4] * y_lo, x[5] * y_lo, 1.0f, 2);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x[6] * y_lo, x[7] * y_lo, 1.0f, 3);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x[0] * y_hi, x[1] * y_hi, 1.0f, 0);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x[2] * y_hi, x[3] * y_hi, 1.0f, 1);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x[4] * y_hi, x[5] * y_hi, 1.0f, 2);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x[6] * y_hi, x[7] * y_hi, 1.0f, 3);
  }
  if (fast) {
    // an element whose brackets disagree sits within 2^-19 of the one
    // midpoint t between its two candidate codes c and c+1; decide it
    // exactly: t * s_block is exact in FP32 (at most 7 significant bits),
    // p + e = t * s_block * s_t exactly (e from an FMA), and |x| - p is exact
    // (Sterbenz: |x| and p are within 2^-18 of each other)
    uint32_t diff = (lo ^ hi) & 0x77777777u;
    if (diff) {
      const float sbv = e4m3_code_value(sb_code);
      do {
        const int sh = (__builtin_ctz(diff) >> 2) << 2;
        const uint32_t c = (lo >> sh) & 7u;                   // the lower candidate
        const float t = c < 4u ? 0.25f + 0.5f * (float)c : (c == 4u ? 2.5f : (c == 5u ? 3.5f : 5.0f));
        const float a = sbv * t;
        const float pr = a * s_t;
        const float e = __builtin_fmaf(a, s_t, -pr);
        const float r = fabsf(x[sh >> 2]) - pr;
        const bool up = r > e || (r == e && ((c + 1u) & 1u) == 0u);
        lo = (lo & ~(7u << sh)) | ((c + (up ? 1u : 0u)) << sh);
        diff &= ~(15u << sh);
      } while (diff);
    }
    // the conversion keeps the sign of x * y, which is that of x (y > 0;
    // -0 and an element rounded to zero give the sign bit too, a value
    // past 6 saturates with its sign)
    return lo;
  }
  const double d = (double)e4m3_to_float(sb_code) * (double)s_t;   // exact
  uint32_t w = signs();
#pragma unroll
  for (int j = 0; j < 8; ++j) w |= e2m1_mag_exact(x[j], d) << (4 * j);
  return w;
}

// encode8 for a whole 16-element block (x0: elements 0-7, x1: 8-15): the
// same rounding, with the block's step, reciprocal and brackets computed
// once and one check for an undecided element.
__device__ __forceinline__ uint2 encode16(const float x0[8], const float x1[8], uint32_t sb_code, float s_t) {
#pragma clang fp contract(off)
  const float df = e4m3_code_value(sb_code) * s_t;
  if (sb_code == 0u || !(df >= 0x1p-100f && df <= 0x1p100f))
    return make_uint2(encode8(x0, sb_code, s_t), encode8(x1, sb_code, s_t));
  const float y = __builtin_amdgcn_rcpf(df);
  const float y_lo = y * (1.0f - 0x1p-20f);
  const float y_hi = y * (1.0f + 0x1p-20f);
  uint32_t lo[2] = {0u, 0u}, hi[2] = {0u, 0u};
  // (the conversion's word select must be a literal)
#define NVFP4_BRACKETS(H, X)                                                                          \
  lo[H] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo[H], X[0] * y_lo, X[1] * y_lo, 1.0f, 0);          \
  lo[H] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo[H], X[2] * y_lo, X[3] * y_lo, 1.0f, 1);          \
  lo[H] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo[H], X[4] * y_lo, X[5] * y_lo, 1.0f, 2);          \
  lo[H] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo[H], X[6] * y_lo, X[7] * y_lo, 1.0f, 3);          \
  hi[H] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi[H], X[0] * y_hi, X[1] * y_hi, 1.0f, 0);          \
  hi[H] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi[H], X[2] * y_hi, X[3] * y_hi, 1.0f, 1);          \
  hi[H] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi[H], X[4] * y_hi, X[5] * y_hi, 1.0f, 2);          \
  hi[H] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi[H], X[6] * y_hi, X[7] * y_hi, 1.0f, 3);
  NVFP4_BRACKETS(0, x0)
  NVFP4_BRACKETS(1, x1)
#undef NVFP4_BRACKETS
  if (((lo[0] ^ hi[0]) | (lo[1] ^ hi[1])) & 0x77777777u) {
    // an element between its brackets: decided exactly as in encode8
    const float sbv = e4m3_code_value(sb_code);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* x = h ? x1 : x0;
      uint32_t diff = (lo[h] ^ hi[h]) & 0x77777777u;
      while (diff) {
        const int sh = (__builtin_ctz(diff) >> 2) << 2;
        const uint32_t c = (lo[h] >> sh) & 7u;
        const float t = c < 4u ? 0.25f + 0.5f * (float)c : (c == 4u ? 2.5f : (c == 5u ? 3.5f : 5.0f));
        const float a = sbv * t;
        const float pr = a * s_t;
        const float e = __builtin_fmaf(a, s_t, -pr);
        const float r = fabsf(x[sh >> 2]) - pr;
        const bool up = r > e || (r == e && ((c + 1u) & 1u) == 0u);
        lo[h] = (lo[h] & ~(7u << sh)) | ((c + (up ? 1u : 0u)) << sh);
        diff &= ~(15u << sh);
      }
    }
  }
  return make_uint2(lo[0], lo[1]);
}

// 2^x with the hardware exponential (results below 2^-126 flush to zero,
// which is harmless for softmax weights; exp2(-inf) = 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, nearest even (finite inputs)
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// float -> bf16 bits, nearest even (the hardware conversion)
__device__ __forceinline__ short bf16_bits(float f) { return __builtin_bit_cast(short, (__bf16)f); }

// Cross-row reductions inside a wave64 (rows of 16 lanes).  permlane16_swap
// with the same register on both sides yields, per lane, its own value and
// the value of the lane 16 away in the paired row; permlane32_swap likewise
// across the two halves.
__device__ __forceinline__ float max_across_rows(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across_rows(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float max_across_halves(float v) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across_halves(float v) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace nvfp4
