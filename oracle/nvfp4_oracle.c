/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for the NVFP4 KV-cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product library
 * (decode_attention_nvfp4_amd/) never calls it and shares no code with it.
 *
 * Everything here is written from the definitions on the source pages, in
 * the simplest form that can be checked by eye: scalar loops, exact
 * threshold comparisons done in IEEE double where the operands are provably
 * exact, and double accumulation for attention.  No blocking, no fusion,
 * no fast-math.
 *
 * Sources (page titles; sections named where cited below):
 *  [EXPL] "NVIDIA解説: NVFP4 KV Cacheで長コンテキストLLM推論を最適化 —
 *          メモリ50%削減・TTFT 3倍高速化"
 *  [GB10] "一個 Triton FP8 繞道補丁，為 DGX Spark 的 GB10 擠出多 17% 的 NVFP4 速度"
 *  [RC17] "TensorRT-LLM rc17 が SM121（DGX Spark）向けに NVFP4 MoE バックエンドと
 *          NVFP4 KV キャッシュを追加"
 *  [TRTL] "Compilation d'inferences spécialisées en matériel FP8 et NVFP4 sur
 *          Blackwell"
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *  - E2M1 grid: sign + 2-bit exponent (bias 1) + 1-bit mantissa, giving the
 *    magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; the pages fix only the bit
 *    widths and the ~[-6, 6] range ([EXPL] §E2M1 + 2レベルスケーリング).
 *  - E4M3 is the OCP E4M3FN encoding (bias 7, no infinities, 0x7F/0xFF NaN,
 *    largest finite 448).
 *  - Tensor scale s_t = amax(|X|) / (6 * 448), computed in FP32, so that the
 *    tensor's largest magnitude maps onto the largest block scale times the
 *    largest E2M1 value.  The pages only say it is one FP32 value per tensor.
 *  - Block scale: the E4M3 value nearest to (block amax) / (6 * s_t), ties to
 *    the even code, clamped to 448 (never NaN).  The pages do not give the
 *    selection rule; this maps each block's largest magnitude onto 6.
 *  - Element code: the E2M1 value nearest to x / (s_block * s_t), computed in
 *    exact real arithmetic, ties to the even code, clamped to 6.  The sign bit
 *    is always the sign of x (so -0 and small negatives give code 0x8).
 *    A zero block scale gives magnitude 0 for every element.
 *  - Dequantization multiplies by s_t, which is dividing by the global
 *    encode scale g = 1/s_t ([GB10] §這個 80 行的 Triton 繞道: the global
 *    scale must divide, not multiply).
 *  - MSE-searched block scale ([EXPL] §E2M1 + 2レベルスケーリング describes
 *    the E4M3 block scale as chosen for least squared error, with no
 *    procedure): among the E4M3 codes within 8 of the amax/6 code (code 0
 *    excluded), the one whose element codes give the smallest squared error
 *    of the block against the
 *    exact products e2m1 * s_block * s_t; the error is summed in double over
 *    elements 0..15 in order, each operation rounded once (no fused
 *    multiply-add); ties go to the candidate nearest the amax/6 code, then
 *    to the smaller code.  A block whose amax/6 code is 0 keeps 0.
 *  - The comparison formats.  FP8 KV cache ([EXPL] and [TRTL] set NVFP4
 *    against an FP8 cache without defining it): every element is the E4M3
 *    value nearest to x / s_t8 (FP32 quotient), ties to the even code,
 *    clamped to 448, with one FP32 scale per tensor s_t8 = amax(|X|) / 448;
 *    dequantization multiplies by s_t8.  BF16 KV cache: the bf16 values
 *    themselves.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_D 128      /* head dimension */
#define ORC_BLOCK 16   /* micro-block length ([EXPL] §E2M1 + 2レベルスケーリング, Level 1) */
#define ORC_NBLK (ORC_D / ORC_BLOCK)

/* ---------------------------------------------------------------- formats */

/* E2M1 magnitudes, code order 0..7 ([EXPL] §E2M1 + 2レベルスケーリング). */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Value of a 4-bit E2M1 code (bit 3 = sign). */
double orc_e2m1_value(unsigned code) {
  double m = kE2M1[code & 7u];
  return (code & 8u) ? -m : m;
}

/* Value of an OCP E4M3FN byte: 1 sign, 4 exponent (bias 7), 3 mantissa
 * bits; exponent field 0 is subnormal (m/8 * 2^-6); 0x7F and 0xFF are NaN. */
double orc_e4m3_value(unsigned byte) {
  unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  double v;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -v : v;
}

/* ------------------------------------------------------- tensor scale (A0) */

/* s_t = amax(|x|) / (6 * 448) in FP32. */
float orc_tensor_scale(const float* x, size_t n) {
  float amax = 0.0f;
  for (size_t i = 0; i < n; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  return amax / 2688.0f;
}

/* s_t for a given amax (the same formula, for callers that reduce in pieces). */
float orc_tensor_scale_from_amax(float amax) { return amax / 2688.0f; }

float orc_abs_max(const float* x, size_t n) {
  float amax = 0.0f;
  for (size_t i = 0; i < n; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  return amax;
}

/* ------------------------------------------------------------ block scale */

/* Nearest non-negative finite E4M3 code to the exact quotient a / (6 s_t),
 * ties to the even code, clamped to the largest finite code 0x7E (448).
 * Walks the 126 midpoints between consecutive codes in increasing order.
 * Each threshold 6 * s_t * mid is exact in double: 2 + 24 + 5 significant
 * bits.  a is an FP32 magnitude, also exact in double. */
unsigned orc_block_scale_code(float amax_block, float s_t) {
  double a = (double)amax_block;
  double six_st = 6.0 * (double)s_t;
  unsigned code = 0;
  for (unsigned k = 0; k < 126u; ++k) {
    double mid = 0.5 * (orc_e4m3_value(k) + orc_e4m3_value(k + 1u));
    double t = six_st * mid;
    if (a > t) {
      code = k + 1u;
    } else {
      if (a == t) code = (k % 2u == 0u) ? k : k + 1u;
      break;
    }
  }
  return code;
}

/* --------------------------------------------------------- element code */

/* 4-bit code of x for block-scale byte sb and tensor scale s_t: the E2M1
 * magnitude nearest to |x| / (sb * s_t), ties to the even code, clamped to 6;
 * sign bit from x.  Thresholds sb * s_t * mid are exact in double
 * (4 + 24 + 3 significant bits). */
unsigned orc_element_code(float x, unsigned sb_code, float s_t) {
  unsigned sign = signbit(x) ? 8u : 0u;
  double sb = orc_e4m3_value(sb_code);
  double d = sb * (double)s_t;
  double ax = fabs((double)x);
  unsigned mag = 0;
  if (d > 0.0) {
    for (unsigned k = 0; k < 7u; ++k) {
      double mid = 0.5 * (kE2M1[k] + kE2M1[k + 1u]);
      double t = d * mid;
      if (ax > t) {
        mag = k + 1u;
      } else {
        if (ax == t) mag = (k % 2u == 0u) ? k : k + 1u;
        break;
      }
    }
  }
  return sign | mag;
}

/* Array forms of the two encoders above (used by the exhaustive checks). */
void orc_element_codes(const float* x, size_t n, unsigned sb_code, float s_t, uint8_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_element_code(x[i], sb_code, s_t);
}

void orc_block_scale_codes(const float* amax, size_t n, float s_t, uint8_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_block_scale_code(amax[i], s_t);
}

/* ---------------------------------------------------- quantize rows (A1) */

/* Quantize nrows rows of 128 FP32 values.  codes: one 4-bit code per byte,
 * [nrows][128]; scales: E4M3 bytes, [nrows][8], block j covering elements
 * 16j..16j+15 of the row ([EXPL] §量子化・逆量子化フロー, quantize in
 * 16-element blocks on append). */
void orc_quantize_rows(const float* x, size_t nrows, float s_t,
                       uint8_t* codes, uint8_t* scales) {
  for (size_t r = 0; r < nrows; ++r) {
    const float* row = x + r * ORC_D;
    for (unsigned j = 0; j < ORC_NBLK; ++j) {
      float amax = 0.0f;
      for (unsigned i = 0; i < ORC_BLOCK; ++i) {
        float a = fabsf(row[j * ORC_BLOCK + i]);
        if (a > amax) amax = a;
      }
      unsigned sb = orc_block_scale_code(amax, s_t);
      scales[r * ORC_NBLK + j] = (uint8_t)sb;
      for (unsigned i = 0; i < ORC_BLOCK; ++i) {
        unsigned e = j * ORC_BLOCK + i;
        codes[r * ORC_D + e] = (uint8_t)orc_element_code(row[e], sb, s_t);
      }
    }
  }
}

/* ------------------------------------------ MSE-searched block scale */

#define ORC_MSE_RADIUS 8

/* Squared error of a 16-element block under block-scale code sb: the sum
 * over e = 0..15, in order, of (x_e - e2m1(code_e) * sb * s_t)^2, with the
 * element codes of orc_element_code.  The product is exact in double; the
 * difference, the square and each partial sum are rounded once. */
double orc_block_sq_error(const float* x, unsigned sb, float s_t) {
  double sum = 0.0;
  for (unsigned e = 0; e < ORC_BLOCK; ++e) {
    unsigned c = orc_element_code(x[e], sb, s_t);
    double p = orc_e2m1_value(c) * orc_e4m3_value(sb) * (double)s_t;
    double d = (double)x[e] - p;
    double sq = d * d;
    sum = sum + sq;
  }
  return sum;
}

/* The MSE-searched block-scale code of x[0..15] (rule in the header). */
unsigned orc_block_scale_code_mse(const float* x, float s_t) {
  float amax = 0.0f;
  for (unsigned e = 0; e < ORC_BLOCK; ++e) {
    float a = fabsf(x[e]);
    if (a > amax) amax = a;
  }
  unsigned c0 = orc_block_scale_code(amax, s_t);
  if (c0 == 0u) return 0u;
  unsigned best = c0;
  double best_err = orc_block_sq_error(x, c0, s_t);
  for (int dist = 1; dist <= ORC_MSE_RADIUS; ++dist) {
    for (int sgn = -1; sgn <= 1; sgn += 2) {      /* the smaller code first */
      int c = (int)c0 + sgn * dist;
      if (c < 1 || c > 126) continue;
      double err = orc_block_sq_error(x, (unsigned)c, s_t);
      if (err < best_err) {
        best = (unsigned)c;
        best_err = err;
      }
    }
  }
  return best;
}

/* quantize_rows with the MSE-searched block scale. */
void orc_quantize_rows_mse(const float* x, size_t nrows, float s_t,
                           uint8_t* codes, uint8_t* scales) {
  for (size_t r = 0; r < nrows; ++r) {
    const float* row = x + r * ORC_D;
    for (unsigned blk = 0; blk < ORC_NBLK; ++blk) {
      unsigned sb = orc_block_scale_code_mse(row + blk * ORC_BLOCK, s_t);
      scales[r * ORC_NBLK + blk] = (uint8_t)sb;
      for (unsigned e = blk * ORC_BLOCK; e < (blk + 1) * ORC_BLOCK; ++e)
        codes[r * ORC_D + e] = (uint8_t)orc_element_code(row[e], sb, s_t);
    }
  }
}

/* -------------------------------------------------- dequantize rows (A10) */

/* x_hat = FP32( e2m1(code) * sb * s_t ): the two-level product of [EXPL]
 * §E2M1 + 2レベルスケーリング, with s_t the decode-direction tensor scale.
 * The product e2m1 * sb * s_t is exact in double (3 + 4 + 24 bits), so the
 * cast gives one FP32 rounding. */
float orc_dequant_value(unsigned code, unsigned sb_code, float s_t) {
  double v = orc_e2m1_value(code) * orc_e4m3_value(sb_code) * (double)s_t;
  return (float)v;
}

void orc_dequant_rows(const uint8_t* codes, const uint8_t* scales, size_t nrows,
                      float s_t, float* out) {
  for (size_t r = 0; r < nrows; ++r)
    for (unsigned e = 0; e < ORC_D; ++e)
      out[r * ORC_D + e] =
          orc_dequant_value(codes[r * ORC_D + e], scales[r * ORC_NBLK + e / ORC_BLOCK], s_t);
}

/* FP32 -> bfloat16 bits, round to nearest even (NaN kept quiet). */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

void orc_f32_to_bf16_array(const float* x, size_t n, uint16_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(x[i]);
}

/* ------------------------------------------ FP8 comparison format (E4M3) */

/* Tensor scale of the FP8 cache: amax / 448 in FP32. */
float orc_fp8_tensor_scale_from_amax(float amax) { return amax / 448.0f; }

/* FP8 code of x: v = x / s_t in FP32 (IEEE division), then the finite E4M3
 * magnitude nearest to |v|, ties to the even code, clamped to 448 (code
 * 0x7E); bit 7 is the sign of v.  Walks the 126 midpoints between
 * consecutive codes; |v| and each midpoint are exact in double. */
unsigned orc_fp8_code(float x, float s_t) {
  float v = x / s_t;
  unsigned sign = signbit(v) ? 0x80u : 0u;
  double a = fabs((double)v);
  unsigned code = 0;
  for (unsigned k = 0; k < 126u; ++k) {
    double mid = 0.5 * (orc_e4m3_value(k) + orc_e4m3_value(k + 1u));
    if (a > mid) {
      code = k + 1u;
    } else {
      if (a == mid) code = (k % 2u == 0u) ? k : k + 1u;
      break;
    }
  }
  return sign | code;
}

void orc_fp8_codes(const float* x, size_t n, float s_t, uint8_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_fp8_code(x[i], s_t);
}

/* Dequantized FP8 element: fl32(e4m3(code) * s_t); the product of a 4-bit
 * and a 24-bit significand is exact in double, so one rounding.  Code 0x80
 * gives -0.0. */
float orc_fp8_value(unsigned code, float s_t) {
  double m = orc_e4m3_value(code & 0x7Fu) * (double)s_t;
  return (float)((code & 0x80u) ? -m : m);
}

void orc_fp8_dequant(const uint8_t* codes, size_t n, float s_t, float* out) {
  for (size_t i = 0; i < n; ++i) out[i] = orc_fp8_value(codes[i], s_t);
}

/* ---------------------------------------------------------------- MXFP4 */

/* MXFP4, the OCP format set against NVFP4 in [EXPL] §MXFP4との比較 (table):
 * E2M1 elements in blocks of 32, one E8M0 (power-of-two) scale per block,
 * no tensor scale.  Readings (the page gives only block size and scale
 * type; the rest follows the OCP MX definition): block exponent
 * e = floor(log2(amax)) - 2, 2 being the exponent of E2M1's largest value
 * 6 = 1.5 * 2^2, clamped to [-127, 127]; a zero block takes -127; the
 * scale byte is e + 127.  Element: the E2M1 magnitude nearest to |x| / 2^e,
 * ties to the even code, clamped to 6; sign bit from x. */
#define ORC_MX_BLOCK 32
#define ORC_MX_NBLK (ORC_D / ORC_MX_BLOCK)

int orc_mx_block_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e = ilogbf(amax) - 2;          /* floor(log2(amax)), subnormals included */
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* 2^(byte - 127); the byte 0xFF (NaN in E8M0) is not produced here. */
double orc_e8m0_value(unsigned byte) { return ldexp(1.0, (int)byte - 127); }

unsigned orc_mx_element_code(float x, int e) {
  unsigned sign = signbit(x) ? 8u : 0u;
  double r = fabs((double)x) / ldexp(1.0, e);   /* exact: a power-of-two scaling */
  unsigned mag = 0;
  for (unsigned k = 0; k < 7u; ++k) {
    double mid = 0.5 * (kE2M1[k] + kE2M1[k + 1u]);
    if (r > mid) {
      mag = k + 1u;
    } else {
      if (r == mid) mag = (k % 2u == 0u) ? k : k + 1u;
      break;
    }
  }
  return sign | mag;
}

/* Quantize nrows rows of 128 values: codes [nrows][128] (one 4-bit code per
 * byte), scales [nrows][4] E8M0 bytes, block j covering elements
 * 32j..32j+31. */
void orc_mx_quantize_rows(const float* x, size_t nrows, uint8_t* codes, uint8_t* scales) {
  for (size_t r = 0; r < nrows; ++r) {
    const float* row = x + r * ORC_D;
    for (unsigned j = 0; j < ORC_MX_NBLK; ++j) {
      float amax = 0.0f;
      for (unsigned i = 0; i < ORC_MX_BLOCK; ++i) {
        float a = fabsf(row[j * ORC_MX_BLOCK + i]);
        if (a > amax) amax = a;
      }
      int e = orc_mx_block_exp(amax);
      scales[r * ORC_MX_NBLK + j] = (uint8_t)(e + 127);
      for (unsigned i = 0; i < ORC_MX_BLOCK; ++i) {
        unsigned k = j * ORC_MX_BLOCK + i;
        codes[r * ORC_D + k] = (uint8_t)orc_mx_element_code(row[k], e);
      }
    }
  }
}

/* x_hat = e2m1(code) * 2^(scale - 127), exact in FP32 for every value the
 * quantizer produces from FP32 input (at least 0.5 * 2^-127). */
void orc_mx_dequant_rows(const uint8_t* codes, const uint8_t* scales, size_t nrows, float* out) {
  for (size_t r = 0; r < nrows; ++r)
    for (unsigned k = 0; k < ORC_D; ++k)
      out[r * ORC_D + k] = (float)(orc_e2m1_value(codes[r * ORC_D + k]) *
                                   orc_e8m0_value(scales[r * ORC_MX_NBLK + k / ORC_MX_BLOCK]));
}

/* ------------------------------------------------- NVFP4 -> FP8 conversion */

/* Conversion of a row-major NVFP4 tensor to FP8 for an FP8 GEMM ([GB10]
 * §這個 80 行的 Triton 繞道: NVFP4 weights are turned into FP8 when the model
 * loads, and the dequantization divides by the global scale).  Element e of
 * the flat tensor: code = nibble e%2 (low nibble first) of byte e/2, block
 * scale byte e/16; its value e2m1 * s_block (exact in FP32) is divided by
 * the global encode scale g in FP32 (IEEE division), and the result is
 * written as the FP8 code of that value over the output scale s8 (the rule
 * of orc_fp8_code: FP32 quotient, nearest E4M3, ties to even, clamped to
 * 448).  Dequantizing the output multiplies by s8. */
unsigned orc_nvfp4_to_fp8_code(unsigned code, unsigned sb, float g, float s8) {
  float v = (float)(orc_e2m1_value(code) * orc_e4m3_value(sb));
  float xh = v / g;
  return orc_fp8_code(xh, s8);
}

void orc_nvfp4_to_fp8(const uint8_t* codes, const uint8_t* scales, size_t n,
                      float g, float s8, uint8_t* out) {
  for (size_t e = 0; e < n; ++e) {
    unsigned byte = codes[e / 2];
    unsigned c = (e % 2 == 0) ? (byte & 15u) : (byte >> 4);
    /* block scales are non-negative; a set sign bit is ignored */
    out[e] = (uint8_t)orc_nvfp4_to_fp8_code(c, scales[e / 16] & 0x7Fu, g, s8);
  }
}

/* ----------------------------------------------------------- attention */

/* Softmax attention of Hq query rows over L tokens of an already dequantized
 * cache kh, vh ([L][Hkv][128] FP32).  Products and sums in double; query head
 * h reads KV head h / (Hq / Hkv); L == 0 gives zeros. */
static void attend_dequantized(const float* q, int Hq, int Hkv, const float* kh,
                               const float* vh, int L, double scale, double* work,
                               float* out) {
  int G = Hq / Hkv;
  for (int h = 0; h < Hq; ++h) {
    int kvh = h / G;
    const float* qh = q + (size_t)h * ORC_D;
    if (L <= 0) {
      for (int d = 0; d < ORC_D; ++d) out[(size_t)h * ORC_D + d] = 0.0f;
      continue;
    }
    double mx = -INFINITY;
    for (int t = 0; t < L; ++t) {
      const float* k = kh + ((size_t)t * Hkv + kvh) * ORC_D;
      double s = 0.0;
      for (int d = 0; d < ORC_D; ++d) s += (double)qh[d] * (double)k[d];
      s *= scale;
      work[t] = s;
      if (s > mx) mx = s;
    }
    double den = 0.0;
    double num[ORC_D];
    for (int d = 0; d < ORC_D; ++d) num[d] = 0.0;
    for (int t = 0; t < L; ++t) {
      const float* v = vh + ((size_t)t * Hkv + kvh) * ORC_D;
      double p = exp(work[t] - mx);
      den += p;
      for (int d = 0; d < ORC_D; ++d) num[d] += p * (double)v[d];
    }
    for (int d = 0; d < ORC_D; ++d) out[(size_t)h * ORC_D + d] = (float)(num[d] / den);
  }
}

/* Attention over an already dequantized cache ([L][Hkv][128] FP32 each), as
 * for the comparison formats: FP8 values after orc_fp8_dequant, BF16 values
 * widened.  Returns 0. */
int orc_attend_dense(const float* q, int Hq, int Hkv, const float* kh, const float* vh,
                     int L, double scale, double* work, float* out) {
  attend_dequantized(q, Hq, Hkv, kh, vh, L, scale, work, out);
  return 0;
}

/* Attention of Hq query rows of one sequence over its first L cached tokens:
 * the cache is dequantized first, then attended ([EXPL] §量子化・逆量子化フロー:
 * dequantize before the attention math; [TRTL] §Pourquoi FP8 est toujours le
 * sol pour KV cache: FP32 accumulator -- here double).
 *   q:       [Hq][128] FP32 (bf16 inputs widened exactly)
 *   kcodes:  [L][Hkv][128] one code per byte;  kscales: [L][Hkv][8]
 *   vcodes / vscales: same for V
 *   work:    >= L doubles of scratch
 *   out:     [Hq][128] FP32
 * Returns 0, or -1 if scratch memory could not be allocated. */
int orc_attend(const float* q, int Hq, int Hkv,
               const uint8_t* kcodes, const uint8_t* kscales, float s_tk,
               const uint8_t* vcodes, const uint8_t* vscales, float s_tv,
               int L, double scale, double* work, float* out) {
  size_t n = (size_t)(L > 0 ? L : 0) * Hkv;
  float* kh = (float*)malloc((n ? n : 1) * ORC_D * sizeof(float));
  float* vh = (float*)malloc((n ? n : 1) * ORC_D * sizeof(float));
  if (!kh || !vh) { free(kh); free(vh); return -1; }
  orc_dequant_rows(kcodes, kscales, n, s_tk, kh);
  orc_dequant_rows(vcodes, vscales, n, s_tv, vh);
  attend_dequantized(q, Hq, Hkv, kh, vh, L, scale, work, out);
  free(kh);
  free(vh);
  return 0;
}

/* Causal chunk: query i of a chunk sits at absolute position prefix + i and
 * attends to cached tokens 0 .. prefix + i (all total_len tokens when causal
 * is 0).  Only the listed query indices rows[] are computed, so a caller can
 * sample a large chunk.  q and out: [nrows][Hq][128]; the cache arrays hold
 * total_len tokens.  Returns 0, or -1 on allocation failure. */
int orc_prefill_rows(const float* q, const int* rows, int nrows, int Hq, int Hkv,
                     const uint8_t* kcodes, const uint8_t* kscales, float s_tk,
                     const uint8_t* vcodes, const uint8_t* vscales, float s_tv,
                     int prefix, int causal, int total_len, double scale,
                     double* work, float* out) {
  size_t n = (size_t)total_len * Hkv;
  float* kh = (float*)malloc((n ? n : 1) * ORC_D * sizeof(float));
  float* vh = (float*)malloc((n ? n : 1) * ORC_D * sizeof(float));
  if (!kh || !vh) { free(kh); free(vh); return -1; }
  orc_dequant_rows(kcodes, kscales, n, s_tk, kh);
  orc_dequant_rows(vcodes, vscales, n, s_tv, vh);
  for (int r = 0; r < nrows; ++r) {
    int L = causal ? prefix + rows[r] + 1 : total_len;
    if (L > total_len) L = total_len;
    attend_dequantized(q + (size_t)r * Hq * ORC_D, Hq, Hkv, kh, vh, L, scale, work,
                       out + (size_t)r * Hq * ORC_D);
  }
  free(kh);
  free(vh);
  return 0;
}
