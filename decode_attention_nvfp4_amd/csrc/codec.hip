// codec.hip -- quantize-on-append, dequantize, and tensor amax kernels.
//
// Quantize-on-append follows the flow of "NVIDIA解説: NVFP4 KV Cacheで長コン
// テキストLLM推論を最適化" (section 量子化・逆量子化フロー): each new K/V row is
// quantized in 16-element blocks and written to the NVFP4 cache.  The block
// scale and element rounding rules are stated in include/nvfp4kv.h.
//
// Thread mapping: 16 lanes own one (token, head) row of 128 elements; lane i
// owns elements 8i..8i+7 (half of block i/2) and exchanges its half-block
// amax with lane i^1.  A 256-thread workgroup handles 16 rows.
#include "common.h"
#include "internal.h"

namespace nvfp4 {

// A lane's 8 input elements (half of one block) as raw bits: 32 bytes of
// FP32 or 16 bytes of BF16.  Converted to float only when quantized, so that
// the loads of a row can all be in flight together.  The input is read once
// (non-temporal hint).
struct Raw8 {
  uint4 a, b;
};

template <bool F32IN>
__device__ __forceinline__ Raw8 load_raw8(const void* base, size_t row, int lane16) {
  Raw8 r;
  if (F32IN) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + row * kD + lane16 * 8);
    r.a = load_once16(p);
    r.b = load_once16(p + 1);
  } else {
    r.a = load_once16(static_cast<const uint16_t*>(base) + row * kD + lane16 * 8);
    r.b = uint4{0u, 0u, 0u, 0u};
  }
  return r;
}

template <bool F32IN>
__device__ __forceinline__ void unpack8(const Raw8& r, float x[8]) {
  if (F32IN) {
    x[0] = __uint_as_float(r.a.x); x[1] = __uint_as_float(r.a.y);
    x[2] = __uint_as_float(r.a.z); x[3] = __uint_as_float(r.a.w);
    x[4] = __uint_as_float(r.b.x); x[5] = __uint_as_float(r.b.y);
    x[6] = __uint_as_float(r.b.z); x[7] = __uint_as_float(r.b.w);
  } else {
    x[0] = bf16_lo(r.a.x); x[1] = bf16_hi(r.a.x); x[2] = bf16_lo(r.a.y); x[3] = bf16_hi(r.a.y);
    x[4] = bf16_lo(r.a.z); x[5] = bf16_hi(r.a.z); x[6] = bf16_lo(r.a.w); x[7] = bf16_hi(r.a.w);
  }
}

// ------------------------------------------------ MSE-searched block scale
//
// The block scale may instead be searched ("NVIDIA解説: NVFP4 KV Cacheで長コン
// テキストLLM推論を最適化", section E2M1 + 2レベルスケーリング, describes the
// NVFP4 block scale as chosen for least squared error): the E4M3 codes within
// kMseRadius of the amax/6 code (code 0 excluded) are tried and the one whose
// element codes give the smallest squared error of the block is kept.  The
// error of a candidate is summed in double over the block's elements in
// order, every operation rounded once (no fused multiply-add); ties go to
// the candidate nearest the amax/6 code, then to the smaller code.  A zero
// amax/6 code stays zero.
constexpr int kMseRadius = 8;

// Squared error of the 16-element block xb under block-scale code c.  The
// product e2m1 * s_block * s_t is exact in double (3 + 4 + 24 significant
// bits); |x| - |p| has the magnitude of x - p because an element's code
// carries the sign of x.
__device__ __forceinline__ double block_sq_error(const float xb[16], uint32_t c, float s_t) {
#pragma clang fp contract(off)
  const uint32_t w0 = encode8(xb, c, s_t), w1 = encode8(xb + 8, c, s_t);
  const double step = (double)e4m3_to_float(c) * (double)s_t;
  double sum = 0.0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t m = ((e < 8 ? w0 >> (4 * e) : w1 >> (4 * (e - 8)))) & 7u;
    const double g = m < 4u ? 0.5 * (double)m : (m == 7u ? 6.0 : (double)m - 2.0);
    const double d = (double)fabsf(xb[e]) - g * step;
    sum = sum + d * d;
  }
  return sum;
}

// An FP32 estimate of block_sq_error(xb, c, s_t) with a bound on its
// distance from it: [*lo, *hi] holds the double criterion.  Element codes
// come from the hardware conversion of |x| * rcp(d) (d = s_block * s_t in
// FP32), so a code may differ from the exact one only when |x| / d lies
// within 2^-21 of an E2M1 midpoint, which moves that element's squared
// error by at most 24 * 2^-21 * d^2; the FP32 arithmetic adds at most
// 2^-17 d^2 + 2^-18.6 * (the sum) over the 16 elements.  The bound used,
// 2^-11 d^2 + 2^-17 * sum, covers both with a margin.  Returns false where
// the estimate does not apply (d outside [2^-40, 2^40], or a non-finite
// sum), and the candidate is then evaluated exactly.
__device__ __forceinline__ bool block_sq_error_est(const float xb[16], uint32_t c, float s_t, float* lo,
                                                   float* hi) {
  const float d = e4m3_to_float(c) * s_t;
  if (!(d >= 0x1p-40f && d <= 0x1p40f)) return false;
  const float y = __builtin_amdgcn_rcpf(d);
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const float* v = xb + 8 * q;
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, fabsf(v[0]) * y, fabsf(v[1]) * y, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, fabsf(v[2]) * y, fabsf(v[3]) * y, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, fabsf(v[4]) * y, fabsf(v[5]) * y, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, fabsf(v[6]) * y, fabsf(v[7]) * y, 1.0f, 3);
    floatx2 g[4];
    g[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    g[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    g[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    g[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float r = __builtin_fmaf(-g[e >> 1][e & 1], d, fabsf(v[e]));
      acc = __builtin_fmaf(r, r, acc);
    }
  }
  if (!__builtin_isfinite(acc)) return false;
  const float tol = 0x1p-11f * d * d + 0x1p-17f * acc;
  *lo = acc - tol;
  *hi = acc + tol;
  return true;
}

// A lane's 8 packed codes (half of a block held by a lane pair) under the
// searched block scale, *sb the scale code.  The lane pair swaps halves so
// both hold the block's 16 elements in order; search position k = 0 is
// the amax/6 code, k = 2j - 1 and 2j its neighbours at distance j below and
// above.  The even lane tries the even positions, the odd lane the odd ones,
// and the pair keeps the smallest (error, position); an unusable position
// (code outside 1..126) is skipped.  Non-finite errors (non-finite inputs)
// compare as ties, so the amax/6 code is kept, as in a plain ordered scan.
// The exact error is computed only for candidates whose FP32 interval
// (block_sq_error_est) reaches below the smallest upper end of the pair's
// intervals: any other candidate is strictly worse than the candidate with
// that upper end, which is always evaluated, so the choice is unchanged.
__device__ __forceinline__ uint32_t quantize_half_block_mse(const float x[8], float s_t, float inv6,
                                                            double six_st, uint32_t* sb) {
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(x[j]));
  a = fmaxf(a, __shfl_xor(a, 1));
  const int c0 = (int)block_scale_code_fast(a, inv6, six_st);
  const int odd = (int)(threadIdx.x & 1);
  float xb[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float o = __shfl_xor(x[j], 1);
    xb[j] = odd ? o : x[j];
    xb[8 + j] = odd ? x[j] : o;
  }
  uint32_t code = 0u;
  if (c0 != 0) {
    // a lane may have no usable position (the odd lane when c0 is 1): its
    // (inf, past-the-end) then loses to any of its partner's
    constexpr int kMine = kMseRadius + 1;       // positions of one lane
    float lo[kMine];
    bool est[kMine];
    float min_hi = __builtin_huge_valf();
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      const int k = odd + 2 * i;
      const int c = k == 0 ? c0 : ((k & 1) ? c0 - (k + 1) / 2 : c0 + k / 2);
      est[i] = false;
      lo[i] = 0.0f;
      if (k > 2 * kMseRadius || c < 1 || c > 126) continue;
      float hi;
      est[i] = block_sq_error_est(xb, (uint32_t)c, s_t, &lo[i], &hi);
      if (est[i]) min_hi = fminf(min_hi, hi);
    }
    min_hi = fminf(min_hi, __shfl_xor(min_hi, 1));
    // the lane's candidates still in the running, as a bit mask; each
    // pass evaluates one per lane, so the wave makes as many passes as its
    // lanes have survivors at most (usually one), not one per position
    uint32_t mask = 0u;
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      const int k = odd + 2 * i;
      const int c = k == 0 ? c0 : ((k & 1) ? c0 - (k + 1) / 2 : c0 + k / 2);
      if (k > 2 * kMseRadius || c < 1 || c > 126) continue;
      if (est[i] && lo[i] > min_hi) continue;   // strictly worse than another candidate
      mask |= 1u << i;
    }
    double best = __builtin_huge_val();
    int best_k = 2 * kMseRadius + 1;
    while (__any(mask != 0u)) {
      if (mask != 0u) {
        const int i = __builtin_ctz(mask);      // increasing position order
        mask &= mask - 1u;
        const int k = odd + 2 * i;
        const int c = k == 0 ? c0 : ((k & 1) ? c0 - (k + 1) / 2 : c0 + k / 2);
        const double err = block_sq_error(xb, (uint32_t)c, s_t);
        if (best_k > 2 * kMseRadius || err < best) {
          best = err;
          best_k = k;
        }
      }
    }
    const double o_best = __shfl_xor(best, 1);
    const int o_k = __shfl_xor(best_k, 1);
    if (o_best < best || (!(best < o_best) && o_k < best_k)) best_k = o_k;
    code = (uint32_t)(best_k == 0 ? c0 : ((best_k & 1) ? c0 - (best_k + 1) / 2 : c0 + best_k / 2));
  }
  *sb = code;
  return encode8(x, code, s_t);
}

// ------------------------------------------------------------ MXFP4 blocks
//
// MXFP4 (the OCP format set against NVFP4 in "NVIDIA解説: NVFP4 KV Cacheで
// 長コンテキストLLM推論を最適化", section MXFP4との比較): 32-element blocks
// (four lanes of a row), E8M0 scale 2^e with e = floor(log2(amax)) - 2
// clamped to [-127, 127] (-127 for a zero block), elements the E2M1 value
// nearest to |x| / 2^e, ties to the even code, clamped to 6.

// floor(log2(a)) of a finite a > 0 from its bits, subnormals included.
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t b = __float_as_uint(a);
  const int field = (int)(b >> 23);
  if (field > 0) return field - 127;
  return (31 - (int)__builtin_clz(b & 0x7FFFFFu)) - 149;
}

// The lane's 8 packed codes; *sb gets the block's E8M0 byte.  |x| * 2^-e is
// exact (a power-of-two scaling; a product below the FP32 normal range is
// far below the first threshold), so the thresholds decide exactly.
__device__ __forceinline__ uint32_t quantize_half_block_mx(const float x[8], uint32_t* sb) {
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(x[j]));
  a = fmaxf(a, __shfl_xor(a, 1));
  a = fmaxf(a, __shfl_xor(a, 2));
  int e = a > 0.0f ? floor_log2(a) - 2 : -127;
  e = max(-127, min(127, e));                 // a finite amax gives e <= 125
  *sb = (uint32_t)(e + 127);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, a normal FP32
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float r = fabsf(x[j]) * inv;
    uint32_t m = 0;
    m += r > 0.25f;
    m += r >= 0.75f;
    m += r > 1.25f;
    m += r >= 1.75f;
    m += r > 2.5f;
    m += r >= 3.5f;
    m += r > 5.0f;
    w |= (m | ((__float_as_uint(x[j]) >> 31) << 3)) << (4 * j);
  }
  return w;
}

// The V bytes of a token pair from the two tokens' eight codes each (element
// e in bits 4e..4e+3 of a for the even token, of b for the odd one): byte e
// holds element e of a in its low nibble and of b in its high nibble,
// elements 0..3 in .x and 4..7 in .y.  The even elements 0, 2, 4, 6 and the
// odd ones 1, 3, 5, 7 are paired up within bytes with masks, then two byte
// permutes put the bytes in element order.  (b = 0 gives the even token's
// nibbles alone, a = 0 the odd token's.)
__device__ __forceinline__ uint2 pair_bytes(uint32_t a, uint32_t b) {
  const uint32_t even = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);   // bytes: elements 0, 2, 4, 6
  const uint32_t odd = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);    // bytes: elements 1, 3, 5, 7
  return make_uint2(__builtin_amdgcn_perm(odd, even, 0x05010400u), __builtin_amdgcn_perm(odd, even, 0x07030602u));
}

// The MSE-searched and MXFP4 appends (a block spans a lane pair or quad,
// which exchange the block's amax or candidates): workgroup = 16 consecutive
// tokens of the call x one KV head (grid.y).  The V codes of a token pair
// (2i, 2i+1) share bytes: when both tokens of a pair
// sit in the same workgroup (consecutive rows, same sequence, positions 2i
// and 2i+1) the even row writes the whole bytes; a token whose partner is
// elsewhere updates its nibbles with atomic AND / OR, which commute with the
// partner's own update of the other nibbles.
template <bool F32IN, int MODE>
__global__ void __launch_bounds__(256) append_kernel(AppendArgs p) {
  const int lane16 = threadIdx.x & 15, r = threadIdx.x >> 4;
  const int tok = blockIdx.x * 16 + r;
  const int h = blockIdx.y;
  const bool valid = tok < p.n_tok;
  __shared__ int s_seq[16], s_pos[16];
  __shared__ uint32_t s_vw[16][16];
  // all of the row's loads go out first (position, then the K and V data),
  // so their latencies overlap; the page-table lookup waits only for the
  // position, and the quantization only for the data
  int seq = -1, pos = 0;
  Raw8 rk = {}, rv = {};
  const size_t row = (size_t)tok * p.hkv + h;
  if (valid) {
    seq = p.tok_seq[tok];
    pos = p.tok_pos[tok];
    rk = load_raw8<F32IN>(p.k_new, row, lane16);
    rv = load_raw8<F32IN>(p.v_new, row, lane16);
  }
  if (lane16 == 0) {
    s_seq[r] = seq;
    s_pos[r] = pos;
  }
  size_t slab = 0;
  int slot = 0;
  uint32_t vw = 0, vsb = 0;
  if (valid) {
    const int page = clamp_page(p.page_table[(size_t)seq * p.max_pages + pos / kPage], p.num_pages);
    slot = pos % kPage;
    uint32_t ksb;
    float x[8];
    unpack8<F32IN>(rk, x);
    uint32_t kw;
    if constexpr (MODE == kAppendMse) {
      kw = quantize_half_block_mse(x, p.k_scale, p.k_inv6, p.k_six_st, &ksb);
      unpack8<F32IN>(rv, x);
      vw = quantize_half_block_mse(x, p.v_scale, p.v_inv6, p.v_six_st, &vsb);
    } else {
      static_assert(MODE == kAppendMx, "the amax/6 append is append_block_kernel");
      kw = quantize_half_block_mx(x, &ksb);
      unpack8<F32IN>(rv, x);
      vw = quantize_half_block_mx(x, &vsb);
    }
    slab = (size_t)page * p.hkv + h;
    // K: token-major codes [16][64 B]; the V codes follow below
    *reinterpret_cast<uint32_t*>(p.k_codes + slab * kSlab + slot * 64 + lane16 * 4) = kw;
    if constexpr (MODE == kAppendMx) {
      // K scales [token 16][block 4], V scales [block 4][token 16]
      if ((lane16 & 3) == 0) {
        p.k_scales[slab * kMxScaleSlab + slot * kMxNBlk + (lane16 >> 2)] = (uint8_t)ksb;
        p.v_scales[slab * kMxScaleSlab + (lane16 >> 2) * kPage + slot] = (uint8_t)vsb;
      }
    } else {
      // K scales [token 16][block 8], V scales [block 8][token 16]
      if ((lane16 & 1) == 0) {
        p.k_scales[slab * kScaleSlab + slot * kNBlk + (lane16 >> 1)] = (uint8_t)ksb;
        p.v_scales[slab * kScaleSlab + (lane16 >> 1) * kPage + slot] = (uint8_t)vsb;
      }
    }
  }
  s_vw[r][lane16] = vw;
  __syncthreads();
  if (!valid) return;
  const int odd = pos & 1;
  const int pr = odd ? r - 1 : r + 1;           // the partner's row, if it is here
  const bool paired = pr >= 0 && pr < 16 && s_seq[pr] == seq && s_pos[pr] == (pos ^ 1);
  uint32_t* dst = reinterpret_cast<uint32_t*>(p.v_codes + slab * kSlab + (slot >> 2) * 256 + lane16 * 16 +
                                              ((slot >> 1) & 1) * 8);
  if (paired) {
    if (odd) return;                            // written by the even row
    *reinterpret_cast<uint2*>(dst) = pair_bytes(vw, s_vw[pr][lane16]);
  } else {
    // the partner's nibbles kept (one 64-bit clear and set, 8-byte aligned)
    const unsigned long long keep = odd ? 0x0F0F0F0F0F0F0F0Full : 0xF0F0F0F0F0F0F0F0ull;
    const uint2 own = odd ? pair_bytes(0u, vw) : pair_bytes(vw, 0u);
    unsigned long long* d64 = reinterpret_cast<unsigned long long*>(dst);
    atomicAnd(d64, keep);
    atomicOr(d64, (unsigned long long)own.x | ((unsigned long long)own.y << 32));
  }
}

// The amax/6 append with one lane per 16-element block: workgroup = ROWS
// consecutive tokens of the call x one KV head.  A lane holds its whole
// block, so the block's amax, scale code and reciprocal are computed once
// (the lane-pair layout above computes them in both lanes and exchanges the
// amax); the element rounding is encode8's, so the codes are those of
// append_kernel.  V pairs as in append_kernel.  SPLIT = false: 8 lanes per
// token, each encoding K block j and V block j (bulk appends, where the
// chip is full and fewer instructions per block count).  SPLIT = true: 16
// lanes per token, lanes 0-7 take the K blocks and 8-15 the V blocks, half
// the serial work per lane for appends too small to fill the chip.
template <bool F32IN, bool SPLIT, int ROWS>
__global__ void __launch_bounds__(ROWS * (SPLIT ? 16 : 8)) append_block_kernel(AppendArgs p) {
  constexpr int kLanes = SPLIT ? 16 : 8;
  static_assert(ROWS * kLanes <= 1024, "one workgroup holds ROWS tokens");
  const int j = threadIdx.x & 7, r = threadIdx.x / kLanes;  // block j of row r
  const bool vlane = SPLIT && (threadIdx.x & 8);            // SPLIT: a V block
  const int tok = blockIdx.x * ROWS + r;
  const int h = blockIdx.y;
  const bool valid = tok < p.n_tok;
  __shared__ int s_seq[ROWS], s_pos[ROWS];
  __shared__ uint2 s_vw[ROWS][8];
  // rows past the call's end load the last row (their results are dropped)
  const int ltok = valid ? tok : p.n_tok - 1;
  const size_t row = (size_t)ltok * p.hkv + h;
  const int seq = valid ? p.tok_seq[ltok] : -1;
  const int pos = p.tok_pos[ltok];
  const void* src0 = vlane ? p.v_new : p.k_new;
  const Raw8 rk0 = load_raw8<F32IN>(src0, row, 2 * j), rk1 = load_raw8<F32IN>(src0, row, 2 * j + 1);
  Raw8 rv0, rv1;
  if constexpr (!SPLIT) {
    rv0 = load_raw8<F32IN>(p.v_new, row, 2 * j);
    rv1 = load_raw8<F32IN>(p.v_new, row, 2 * j + 1);
  }
  if (j == 0 && !vlane) {
    s_seq[r] = seq;
    s_pos[r] = pos;
  }
  // the block's codes (elements 0-7, 8-15) and scale code.  The amax is
  // the largest magnitude's bit pattern as an integer (the same value for
  // finite elements; bf16 halves compared two at a time)
  auto quantize = [&](const Raw8& r0, const Raw8& r1, float s_t, float inv6, double six_st, uint32_t* sb) {
    float a;
    if constexpr (F32IN) {
      uint32_t m = 0u;
      const uint4 w[4] = {r0.a, r0.b, r1.a, r1.b};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        m = max(m, max(max(w[i].x & 0x7FFFFFFFu, w[i].y & 0x7FFFFFFFu), max(w[i].z & 0x7FFFFFFFu, w[i].w & 0x7FFFFFFFu)));
      a = __uint_as_float(m);
    } else {
      typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
      const uint32_t w[8] = {r0.a.x, r0.a.y, r0.a.z, r0.a.w, r1.a.x, r1.a.y, r1.a.z, r1.a.w};
      u16x2 m = {0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
      a = __uint_as_float((uint32_t)max(m.x, m.y) << 16);
    }
    float x0[8], x1[8];
    unpack8<F32IN>(r0, x0);
    unpack8<F32IN>(r1, x1);
    const uint32_t code = block_scale_code_fast(a, inv6, six_st);
    *sb = code;
    return encode16(x0, x1, code, s_t);
  };
  size_t slab = 0;
  int slot = 0;
  uint2 vw = make_uint2(0u, 0u);
  if (valid) {
    const int page = clamp_page(p.page_table[(size_t)seq * p.max_pages + pos / kPage], p.num_pages);
    slot = pos % kPage;
    slab = (size_t)page * p.hkv + h;
    // K: token-major codes [16][64 B], block j at byte 8j; scales K [token
    // 16][block 8], V [block 8][token 16]
    uint32_t ksb, vsb;
    uint2 kw;
    if constexpr (SPLIT) {
      // one quantize with per-lane parameters: K and V lanes share a wave,
      // so a branch per plane would run both sides one after the other
      const float s_t = vlane ? p.v_scale : p.k_scale, inv6 = vlane ? p.v_inv6 : p.k_inv6;
      const double six_st = vlane ? p.v_six_st : p.k_six_st;
      kw = quantize(rk0, rk1, s_t, inv6, six_st, &ksb);
      vw = kw;
      vsb = ksb;
    } else {
      kw = quantize(rk0, rk1, p.k_scale, p.k_inv6, p.k_six_st, &ksb);
      vw = quantize(rv0, rv1, p.v_scale, p.v_inv6, p.v_six_st, &vsb);
    }
    if (!vlane) {
      *reinterpret_cast<uint2*>(p.k_codes + slab * kSlab + slot * 64 + j * 8) = kw;
      p.k_scales[slab * kScaleSlab + slot * kNBlk + j] = (uint8_t)ksb;
    }
    if (!SPLIT || vlane) p.v_scales[slab * kScaleSlab + j * kPage + slot] = (uint8_t)vsb;
  }
  if (!SPLIT || vlane) s_vw[r][j] = vw;
  __syncthreads();
  if (!valid || (SPLIT && !vlane)) return;
  const int odd = pos & 1;
  const int pr = odd ? r - 1 : r + 1;           // the partner's row, if it is here
  const bool paired = pr >= 0 && pr < ROWS && s_seq[pr] == seq && s_pos[pr] == (pos ^ 1);
  // V: the block's element groups 2j and 2j+1 (8 elements each, 16 bytes apart)
  uint32_t* dst = reinterpret_cast<uint32_t*>(p.v_codes + slab * kSlab + (slot >> 2) * 256 + j * 32 +
                                              ((slot >> 1) & 1) * 8);
  if (paired) {
    if (odd) return;                            // written by the even row
    const uint2 pv = s_vw[pr][j];
    *reinterpret_cast<uint2*>(dst) = pair_bytes(vw.x, pv.x);
    *reinterpret_cast<uint2*>(dst + 4) = pair_bytes(vw.y, pv.y);
  } else {
    // the partner's nibbles kept: one 64-bit clear and one 64-bit set per
    // 8-byte group (8-byte aligned), half the atomics of 32-bit words
    const unsigned long long keep = odd ? 0x0F0F0F0F0F0F0F0Full : 0xF0F0F0F0F0F0F0F0ull;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint32_t w = g ? vw.y : vw.x;
      const uint2 own = odd ? pair_bytes(0u, w) : pair_bytes(w, 0u);
      unsigned long long* d64 = reinterpret_cast<unsigned long long*>(dst + 4 * g);
      atomicAnd(d64, keep);
      atomicOr(d64, (unsigned long long)own.x | ((unsigned long long)own.y << 32));
    }
  }
}

// ------------------------------------------------ comparison formats

// Append to an FP8 or BF16 cache.  16 lanes per (token, head) row, lane g
// takes elements 8g .. 8g+7 of K and of V.  FP8: the E4M3 code of the FP32
// quotient x / s_t (IEEE division), clamped to +-448 first so that the
// hardware's nearest-even conversion saturates like the format's rule.
// BF16: nearest even (input bf16 is copied).  K rows are contiguous; the V
// element d of token t sits at ((t/4) * 128 + d) * 4 + t%4 (elements), so a
// row's V goes out as single-element stores.
template <bool F32IN>
__global__ void __launch_bounds__(256) cmp_append_kernel(CmpAppendArgs a) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid >> 4;
  const int g = (int)(gid & 15);
  if (row >= (long long)a.n_tok * a.hkv) return;
  const int tok = (int)(row / a.hkv), head = (int)(row % a.hkv);
  const Raw8 rk = load_raw8<F32IN>(a.k_new, (size_t)row, g);
  const Raw8 rv = load_raw8<F32IN>(a.v_new, (size_t)row, g);
  const int seq = a.tok_seq[tok], pos = a.tok_pos[tok];
  const int page = clamp_page(a.page_table[(size_t)seq * a.max_pages + pos / kPage], a.num_pages);
  const int t = pos % kPage;
  const size_t slab = (size_t)page * a.hkv + head;
  const size_t kelem = slab * kPage * kD + (size_t)t * kD + 8 * g;              // K element index
  const size_t velem = slab * kPage * kD + ((size_t)(t >> 2) * kD + 8 * g) * 4 + (t & 3);
  float k[8], v[8];
  unpack8<F32IN>(rk, k);
  unpack8<F32IN>(rv, v);
  if (a.fmt == kFmtFp8) {
    auto q = [](float x, float s) { return fminf(fmaxf(x / s, -448.0f), 448.0f); };
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q(k[4 * h], a.k_scale), q(k[4 * h + 1], a.k_scale), 0, false);
      w[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q(k[4 * h + 2], a.k_scale), q(k[4 * h + 3], a.k_scale), lo, true);
    }
    *reinterpret_cast<uint2*>(a.k + kelem) = uint2{w[0], w[1]};
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t b = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q(v[e], a.v_scale), q(v[e + 1], a.v_scale), 0, false);
      a.v[velem + 4 * e] = (uint8_t)(b & 0xFFu);
      a.v[velem + 4 * (e + 1)] = (uint8_t)((b >> 8) & 0xFFu);
    }
  } else {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = ((uint32_t)(uint16_t)bf16_bits(k[2 * j])) | ((uint32_t)(uint16_t)bf16_bits(k[2 * j + 1]) << 16);
    *reinterpret_cast<uint4*>(a.k + 2 * kelem) = uint4{w[0], w[1], w[2], w[3]};
    uint16_t* vp = reinterpret_cast<uint16_t*>(a.v);
#pragma unroll
    for (int e = 0; e < 8; ++e) vp[velem + 4 * e] = (uint16_t)bf16_bits(v[e]);
  }
}

hipError_t launch_cmp_append(const CmpAppendArgs& a, bool f32, hipStream_t s) {
  const long long threads = (long long)a.n_tok * a.hkv * 16;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (f32) cmp_append_kernel<true><<<blocks, 256, 0, s>>>(a);
  else cmp_append_kernel<false><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int MODE>
static void launch_append_mode(const AppendArgs& a, bool f32, dim3 grid, hipStream_t s) {
  if (f32) append_kernel<true, MODE><<<grid, 256, 0, s>>>(a);
  else append_kernel<false, MODE><<<grid, 256, 0, s>>>(a);
}

template <bool SPLIT, int ROWS>
static void launch_block(const AppendArgs& a, bool f32, hipStream_t s) {
  const dim3 grid((unsigned)((a.n_tok + ROWS - 1) / ROWS), (unsigned)a.hkv);
  constexpr unsigned threads = ROWS * (SPLIT ? 16 : 8);
  if (f32) append_block_kernel<true, SPLIT, ROWS><<<grid, threads, 0, s>>>(a);
  else append_block_kernel<false, SPLIT, ROWS><<<grid, threads, 0, s>>>(a);
}

hipError_t launch_append(const AppendArgs& a, bool f32, int mode, hipStream_t s) {
  const dim3 grid((unsigned)((a.n_tok + 15) / 16), (unsigned)a.hkv);
  if (mode == kAppendMse) launch_append_mode<kAppendMse>(a, f32, grid, s);
  else if (mode == kAppendMx) launch_append_mode<kAppendMx>(a, f32, grid, s);
  else {
    // amax/6 by (token, head) rows: from 32768 rows (1024 workgroups of 32
    // tokens) the chip is full and the 8-lane layout's fewer instructions
    // per block win; below, the call is latency bound and the split layout
    // halves each lane's serial work, with 16 tokens per workgroup down to
    // 4096 rows (256 workgroups) and single-wave workgroups of 4 tokens below.
    // From 262144 rows (1024 workgroups of 128 tokens) the windows grow to
    // 128 tokens: a window whose ends fall inside pages writes partial lines
    // of those pages' planes, which the neighbouring window writes again, and
    // wider windows have fewer ends (configuration 4's bulk append, sequences
    // back to back: 0.855 GB written at 32 tokens, 0.728 GB at 128, against
    // 0.685 GB of codes and scales; 1.5-2 % faster, measured on MI355X)
    const long long rows = (long long)a.n_tok * a.hkv;
    if (rows >= 262144) launch_block<false, 128>(a, f32, s);
    else if (rows >= 32768) launch_block<false, 32>(a, f32, s);
    else if (rows >= 4096) launch_block<true, 16>(a, f32, s);
    else launch_block<true, 4>(a, f32, s);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- dequantize

template <bool F32OUT>
__global__ void __launch_bounds__(256) dequant_kernel(DequantArgs p) {
  const int lane16 = threadIdx.x & 15;
  const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= (size_t)p.n * p.hkv) return;
  const int i = (int)(row / p.hkv);
  const int h = (int)(row - (size_t)i * p.hkv);
  const int pos = p.pos0 + i;
  const int page = clamp_page(p.page_table_row[pos / kPage], p.num_pages);
  const int slot = pos % kPage;
  const size_t slab = (size_t)page * p.hkv + h;
  for (int kv = 0; kv < 2; ++kv) {
    void* out = kv ? p.v_out : p.k_out;
    if (!out) continue;
    uint32_t w, sb;
    float st;
    if (kv == 0) {
      w = *reinterpret_cast<const uint32_t*>(p.k_codes + slab * kSlab + slot * 64 + lane16 * 4);
      sb = p.k_scales[slab * kScaleSlab + slot * kNBlk + (lane16 >> 1)];
      st = p.k_scale;
    } else {
      // the nibble of this token in each of the 8 bytes of elements 8 lane16..
      const uint2 b = *reinterpret_cast<const uint2*>(p.v_codes + slab * kSlab + (slot >> 2) * 256 +
                                                      lane16 * 16 + ((slot >> 1) & 1) * 8);
      const int sh = 4 * (slot & 1);
      w = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w |= ((b.x >> (8 * e + sh)) & 15u) << (4 * e);
        w |= ((b.y >> (8 * e + sh)) & 15u) << (4 * (e + 4));
      }
      sb = p.v_scales[slab * kScaleSlab + (lane16 >> 1) * kPage + slot];
      st = p.v_scale;
    }
    float sbf = e4m3_to_float(sb);
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t c = (w >> (4 * j)) & 15u;
      // E2M1 magnitude from its bit fields: exponent bias 1, field 0 subnormal
      uint32_t e = (c >> 1) & 3u, m = c & 1u;
      float mag = e == 0u ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << (e - 1u));
      float v = (mag * sbf) * st;            // mag * sbf is exact; one rounding
      y[j] = (c & 8u) ? -v : v;
    }
    if (F32OUT) {
      float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + row * kD + lane16 * 8);
      o[0] = make_float4(y[0], y[1], y[2], y[3]);
      o[1] = make_float4(y[4], y[5], y[6], y[7]);
    } else {
      uint4 o;
      o.x = float_to_bf16_bits(y[0]) | (float_to_bf16_bits(y[1]) << 16);
      o.y = float_to_bf16_bits(y[2]) | (float_to_bf16_bits(y[3]) << 16);
      o.z = float_to_bf16_bits(y[4]) | (float_to_bf16_bits(y[5]) << 16);
      o.w = float_to_bf16_bits(y[6]) | (float_to_bf16_bits(y[7]) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + row * kD + lane16 * 8) = o;
    }
  }
}

hipError_t launch_dequant(const DequantArgs& a, bool f32, hipStream_t s) {
  size_t rows = (size_t)a.n * a.hkv;
  unsigned grid = (unsigned)((rows + 15) / 16);
  if (f32) dequant_kernel<true><<<grid, 256, 0, s>>>(a);
  else dequant_kernel<false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- abs max

__global__ void zero_float_kernel(float* p) { *p = 0.0f; }

// Wave max, then one atomic per workgroup; non-negative floats order like
// their bit patterns, so the maximum is taken on |x|'s bits.
__device__ __forceinline__ void absmax_publish(uint32_t m, float* out) {
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    atomicMax(reinterpret_cast<unsigned int*>(out), m);
  }
}

// |x| bits of one element: FP32 without its sign, or BF16 widened to FP32.
template <bool F32IN>
__device__ __forceinline__ uint32_t abs_bits(const void* x, int64_t i) {
  return F32IN ? (static_cast<const uint32_t*>(x)[i] & 0x7FFFFFFFu)
               : ((uint32_t)(static_cast<const uint16_t*>(x)[i] & 0x7FFFu) << 16);
}

// Any alignment: one element per thread per step.
template <bool F32IN>
__global__ void __launch_bounds__(256) absmax_kernel(const void* x, int64_t n, float* out) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    m = max(m, abs_bits<F32IN>(x, i));
  absmax_publish(m, out);
}

// 16-byte aligned input: 16 bytes per thread per step (a streaming read),
// then the elements past the last whole 16 bytes.
template <bool F32IN>
__global__ void __launch_bounds__(256) absmax_vec_kernel(const void* x, int64_t n, float* out) {
  constexpr int kPer = F32IN ? 4 : 8;
  const int64_t nvec = n / kPer;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const u32x4* v = static_cast<const u32x4*>(x);
  uint32_t m = 0;
  for (int64_t i = gid; i < nvec; i += stride) {
    const u32x4 w = __builtin_nontemporal_load(v + i);
    if (F32IN) {
      m = max(m, max(max(w.x & 0x7FFFFFFFu, w.y & 0x7FFFFFFFu), max(w.z & 0x7FFFFFFFu, w.w & 0x7FFFFFFFu)));
    } else {
      const uint32_t a = max(max(w.x & 0x7FFFu, (w.x >> 16) & 0x7FFFu), max(w.y & 0x7FFFu, (w.y >> 16) & 0x7FFFu));
      const uint32_t b = max(max(w.z & 0x7FFFu, (w.z >> 16) & 0x7FFFu), max(w.w & 0x7FFFu, (w.w >> 16) & 0x7FFFu));
      m = max(m, max(a, b) << 16);
    }
  }
  for (int64_t i = nvec * kPer + gid; i < n; i += stride) m = max(m, abs_bits<F32IN>(x, i));
  absmax_publish(m, out);
}

hipError_t launch_absmax(const void* x, bool f32, int64_t n, float* out, hipStream_t s) {
  zero_float_kernel<<<1, 1, 0, s>>>(out);
  if (n > 0) {
    const bool vec = (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
    const int64_t per = vec ? (f32 ? 4 : 8) : 1;
    int64_t blocks = (n / per + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) blocks = 1;
    if (vec) {
      if (f32) absmax_vec_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(x, n, out);
      else absmax_vec_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(x, n, out);
    } else {
      if (f32) absmax_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(x, n, out);
      else absmax_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(x, n, out);
    }
  }
  return hipGetLastError();
}

}  // namespace nvfp4
