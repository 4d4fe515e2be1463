// prefill.hip -- chunked-prefill attention over the NVFP4 cache with FP8
// MFMA operands and FP32 accumulation.
//
// Flow ("NVIDIA解説: NVFP4 KV Cacheで長コンテキストLLM推論を最適化", section
// 量子化・逆量子化フロー): the NVFP4 cache is dequantized to FP8 and the
// attention and context products run on FP8 operands.  Here the expansion is
// a separate pass over the sequence's cache (expand_kernel) into an FP8
// workspace laid out as MFMA operands; the attention kernel (fa_kernel) then
// streams 64-key tiles through LDS.  Each K/V element is expanded once
// instead of once per query tile, which keeps the attention loop's VALU
// budget for the softmax.
//
// FP8 values: K~ = E4M3(e2m1 * s_block / 8) (<= 336, no overflow);
// Q = E4M3(q * 2^shift_row) with |q| * 2^shift < 256 per row;
// P = E4M3(p * 256) with p <= 2^0.5 (lazy max, below).  The scores and the
// output take the factors back in FP32.
//
// fa_kernel: a 256-thread workgroup owns 128 consecutive (query, head) rows of
// one KV head (row r = query r / G, head r % G), 32 per wave.  Per 64-key
// tile and wave:
//   S^T[key][row] = K~ Q^T: two key blocks x two 32x32x64 FP8 MFMAs (the
//     contraction over d is permuted identically in K~ and Q: lane half h
//     holds d in [64h, 64h+64)).
//   softmax over keys: each lane holds 32 keys of one row, the other 32 sit
//     in the lane 32 away.
//   O^T[d][row] += V~^T P^T: four 32x32x64 FP8 MFMAs; P^T is the S^T
//     accumulator converted in place, so the key order inside a tile follows
//     the accumulator layout (kappa below), which the V~ workspace matches.
#include "common.h"
#include "internal.h"

namespace nvfp4 {

constexpr int kTile = kPrefillTile;      // 64 keys
constexpr int kKRow = 144;                // LDS bytes per K~ row (128 + pad)
constexpr int kVRow = 80;                 // LDS bytes per V~^T row (64 + pad)

// Position of key kk (0..63) of a tile inside a V~^T row: lane half h and
// element j of the P^T operand.  The S^T accumulator of key block kb gives
// lane (n, h) element r the key kb*32 + 8(r/4) + 4h + r%4, and P^T element
// j = 16 kb + r.
__device__ __forceinline__ int vt_pos(int kk) {
  const int kb = kk >> 5, rem = kk & 31;
  const int h = (rem >> 2) & 1;
  const int j = 16 * kb + (rem >> 3) * 4 + (rem & 3);
  return h * 32 + j;
}

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float mag = e == 0u ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << (e - 1u));
  return (c & 8u) ? -mag : mag;
}

// E4M3 of a value already known to be < 448 in magnitude (nearest even).
__device__ __forceinline__ uint32_t to_fp8(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
}

// Expand one 64-key tile of one KV head to FP8.  K~: [Hkv][tiles*64][128];
// V~^T: [Hkv][tiles][128][64] (keys in vt_pos order).  Keys >= total are 0.
__global__ void __launch_bounds__(256) expand_kernel(PrefillArgs p) {
  const int tile = blockIdx.x, kvh = blockIdx.y, tid = threadIdx.x;
  __shared__ uint8_t vt[kD * kTile];

  // K: thread -> key tid/4, elements 32q..32q+31
  {
    const int kk = tid >> 2, q = tid & 3;
    const int t = tile * kTile + kk;
    u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = {0u, 0u, 0u, 0u};
    if (t < p.total) {
      const int page = p.page_table_row[t / kPage], slot = t % kPage;
      const size_t slab = (size_t)page * p.hkv + kvh;
      const u32x4 kq = *reinterpret_cast<const u32x4*>(p.k_codes + slab * kSlab + slot * 64 + q * 16);
      const uint32_t ksc = *reinterpret_cast<const uint16_t*>(p.k_scales + slab * kScaleSlab + slot * kNBlk + q * 2);
      const float s0 = e4m3_to_float(ksc & 0xFFu) * 0.125f, s1 = e4m3_to_float(ksc >> 8) * 0.125f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = i < 2 ? s0 : s1;
        uint32_t word0 = 0, word1 = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t b8 = to_fp8(e2m1_value((kq[i] >> (4 * j)) & 15u) * sc);
          if (j < 4) word0 |= b8 << (8 * j);
          else word1 |= b8 << (8 * (j - 4));
        }
        if (i < 2) { o0[2 * i] = word0; o0[2 * i + 1] = word1; }
        else { o1[2 * (i - 2)] = word0; o1[2 * (i - 2) + 1] = word1; }
      }
    }
    u32x4* dst = reinterpret_cast<u32x4*>(p.k8 + (((size_t)kvh * p.num_tiles * kTile) + (size_t)t) * kD + q * 32);
    dst[0] = o0;
    dst[1] = o1;
  }
  // V: dword (token group tg, byte b) holds byte b of 4 consecutive tokens
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int idx = tid + 256 * r;
    const int tg = idx >> 6, b = idx & 63;
    const int t0 = tile * kTile + 4 * tg;
    uint32_t W = 0, sc4 = 0;
    if (t0 < p.total) {
      const int page = p.page_table_row[t0 / kPage], slot0 = t0 % kPage;
      const size_t slab = (size_t)page * p.hkv + kvh;
      W = *reinterpret_cast<const uint32_t*>(p.v_codes + slab * kSlab + (slot0 >> 2) * 256 + b * 4);
      sc4 = *reinterpret_cast<const uint32_t*>(p.v_scales + slab * kScaleSlab + (b >> 3) * kPage + slot0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = 4 * tg + j;
      const bool live = t0 + j < p.total;
      const float sc = e4m3_to_float((sc4 >> (8 * j)) & 0xFFu) * 0.125f;
      const uint32_t byte = (W >> (8 * j)) & 0xFFu;
      const int pos = vt_pos(kk);
      vt[(2 * b) * kTile + pos] = live ? (uint8_t)to_fp8(e2m1_value(byte & 15u) * sc) : 0;
      vt[(2 * b + 1) * kTile + pos] = live ? (uint8_t)to_fp8(e2m1_value(byte >> 4) * sc) : 0;
    }
  }
  __syncthreads();
  const u32x4* src = reinterpret_cast<const u32x4*>(vt) + tid * 2;
  u32x4* dst = reinterpret_cast<u32x4*>(p.v8 + ((size_t)kvh * p.num_tiles + tile) * (kD * kTile)) + tid * 2;
  dst[0] = src[0];
  dst[1] = src[1];
}

template <bool F32Q>
__global__ void __launch_bounds__(256) fa_kernel(PrefillArgs p) {
  const int nrows = p.T * p.group;
  const int kvh = blockIdx.x % p.hkv;             // consecutive blocks spread over XCDs;
  const int rt = blockIdx.x / p.hkv;              // one KV head's tiles share an XCD when Hkv divides 8
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int n = lane & 31, h = lane >> 5;
  const int row0 = rt * 128;
  const int row = row0 + wave * 32 + n;
  const bool row_ok = row < nrows;
  const int qi = row_ok ? row / p.group : 0;
  const int head = kvh * p.group + (row_ok ? row % p.group : 0);
  const int lim = p.causal ? p.prefix + qi : p.total - 1;    // last key this row sees

  __shared__ uint8_t ks[2][kTile * kKRow];
  __shared__ uint8_t vs[2][kD * kVRow];

  // ---- Q^T operand: lane (row n, half h) holds q[64h + 32i + j] in byte j of qb[i]
  intx8 qb[2];
  float rowscale;
  {
    float qv[64];
    if (row_ok) {
      const size_t off = ((size_t)qi * p.hq + head) * kD + h * 64;
      if (F32Q) {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(p.q) + off);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float4 v = src[i];
          qv[4 * i] = v.x; qv[4 * i + 1] = v.y; qv[4 * i + 2] = v.z; qv[4 * i + 3] = v.w;
        }
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + off);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint4 v = src[i];
          qv[8 * i + 0] = bf16_lo(v.x); qv[8 * i + 1] = bf16_hi(v.x);
          qv[8 * i + 2] = bf16_lo(v.y); qv[8 * i + 3] = bf16_hi(v.y);
          qv[8 * i + 4] = bf16_lo(v.z); qv[8 * i + 5] = bf16_hi(v.z);
          qv[8 * i + 6] = bf16_lo(v.w); qv[8 * i + 7] = bf16_hi(v.w);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 64; ++i) qv[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(qv[i]));
    amax = max_across_halves(amax);
    int shift = amax > 0.0f ? 7 - ilogbf(amax) : 0;      // amax * 2^shift in [128, 256)
    shift = max(-120, min(120, shift));
    // scores: S * 2^-shift * 8 (K~ carries 2^-3) * s_tK * softmax_scale * log2(e)
    rowscale = ldexpf(1.0f, -shift) * 8.0f * p.k_scale * p.softmax_scale * 1.4426950408889634f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float* v = qv + 32 * i + 4 * w;
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], shift), ldexpf(v[1], shift), 0, false);
        int both = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], shift), ldexpf(v[3], shift), lo, true);
        qb[i][w] = both;
      }
    }
  }

  // ---- key range of this workgroup
  const int last_row = min(row0 + 127, nrows - 1);
  const int first_q = row0 / p.group, last_q = last_row / p.group;
  const int kv_len = p.causal ? min(p.total, p.prefix + last_q + 1) : p.total;
  const int ntiles = (kv_len + kTile - 1) / kTile;
  const int mask_from = p.causal ? (p.prefix + first_q + 1) / kTile : ntiles;   // tiles needing a mask

  const uint8_t* k8 = p.k8 + (size_t)kvh * p.num_tiles * kTile * kD;
  const uint8_t* v8 = p.v8 + (size_t)kvh * p.num_tiles * kD * kTile;

  // tile loads: K~ chunk c (0..511) = key c/8, bytes 16(c%8); V~^T chunk c = d c/4, bytes 16(c%4)
  auto gload = [&](int tile, u32x4 r[4]) {
    const uint8_t* kt = k8 + (size_t)tile * kTile * kD;
    const uint8_t* vt = v8 + (size_t)tile * kD * kTile;
    r[0] = *reinterpret_cast<const u32x4*>(kt + tid * 16);
    r[1] = *reinterpret_cast<const u32x4*>(kt + (tid + 256) * 16);
    r[2] = *reinterpret_cast<const u32x4*>(vt + tid * 16);
    r[3] = *reinterpret_cast<const u32x4*>(vt + (tid + 256) * 16);
  };
  auto sstore = [&](int buf, const u32x4 r[4]) {
    const int c0 = tid, c1 = tid + 256;
    *reinterpret_cast<u32x4*>(&ks[buf][(c0 >> 3) * kKRow + (c0 & 7) * 16]) = r[0];
    *reinterpret_cast<u32x4*>(&ks[buf][(c1 >> 3) * kKRow + (c1 & 7) * 16]) = r[1];
    *reinterpret_cast<u32x4*>(&vs[buf][(c0 >> 2) * kVRow + (c0 & 3) * 16]) = r[2];
    *reinterpret_cast<u32x4*>(&vs[buf][(c1 >> 2) * kVRow + (c1 & 3) * 16]) = r[3];
  };

  floatx16 acc_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[i][r] = 0.0f;
  float m_ref = -INFINITY, l_run = 0.0f;

  u32x4 pre[4];
  if (ntiles > 0) {
    gload(0, pre);
    sstore(0, pre);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1, pre);

    // ---- S^T for the two 32-key blocks
    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint8_t* kr = &ks[buf][(kb * 32 + n) * kKRow + h * 64];
      intx8 a0, a1;
      *reinterpret_cast<u32x4*>(&a0) = *reinterpret_cast<const u32x4*>(kr);
      *(reinterpret_cast<u32x4*>(&a0) + 1) = *reinterpret_cast<const u32x4*>(kr + 16);
      *reinterpret_cast<u32x4*>(&a1) = *reinterpret_cast<const u32x4*>(kr + 32);
      *(reinterpret_cast<u32x4*>(&a1) + 1) = *reinterpret_cast<const u32x4*>(kr + 48);
      floatx16 c = {};
      c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, qb[0], c, 0, 0, 0, 127, 0, 127);
      c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, qb[1], c, 0, 0, 0, 127, 0, 127);
      s[kb] = c;
    }
    // ---- scale, mask, row max
    const int kbase = t * kTile;
    const bool need_mask = t >= mask_from || kbase + kTile > kv_len;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = s[kb][r] * rowscale;
        if (need_mask) {
          const int key = kbase + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key > lim || key >= kv_len) v = -INFINITY;
        }
        s[kb][r] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = max_across_halves(mx);
    // lazy max: rescale only when the row max grows by more than 0.5 (log2),
    // which keeps p <= 2^0.5 so p * 256 stays inside E4M3's range
    const bool grow = mx > m_ref + 0.5f;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_ref;
      const float alpha = grow ? exp2f(m_ref - m_new) : 1.0f;
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_o[i] *= alpha;
    }
    // ---- P^T (FP8, x256) and the row sum
    intx8 pb;
    float lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, r0 = (w & 3) * 4;
      float e0 = exp2f(s[kb][r0] - m_ref), e1 = exp2f(s[kb][r0 + 1] - m_ref);
      float e2 = exp2f(s[kb][r0 + 2] - m_ref), e3 = exp2f(s[kb][r0 + 3] - m_ref);
      lsum += (e0 + e1) + (e2 + e3);
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e0 * 256.0f, e1 * 256.0f, 0, false);
      pb[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e2 * 256.0f, e3 * 256.0f, lo, true);
    }
    l_run += lsum;
    // ---- O^T += V~^T P^T
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const uint8_t* vr = &vs[buf][(db * 32 + n) * kVRow + h * 32];
      intx8 a;
      *reinterpret_cast<u32x4*>(&a) = *reinterpret_cast<const u32x4*>(vr);
      *(reinterpret_cast<u32x4*>(&a) + 1) = *reinterpret_cast<const u32x4*>(vr + 16);
      acc_o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, acc_o[db], 0, 0, 0, 127, 0, 127);
    }
    if (t + 1 < ntiles) sstore(buf ^ 1, pre);
    __syncthreads();
  }

  // ---- epilogue: O / l * s_tV * 8 (V~ carries 2^-3) / 256 (P carries 2^8)
  const float l_tot = sum_across_halves(l_run);
  if (row_ok) {
    const float f = l_tot > 0.0f ? p.v_scale * (8.0f / 256.0f) / l_tot : 0.0f;
    float* o = p.out + ((size_t)qi * p.hq + head) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * h;
        float4 v = make_float4(acc_o[db][4 * g4] * f, acc_o[db][4 * g4 + 1] * f,
                               acc_o[db][4 * g4 + 2] * f, acc_o[db][4 * g4 + 3] * f);
        *reinterpret_cast<float4*>(o + d) = v;
      }
  }
}

hipError_t launch_prefill(const PrefillArgs& a, bool f32_q, hipStream_t s) {
  expand_kernel<<<dim3(a.num_tiles, a.hkv), 256, 0, s>>>(a);
  const int nrows = a.T * a.group;
  const unsigned rtiles = (unsigned)((nrows + 127) / 128);
  if (f32_q) fa_kernel<true><<<rtiles * a.hkv, 256, 0, s>>>(a);
  else fa_kernel<false><<<rtiles * a.hkv, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace nvfp4
