// prefill.hip -- chunked-prefill attention over the NVFP4 cache.
//
// Flow ("NVIDIA解説: NVFP4 KV Cacheで長コンテキストLLM推論を最適化", section
// 量子化・逆量子化フロー): the NVFP4 cache is dequantized and attention runs
// on the dequantized operands with an FP32 accumulator.  Two operand
// precisions share one kernel structure:
//   FP8 (the pages' flow): K~, V~ = E4M3(e2m1 * s_block / 8) (<= 336, no
//     overflow); Q' = E4M3(q * c * 2^-e_row), row maximum in [64, 256), c
//     the score scale into log2 units, with 2^e_row given back by the MFMA's
//     per-row E8M0 operand scale; P = E4M3(p * 256) with p <= 2^0.5 (lazy
//     max, below) and its row sums taken on the matrix core; 32x32x64 FP8
//     MFMAs.
//   F16: K~, V~ = e2m1 * s_block exactly (at most 6 significant bits,
//     magnitudes 2^-10 .. 2688); Q = F16(q * 2^shift_row) (exact for bf16
//     input in range); P = F16(p); 32x32x16 f16 MFMAs at half the FP8 rate.
//   MXFP4 (the MXFP4 cache, [EXPL] §MXFP4との比較): K enters the score
//     MFMAs as the cache's own E2M1 codes with their E8M0 block scales as
//     the MFMA's per-(row, 32-element) operand scales, read straight from
//     the paged cache (the 32-element MX block is the MFMA's scale block);
//     V is expanded to V~ = E4M3(e2m1 * 2^(e - r_V)), r_V = the cache's
//     v_exp_offset + 2 (the largest block's values reach 384 at most), and
//     the rest of the path is the FP8 path (Q', P, 32x32x64 MFMAs).
// The scores and the output take the scale factors back in FP32.
//
// The expansion is a separate pass over the sequence's cache (expand_kernel)
// into a workspace laid out as MFMA operands, so each K/V element is expanded
// once instead of once per query tile; the attention kernel (fa_kernel) then
// streams 64-key tiles through LDS, double-buffered.
//
// fa_kernel: a 512-thread workgroup owns 256 consecutive (query, head) rows of
// one KV head (row r = query r / G, head r % G), 32 per wave (lane n = row,
// lane half h), in two groups of four waves that alternate between matrix
// and softmax work (see the main loop).  Per 64-key tile and wave:
//   S^T[key][row] = K~ Q^T over two 32-key blocks (the contraction over d is
//     permuted identically in K~ and Q: lane half h holds d in [64h, 64h+64)).
//   softmax over keys: each lane holds 32 keys of one row, the other 32 sit in
//     the lane 32 away (one permlane swap per reduction).
//   O^T[d][row] += V~^T P^T: P^T is the S^T accumulator converted in place,
//     so the key order inside a tile follows the accumulator layout
//     (vt_pos below), which the V~ workspace matches.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace nvfp4 {

constexpr int kTile = kPrefillTile;      // 64 keys
typedef short short2v __attribute__((vector_size(4)));

template <int MODE> struct Prec;
template <> struct Prec<kPrefillFP8> {
  static constexpr int EB = 1;                       // bytes per operand element
  static constexpr float kExpand = 0.125f;           // K~, V~ carry 2^-3
};
template <> struct Prec<kPrefillMx> {
  static constexpr int EB = 1;
  static constexpr float kExpand = 1.0f;             // K exact; V~ relative to 2^r_V
};
template <> struct Prec<kPrefillF16> {
  static constexpr int EB = 2;
  static constexpr float kExpand = 1.0f;
  static constexpr int kQTop = 14;                   // |q| 2^shift in [2^14, 2^15)
};

// The FP8 and MXFP4 modes share the FP8 operand path (Q', P, V~ in E4M3).
template <int MODE> constexpr bool kF8Ops = MODE != kPrefillF16;

// Position of key kk (0..63) of a tile inside a V~^T row.
//  FP8 (K = 64 keys per MFMA): S^T key block kb gives lane half h, element r
//    the key kb*32 + 8(r/4) + 4h + r%4; P^T element j = 16 kb + r; the row
//    holds [h][j] for j = 0..31.
//  F16 (K = 16 keys per MFMA u = 0..3): P^T element j = 0..7 of MFMA u is key
//    16u + 8(j/4) + 4h + j%4; the row holds [u][h][j].
template <int MODE>
__device__ __forceinline__ int vt_pos(int kk) {
  if (kF8Ops<MODE>) {
    const int kb = kk >> 5, rem = kk & 31;
    const int h = (rem >> 2) & 1;
    const int j = 16 * kb + (rem >> 3) * 4 + (rem & 3);
    return h * 32 + j;
  } else {
    const int u = kk >> 4, rem = kk & 15;
    const int h = (rem >> 2) & 1;
    const int j = (rem >> 3) * 4 + (rem & 3);
    return (u * 2 + h) * 8 + j;
  }
}

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float mag = e == 0u ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << (e - 1u));
  return (c & 8u) ? -mag : mag;
}

// Operand encoding of a value: E4M3 (nearest even; |v| < 448 here) or F16.
template <int MODE>
__device__ __forceinline__ uint32_t encode(float v) {
  if (kF8Ops<MODE>) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
  _Float16 h = (_Float16)v;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Expand one 64-key tile of one KV head.  K~: [Hkv][tiles*64][128];
// V~^T: [Hkv][tiles][128][64] (keys in vt_pos order).  Keys >= total are 0.
template <int MODE>
__global__ void __launch_bounds__(256) expand_kernel(PrefillArgs p) {
  using P = Prec<MODE>;
  const int tile = blockIdx.x, kvh = blockIdx.y, tid = threadIdx.x;
  __shared__ uint8_t vt[kD * kTile * P::EB];

  // K: thread -> key tid/4, elements 32q..32q+31 (MXFP4: K is read from the
  // cache by the attention kernel)
  if constexpr (MODE != kPrefillMx) {
    const int kk = tid >> 2, q = tid & 3;
    const int t = tile * kTile + kk;
    uint32_t o[8 * P::EB];
#pragma unroll
    for (int i = 0; i < 8 * P::EB; ++i) o[i] = 0u;
    if (t < p.total) {
      const int page = clamp_page(p.page_table_row[t / kPage], p.num_pages), slot = t % kPage;
      const size_t slab = (size_t)page * p.hkv + kvh;
      const u32x4 kq = *reinterpret_cast<const u32x4*>(p.k_codes + slab * kSlab + slot * 64 + q * 16);
      const uint32_t ksc = *reinterpret_cast<const uint16_t*>(p.k_scales + slab * kScaleSlab + slot * kNBlk + q * 2);
      const float s0 = e4m3_to_float(ksc & 0xFFu) * P::kExpand, s1 = e4m3_to_float(ksc >> 8) * P::kExpand;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float sc = e < 16 ? s0 : s1;
        const uint32_t c = (kq[e >> 3] >> (4 * (e & 7))) & 15u;
        const uint32_t b = encode<MODE>(e2m1_value(c) * sc);
        if (P::EB == 1) o[e >> 2] |= b << (8 * (e & 3));
        else o[e >> 1] |= b << (16 * (e & 1));
      }
    }
    u32x4* dst = reinterpret_cast<u32x4*>(p.kx + ((((size_t)kvh * p.num_tiles * kTile) + (size_t)t) * kD + q * 32) * P::EB);
#pragma unroll
    for (int i = 0; i < 2 * P::EB; ++i) dst[i] = u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
  }
  // V: thread -> token quad tq (keys 4tq..4tq+3 of the tile) x element group
  // m (elements 8m..8m+7): 16 bytes, byte 8j + e = element 8m + e of the
  // token pair (4tq + 2j, 4tq + 2j + 1)
  {
    const int tq = tid >> 4, m = tid & 15;
    const int t0 = tile * kTile + 4 * tq;
    u32x4 W = {0u, 0u, 0u, 0u};
    uint32_t sc4 = 0;
    if (t0 < p.total) {
      const int page = clamp_page(p.page_table_row[t0 / kPage], p.num_pages), slot0 = t0 % kPage;
      const size_t slab = (size_t)page * p.hkv + kvh;
      W = *reinterpret_cast<const u32x4*>(p.v_codes + slab * kSlab + (slot0 >> 2) * 256 + m * 16);
      // the block of elements 8m..8m+7 for the 4 tokens: NVFP4 block m/2 of
      // 16, MXFP4 block m/4 of 32 (scale planes [block][token 16])
      if constexpr (MODE == kPrefillMx)
        sc4 = *reinterpret_cast<const uint32_t*>(p.v_scales + slab * kMxScaleSlab + (m >> 2) * kPage + slot0);
      else
        sc4 = *reinterpret_cast<const uint32_t*>(p.v_scales + slab * kScaleSlab + (m >> 1) * kPage + slot0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {               // token 4tq + j
      const int kk = 4 * tq + j;
      const bool live = t0 + j < p.total;
      const uint32_t sb = (sc4 >> (8 * j)) & 0xFFu;
      // MXFP4: 2^(e - r_V) with e = sb - 127 (a power of two, possibly a
      // subnormal FP32 or zero far below the tensor's blocks)
      const float sc = MODE == kPrefillMx ? ldexpf(1.0f, (int)sb - 127 - p.v_ref) : e4m3_to_float(sb) * P::kExpand;
      const int pos = vt_pos<MODE>(kk);
      const int sh = 4 * (j & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {             // element 8m + e
        const uint32_t c = (W[(j >> 1) * 2 + (e >> 2)] >> (8 * (e & 3) + sh)) & 15u;
        // (MXFP4: a block above the range the cache's offset was set for
        // saturates at 448)
        const float x = MODE == kPrefillMx ? fminf(fmaxf(e2m1_value(c) * sc, -448.0f), 448.0f) : e2m1_value(c) * sc;
        const uint32_t v = live ? encode<MODE>(x) : 0u;
        if (P::EB == 1) vt[(8 * m + e) * kTile + pos] = (uint8_t)v;
        else reinterpret_cast<uint16_t*>(vt)[(8 * m + e) * kTile + pos] = (uint16_t)v;
      }
    }
  }
  __syncthreads();
  const u32x4* src = reinterpret_cast<const u32x4*>(vt) + tid * 2 * P::EB;
  u32x4* dst = reinterpret_cast<u32x4*>(p.vx + ((size_t)kvh * p.num_tiles + tile) * (kD * kTile * P::EB)) + tid * 2 * P::EB;
#pragma unroll
  for (int i = 0; i < 2 * P::EB; ++i) dst[i] = src[i];
}

template <int MODE, bool F32Q>
__global__ void __launch_bounds__(512) fa_kernel(PrefillArgs p) {
  using P = Prec<MODE>;
  constexpr int EB = P::EB;
  // LDS bytes per K row (padded): the expanded K~, or for MXFP4 the cache's
  // 64 code bytes, followed (MXFP4) by the 4 block scales of each key
  constexpr int KROW = MODE == kPrefillMx ? 64 + 16 : kD * EB + 16;
  constexpr int KBYTES = MODE == kPrefillMx ? kTile * KROW + kTile * 4 : kTile * KROW;
  constexpr int VROW = kTile * EB + 16;     // LDS bytes per V~^T row (padded)
  constexpr int NT = 512;                   // threads: 8 waves of 32 rows
  constexpr int ROWS = NT / 2;              // (query, head) rows per workgroup
  constexpr int NCH = 512 * EB;             // 16-byte chunks per operand tile
  constexpr int CPT = NCH / NT;             // chunks per thread per operand

  const int nrows = p.T * p.group;
  const int kvh = blockIdx.x % p.hkv;       // one KV head's row tiles land on the same XCD
  const int rt = blockIdx.x / p.hkv;        // when Hkv divides the 8 XCDs
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int n = lane & 31, h = lane >> 5;
  const int row0 = rt * ROWS;
  const int row = row0 + wave * 32 + n;
  const bool row_ok = row < nrows;
  const int qi = row_ok ? row / p.group : 0;
  const int head = kvh * p.group + (row_ok ? row % p.group : 0);
  const int lim = p.causal ? p.prefix + qi : p.total - 1;    // last key this row sees

  __shared__ __attribute__((aligned(16))) uint8_t ks[2][KBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vs[2][kD * VROW];

  // ---- Q^T operand: lane (row n, half h) holds q[64h + e], e = 0..63, in
  // operand order (byte e for FP8, half e for F16).  MXFP4: the FP4 A
  // operand of a 32x32x64 product gives lane (row, half h) the contraction
  // indices 16h .. 16h+15 (its nibbles 0-15) and 32+16h .. 47+16h (nibbles
  // 16-31) under one scale, and the lane loads one 32-element MX block of K
  // (block 2h + i in product i); Q' then holds, for product i and lane half
  // h, byte e = q[64 (e/16) + 32 i + 16 h + e%16]: the lane keeps the
  // 16-element chunks q[32 c + 16 h ..] (c = 0..3) as qv[16 c ..]
  uint32_t qw[16 * EB];
  float rowscale = 1.0f;    // F16: scores * rowscale are in log2 units
  int qscale = 127;         // FP8: E8M0 scale of the Q' operand
  {
    float qv[64];
    if (row_ok && MODE == kPrefillMx) {
      const size_t base = ((size_t)qi * p.hq + head) * kD + h * 16;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (F32Q) {
          const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(p.q) + base + 32 * c);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float4 v = src[i];
            float* d = qv + 16 * c + 4 * i;
            d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
          }
        } else {
          const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + base + 32 * c);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            uint4 v = src[i];
            float* d = qv + 16 * c + 8 * i;
            d[0] = bf16_lo(v.x); d[1] = bf16_hi(v.x); d[2] = bf16_lo(v.y); d[3] = bf16_hi(v.y);
            d[4] = bf16_lo(v.z); d[5] = bf16_hi(v.z); d[6] = bf16_lo(v.w); d[7] = bf16_hi(v.w);
          }
        }
      }
    } else if (row_ok) {
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
    // score scale: (q . K~) * c is the score in log2 units
    const float c = p.k_scale * p.softmax_scale * 1.4426950408889634f / P::kExpand;
    if constexpr (kF8Ops<MODE>) {
      // Q' = E4M3(q c 2^-(ea + ec - 6)) with the row maximum in [64, 256);
      // the MFMA's per-row E8M0 scale on Q' gives back 2^(ea + ec - 6), so
      // the scores come out of the MFMA in log2 units
      const int ea = amax > 0.0f ? ilogbf(amax) : 0;
      const int ec = c > 0.0f ? ilogbf(c) : 0;
      const float cn = c > 0.0f ? ldexpf(c, 6 - ec) : 0.0f;
      qscale = 127 + max(-127, min(127, ea + ec - 6));
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        // product w / 8, bytes 4 (w % 8) .. +3 (MXFP4: chunk w/8 for the
        // first 16 bytes, chunk 2 + w/8 for the last 16)
        const float* v = qv + (MODE == kPrefillMx ? ((w & 4) ? 32 : 0) + 16 * (w >> 3) + 4 * (w & 3) : 4 * w);
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], -ea) * cn, ldexpf(v[1], -ea) * cn, 0, false);
        qw[w] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], -ea) * cn, ldexpf(v[3], -ea) * cn, lo, true);
      }
    } else {
      int shift = amax > 0.0f ? P::kQTop - ilogbf(amax) : 0;
      shift = max(-120, min(120, shift));
      rowscale = ldexpf(c, -shift);
#pragma unroll
      for (int w = 0; w < 32; ++w) {
        const float* v = qv + 2 * w;
        qw[w] = encode<MODE>(ldexpf(v[0], shift)) | (encode<MODE>(ldexpf(v[1], shift)) << 16);
      }
    }
  }

  // ---- key range of this workgroup
  const int last_row = min(row0 + ROWS - 1, nrows - 1);
  const int first_q = row0 / p.group, last_q = last_row / p.group;
  const int kv_len = p.causal ? min(p.total, p.prefix + last_q + 1) : p.total;
  const int ntiles = (kv_len + kTile - 1) / kTile;
  const int mask_from = p.causal ? (p.prefix + first_q + 1) / kTile : ntiles;   // tiles needing a mask

  const uint8_t* kx = p.kx + (size_t)kvh * p.num_tiles * kTile * kD * EB;
  const uint8_t* vx = p.vx + (size_t)kvh * p.num_tiles * kD * kTile * EB;

  // tile loads: K~ chunk c = key c/(8 EB), 16 bytes at (c % (8 EB)) * 16;
  // V~^T chunk c = d c/(4 EB), 16 bytes at (c % (4 EB)) * 16
  // V~^T chunk of thread tid, as (row d, 16-byte column): FP8 rows hold 4
  // chunks, and 8 consecutive lanes take one column of 8 consecutive rows, so
  // that their LDS stores (row stride 80 bytes) fall in distinct banks; the
  // wave still covers 1 KiB of the tile contiguously
  auto vchunk = [&](int c) -> int2 {
    if constexpr (EB == 1) return make_int2(8 * (c >> 5) + (c & 7), (c >> 3) & 3);
    else return make_int2(c / (4 * EB), c % (4 * EB));
  };
  // K tile loads.  MXFP4: thread c < 256 takes 16 code bytes of key
  // vchunk(c) (row = key, column = 16-byte group; the same bank-spread
  // lane mapping), thread 256 + u the 16 scale bytes of keys 4u .. 4u+3
  // ([token][block 4], one page), straight from the paged cache; keys past
  // the context load zeros
  auto gload_k = [&](int tile, u32x4 r[CPT]) {
    if constexpr (MODE == kPrefillMx) {
      r[0] = u32x4{0u, 0u, 0u, 0u};
      const int c = tid;
      if (c < 256 + kTile / 4) {
        const int key = c < 256 ? vchunk(c).x : 4 * (c - 256);
        const int t = tile * kTile + key;
        if (t < p.total) {
          const int page = clamp_page(p.page_table_row[t / kPage], p.num_pages), slot = t % kPage;
          const size_t slab = (size_t)page * p.hkv + kvh;
          r[0] = c < 256 ? *reinterpret_cast<const u32x4*>(p.k_codes + slab * kSlab + slot * 64 + vchunk(c).y * 16)
                         : *reinterpret_cast<const u32x4*>(p.k_scales + slab * kMxScaleSlab + slot * kMxNBlk);
        }
      }
    } else {
      const uint8_t* kt = kx + (size_t)tile * kTile * kD * EB;
#pragma unroll
      for (int i = 0; i < CPT; ++i) r[i] = *reinterpret_cast<const u32x4*>(kt + (tid + NT * i) * 16);
    }
  };
  auto gload_v = [&](int tile, u32x4 r[CPT]) {
    const uint8_t* vt = vx + (size_t)tile * kD * kTile * EB;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int2 rc = vchunk(tid + NT * i);
      r[i] = *reinterpret_cast<const u32x4*>(vt + (rc.x * 4 * EB + rc.y) * 16);
    }
  };
  auto sstore_k = [&](int buf, const u32x4 r[CPT]) {
    if constexpr (MODE == kPrefillMx) {
      const int c = tid;
      if (c < 256) {
        const int2 rc = vchunk(c);
        *reinterpret_cast<u32x4*>(&ks[buf][rc.x * KROW + rc.y * 16]) = r[0];
      } else if (c < 256 + kTile / 4) {
        *reinterpret_cast<u32x4*>(&ks[buf][kTile * KROW + (c - 256) * 16]) = r[0];
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + NT * i;
      *reinterpret_cast<u32x4*>(&ks[buf][(c / (8 * EB)) * KROW + (c % (8 * EB)) * 16]) = r[i];
    }
  };
  auto sstore_v = [&](int buf, const u32x4 r[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int2 rc = vchunk(tid + NT * i);
      *reinterpret_cast<u32x4*>(&vs[buf][rc.x * VROW + rc.y * 16]) = r[i];
    }
  };

  // FP8: the score MFMAs start from -bias (an integer per row, 0 at first),
  // so s and the reference max m are relative to it.  The rescale keeps
  // |m| <= 100, moving the bias when needed; exponentials are then taken of
  // s itself (2^s neither overflows nor loses a weight above 2^-26 of the
  // row max) and the conversion to E4M3 divides by 2^(m - 4).
  float bias = 0.0f;
  floatx16 cbias = {};
  float pscale = 0x1p-4f;

  // ---- S^T of the tile in ks[buf], two 32-key blocks
  auto qk = [&](int buf, floatx16 s[2]) {
    if constexpr (MODE == kPrefillMx) {
      // A = the keys' E2M1 codes (16 bytes = one 32-element MX block per
      // lane) with that block's E8M0 scale; lane half h of product i takes
      // block 2h + i, in the order of the Q' operand above
      intx8 a[2][2];
      int sa[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = kb * 32 + n, blk = 2 * h + i;
          const u32x4 v = *reinterpret_cast<const u32x4*>(&ks[buf][row * KROW + 16 * blk]);
          a[kb][i] = intx8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
          sa[kb][i] = ks[buf][kTile * KROW + row * 4 + blk];
        }
      __builtin_amdgcn_sched_barrier(0);       // keep the reads ahead of the products
      s[0] = cbias;
      s[1] = cbias;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        intx8 b;
#pragma unroll
        for (int w = 0; w < 8; ++w) b[w] = (int)qw[8 * i + w];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[kb][i], b, s[kb], 4, 0, 0, sa[kb][i], 0, qscale);
      }
    } else if constexpr (MODE == kPrefillFP8) {
      // all LDS reads first, then the products with the two key blocks'
      // chains interleaved
      intx8 a[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint8_t* kr = &ks[buf][(kb * 32 + n) * KROW + h * 64 + 32 * i];
          *reinterpret_cast<u32x4*>(&a[kb][i]) = *reinterpret_cast<const u32x4*>(kr);
          *(reinterpret_cast<u32x4*>(&a[kb][i]) + 1) = *reinterpret_cast<const u32x4*>(kr + 16);
        }
      __builtin_amdgcn_sched_barrier(0);       // keep the reads ahead of the products
      s[0] = cbias;
      s[1] = cbias;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        intx8 b;
#pragma unroll
        for (int w = 0; w < 8; ++w) b[w] = (int)qw[8 * i + w];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[kb][i], b, s[kb], 0, 0, 0, 127, 0, qscale);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint8_t* kr = &ks[buf][(kb * 32 + n) * KROW + h * 64 * EB];
        floatx16 c = floatx16{};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const u32x4 av = *reinterpret_cast<const u32x4*>(kr + 16 * i);
          const u32x4 bv = {qw[4 * i], qw[4 * i + 1], qw[4 * i + 2], qw[4 * i + 3]};
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, av),
                                                      __builtin_bit_cast(halfx8, bv), c, 0, 0, 0);
        }
        s[kb] = c;
      }
    }
  };

  floatx16 acc_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[i][r] = 0.0f;
  // ---- O^T += V~^T P^T with the tile in vs[buf]
  auto pv = [&](int buf, const uint32_t pw[8 * EB]) {
    if constexpr (kF8Ops<MODE>) {
      // all LDS reads first, then four independent products
      intx8 a[4], b;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint8_t* vr = &vs[buf][(db * 32 + n) * VROW + h * 32];
        *reinterpret_cast<u32x4*>(&a[db]) = *reinterpret_cast<const u32x4*>(vr);
        *(reinterpret_cast<u32x4*>(&a[db]) + 1) = *reinterpret_cast<const u32x4*>(vr + 16);
      }
#pragma unroll
      for (int w = 0; w < 8; ++w) b[w] = (int)pw[w];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        acc_o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[db], b, acc_o[db], 0, 0, 0, 127, 0, 127);
      return;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const uint8_t* vr = &vs[buf][(db * 32 + n) * VROW];
      if constexpr (kF8Ops<MODE>) {
        intx8 a, b;
#pragma unroll
        for (int w = 0; w < 8; ++w) b[w] = (int)pw[w];
        *reinterpret_cast<u32x4*>(&a) = *reinterpret_cast<const u32x4*>(vr + h * 32);
        *(reinterpret_cast<u32x4*>(&a) + 1) = *reinterpret_cast<const u32x4*>(vr + h * 32 + 16);
        acc_o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc_o[db], 0, 0, 0, 127, 0, 127);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const u32x4 av = *reinterpret_cast<const u32x4*>(vr + (u * 2 + h) * 16);
          const u32x4 bv = {pw[4 * u], pw[4 * u + 1], pw[4 * u + 2], pw[4 * u + 3]};
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, av),
                                                              __builtin_bit_cast(halfx8, bv), acc_o[db], 0, 0, 0);
        }
      }
    }
  };

  // the reference max starts finite and far below any score, so that keys
  // masked to -inf give p = 0, never NaN
  float m_ref = -1.0e30f, l_run = 0.0f;
  // FP8: the row sum of P accumulates on the matrix core, next to the
  // product with V~ that consumes the same P (so the softmax interval issues
  // no matrix instruction and never queues behind the other group's).  A
  // 16x16x128 MFMA with P^T as its B operand and a 0/1 A operand: B column c
  // gathers the lanes c, c+16, c+32, c+48 (rows c and c+16, both key halves);
  // A rows 0 and 8 select the key blocks of row c, rows 4 and 12 those of
  // row c+16, so result element 0 of every lane is the sum of its own row.
  floatx4 acc_l = {0.0f, 0.0f, 0.0f, 0.0f};
  intx8 ones;
  {
    const int i = lane & 15, g = lane >> 4;
    const bool one = ((i == 0 || i == 8) && !(g & 1)) || ((i == 4 || i == 12) && (g & 1));
#pragma unroll
    for (int w = 0; w < 8; ++w) ones[w] = one ? 0x38383838 : 0;   // E4M3 1.0
  }

  // ---- mask (diagonal and tail tiles), row max and the lazy rescale (FP8:
  // on log2 scores; F16: on raw scores, the positive row scale being
  // applied inside the exponent)
  auto row_max = [&](int t, floatx16 s[2]) {
    const int kbase = t * kTile;
    if (t >= mask_from || kbase + kTile > kv_len) {
      // this lane's keys are kbase + 4h + off with off = kb*32 + 8*(r/4) + r%4
      const int klim = min(lim, kv_len - 1) - kbase - 4 * h;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
          s[kb][r] = off <= klim ? s[kb][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return max_across_halves(mx) * rowscale;
  };
  // lazy max: rescale only when a row max grows by more than kLazy (log2)
  // over the reference, so p <= 2^kLazy (FP8: p * 2^4 <= 256 stays inside
  // E4M3's range; F16: p <= 256).  A rescale of any row costs the whole
  // wave a pass over its accumulators, so the threshold is kept large
  constexpr float kLazy = kF8Ops<MODE> ? 4.0f : 8.0f;
  auto rescale = [&](float mx, floatx16 s[2]) {
    const bool grow = mx > m_ref + kLazy;
    if (__any(grow)) {
      // FP8 keeps the reference max an integer (the conversion scale is a
      // power of two); m >= mx keeps p <= 1 on this tile
      const float m_new = grow ? (kF8Ops<MODE> ? ceilf(mx) : mx) : m_ref;
      const float alpha = fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
      acc_l *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_o[i] *= alpha;
      if constexpr (kF8Ops<MODE>) {
        // move the bias of rows whose max left [-100, 100] (a row still at
        // the initial reference has seen no key yet and keeps it)
        const float shift = (fabsf(m_ref) > 100.0f && m_ref > -1.0e29f) ? m_ref : 0.0f;
        if (__any(shift != 0.0f)) {
          bias += shift;
          m_ref -= shift;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            cbias[r] = -bias;
            s[0][r] -= shift;
            s[1][r] -= shift;
          }
        }
        pscale = ldexpf(1.0f, (int)fminf(fmaxf(m_ref, -100.0f), 100.0f) - 4);
      }
    }
  };
  // ---- P^T and the row sum
  auto probs = [&](const floatx16 s[2], uint32_t pw[8 * EB]) {
    if constexpr (kF8Ops<MODE>) {
      // P^T = E4M3(2^(s - m + 4)); the factor 2^4 cancels in O / l (weights
      // below 2^-13 of 2^m fall under E4M3's smallest value)
      auto conv = [&](float e0, float e1, float e2, float e3) {
        const short2v lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(short2v{0, 0}, e0, e1, pscale, false);
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, e2, e3, pscale, true));
      };
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2, r0 = (w & 3) * 4;
        pw[w] = conv(fast_exp2(s[kb][r0]), fast_exp2(s[kb][r0 + 1]),
                     fast_exp2(s[kb][r0 + 2]), fast_exp2(s[kb][r0 + 3]));
      }
    } else {
      // P^T = 2^(s * rowscale - m)
      const float cexp = -m_ref;
      float lsum = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2, r0 = (w & 3) * 4;
        const float e0 = fast_exp2(fmaf(s[kb][r0], rowscale, cexp));
        const float e1 = fast_exp2(fmaf(s[kb][r0 + 1], rowscale, cexp));
        const float e2 = fast_exp2(fmaf(s[kb][r0 + 2], rowscale, cexp));
        const float e3 = fast_exp2(fmaf(s[kb][r0 + 3], rowscale, cexp));
        lsum += (e0 + e1) + (e2 + e3);
        pw[2 * w] = encode<MODE>(e0) | (encode<MODE>(e1) << 16);
        pw[2 * w + 1] = encode<MODE>(e2) | (encode<MODE>(e3) << 16);
      }
      l_run += lsum;
    }
  };

  u32x4 rk[CPT];
  uint32_t pw[8 * EB];
  // Two wave groups in ping-pong: waves 0-3 (group A, rows 0-127) and 4-7
  // (group B, rows 128-255) share each SIMD and the K~/V~ tiles.  Between
  // workgroup barriers a group runs either its matrix interval for step t
  // (S(t) = K~(t) Q'^T and O += V~(t-1) P(t-1)) or its softmax interval
  // (P(t) from S(t)); B runs one interval behind A, so on every SIMD one
  // wave feeds the matrix core while the other keeps the VALU busy.
  // Interval k is step (k - g) / 2 of group g: a matrix interval when
  // k - g is even.  K~(j) lives in ks[j&1] from interval 2j-1 on and is
  // read in intervals 2j (A) and 2j+1 (B); V~(j) lives in vs[j&1] from
  // interval 2j+1 on and is read in 2j+2 and 2j+3.  Each group stores its
  // share of K~(t+1+g) and V~(t+g) in its softmax interval of step t, from
  // registers loaded in its matrix interval of step t-1 (tile indices past
  // the end are clamped for the loads and skipped for the stores).
  const int grp = wave >> 2;
  u32x4 stk[2][CPT], stv[2][CPT];
  floatx16 sc[2];
#pragma unroll
  for (int w = 0; w < 8 * EB; ++w) pw[w] = 0u;
  auto tcl = [&](int t) { return min(max(t, 0), ntiles - 1); };
  // matrix interval of step t (0 .. ntiles) and softmax interval of step t
  // (-1 .. ntiles) of group G; the staging set is t & 1, a constant in the
  // unrolled loop below (a run-time index would make the stores wait for
  // the loads just issued)
  auto matrix = [&](auto G, auto B, int t) {
    gload_k(tcl(t + 2 + G()), stk[B()]);
    gload_v(tcl(t + 1 + G()), stv[B()]);
    if (t < ntiles) qk(B(), sc);
    if (t > 0 && t <= ntiles) {               // the last product is O += V~(ntiles-1) P
      pv(B() ^ 1, pw);
      if constexpr (kF8Ops<MODE>) {
        intx8 b;
#pragma unroll
        for (int w = 0; w < 8; ++w) b[w] = (int)pw[w];
        acc_l = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, b, acc_l, 0, 0, 0, 127, 0, 127);
      }
    }
  };
  auto soft = [&](auto G, auto B, int t) {   // B = (t - 1) & 1, the set to store
    // the tile stores go first: the matrix waves' operand reads keep LDS
    // busy, and stores issued ahead of the softmax complete under it
    // instead of holding up the interval's end
    const int tk = t + 1 + G(), tv = t + G();
    if (tk < ntiles) sstore_k(tk & 1, stk[B()]);
    if (tv >= 0 && tv < ntiles) sstore_v(tv & 1, stv[B()]);
    if (t >= 0 && t < ntiles) {
      rescale(row_max(t, sc), sc);
      probs(sc, pw);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  gload_k(0, rk);
  sstore_k(0, rk);
  if (grp == 1) {                        // for its interval 0 (step -1)
    gload_k(tcl(1), stk[0]);
    gload_v(0, stv[0]);
  }
  gload_k(tcl(1 + grp), stk[1]);
  gload_v(tcl(grp), stv[1]);
  __syncthreads();
  // 2 ntiles + 2 intervals, four per iteration (the last ones may idle);
  // every wave passes the same barriers
  const int iters = (2 * ntiles + 2 + 3) / 4;
  if (grp == 0) {
    for (int i = 0; i < iters; ++i) {
      const int t = 2 * i;
      matrix(I0{}, I0{}, t);
      __syncthreads();
      soft(I0{}, I1{}, t);
      __syncthreads();
      matrix(I0{}, I1{}, t + 1);
      __syncthreads();
      soft(I0{}, I0{}, t + 1);
      __syncthreads();
    }
  } else {
    for (int i = 0; i < iters; ++i) {
      const int t = 2 * i;
      soft(I1{}, I0{}, t - 1);
      __syncthreads();
      matrix(I1{}, I0{}, t);
      __syncthreads();
      soft(I1{}, I1{}, t);
      __syncthreads();
      matrix(I1{}, I1{}, t + 1);
      __syncthreads();
    }
  }

  // ---- epilogue: O / l * s_tV, removing the operand scale factors
  const float l_tot = kF8Ops<MODE> ? acc_l[0] : sum_across_halves(l_run);
  if (row_ok) {
    const float f = l_tot > 0.0f ? p.v_scale / P::kExpand / l_tot : 0.0f;
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

template <int MODE>
static void launch_mode(const PrefillArgs& a, bool f32_q, hipStream_t s) {
  expand_kernel<MODE><<<dim3(a.num_tiles, a.hkv), 256, 0, s>>>(a);
  constexpr int NT = 512, ROWS = NT / 2;
  const int nrows = a.T * a.group;
  const unsigned blocks = (unsigned)((nrows + ROWS - 1) / ROWS) * a.hkv;
  if (f32_q) fa_kernel<MODE, true><<<blocks, NT, 0, s>>>(a);
  else fa_kernel<MODE, false><<<blocks, NT, 0, s>>>(a);
}

hipError_t launch_prefill(const PrefillArgs& a, bool f32_q, hipStream_t s) {
  if (a.mode == kPrefillF16) launch_mode<kPrefillF16>(a, f32_q, s);
  else if (a.mode == kPrefillMx) launch_mode<kPrefillMx>(a, f32_q, s);
  else launch_mode<kPrefillFP8>(a, f32_q, s);
  return hipGetLastError();
}

}  // namespace nvfp4
