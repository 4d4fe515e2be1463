// decode.hip -- decode attention over the paged NVFP4 cache.
//
// The cache is dequantized in registers right before the QK^T and PV
// products ("NVIDIA解説: NVFP4 KV Cacheで長コンテキストLLM推論を最適化",
// section 量子化・逆量子化フロー); softmax and accumulation run in FP32.
//
// Work decomposition (balanced stream): the work units are (sequence, KV
// head, page) triples, ordered sequence-major, then KV head, then page.  The
// grid is one wave64 per resident wave slot of the device; wave w takes a
// contiguous unit range, of equal length for every wave (or weighted by the
// issue share a wave gets on its SIMD: RangeMath), whatever the mix of
// sequence lengths (work counts that do not divide the machine evenly waste
// it: "【CUDA 16GB向け】RTX 5090の長文推論遅延修正と…", section 利用者の報告).
// A (sequence, KV head) segment that lies
// inside one wave's range is finished by that wave; a segment cut by range
// boundaries leaves one normalized partial per wave (at most two per wave: its
// first and its last segment) and merge_kernel combines them with a
// log-sum-exp merge.
//
// Per page (16 tokens), lane l = (col = l%16, kg = l/16):
//   * K: 16-byte buffer load = elements 32kg..32kg+31 of token col (one
//     coalesced 1 KiB wave load) plus 2 block scales; nibbles expand to FP16
//     e2m1 * s_block (exact: at most 6 significant bits, magnitudes
//     2^-10 .. 2688); four 16x16x32 f16 MFMAs give S^T[token][head] for the G
//     query heads of the KV head (columns >= G are zero padding).  The
//     contraction index order is permuted identically on the Q side.
//   * softmax: lane holds 4 tokens of head col; the page max reduces across
//     the 4 lane rows with permlane swaps; running max / sum in FP32 (log2),
//     rescaled lazily.
//   * V: the cache stores V with the two tokens of a pair in one byte, so
//     lane (m = col, kg) loads 16 bytes = elements 8m..8m+7 of tokens
//     4kg..4kg+3, which expand (one conversion per byte, then the block
//     scale) to the A operand of eight 16x16x16 f16 MFMAs
//     O^T[d][head] += V^T P^T with d = 8m + tile.  P^T comes straight from
//     the S^T accumulator layout.
// Pages stream through a kDepth-stage register pipeline (loads of pages
// t+1 .. t+kDepth-1 in flight while page t is computed).
#include <atomic>

#include "common.h"
#include "internal.h"

namespace nvfp4 {

// Cache formats the kernel reads: NVFP4 (the product format), MXFP4 (the
// same code planes with E8M0 scales per 32 elements) and the two comparison
// formats (FP8 E4M3 with a tensor scale, BF16), whose planes hold K as
// [token][element] and V as [token quad][element][token % 4].
template <int FMT> struct PageRegs;
template <> struct PageRegs<kFmtNvfp4> {
  u32x4 kq;       // K codes: 32 nibbles of token col
  u32x4 vq;       // V codes: 4 tokens x 8 nibbles
  uint16_t ksc;   // 2 K block scales
  uint32_t vsc;   // 4 V block scales
};
template <> struct PageRegs<kFmtMxfp4> {
  u32x4 kq;       // K codes: 32 nibbles of token col (MX block kg)
  u32x4 vq;       // V codes: 4 tokens x 8 nibbles
  uint32_t ksc;   // the K block's E8M0 byte
  uint32_t vsc;   // 4 V E8M0 bytes (tokens 4kg .. 4kg + 3)
};
template <> struct PageRegs<kFmtFp8> {
  u32x4 kq[2];    // K: 32 E4M3 bytes of token col
  u32x4 vq[2];    // V: elements 8 col .. 8 col + 7 of tokens 4 kg .. 4 kg + 3
};
template <> struct PageRegs<kFmtBf16> {
  u32x4 kq[4];    // K: 32 bf16 of token col
  u32x4 vq[4];    // V: elements 8 col .. 8 col + 7 of tokens 4 kg .. 4 kg + 3
};

// Bytes per element of a comparison format (FP8 1, BF16 2).
template <int FMT> constexpr int kElemBytes = FMT == kFmtBf16 ? 2 : 1;

// Per-lane byte offsets of the loads of a page (fixed per lane).
struct LaneOffsets {
  int k, ks, v, vs;
};

template <int FMT>
__device__ __forceinline__ LaneOffsets lane_offsets(int col, int kg) {
  if constexpr (FMT == kFmtNvfp4) {
    return {col * 64 + kg * 16, col * kNBlk + kg * 2, kg * 256 + col * 16, (col >> 1) * kPage + kg * 4};
  } else if constexpr (FMT == kFmtMxfp4) {
    // K scales [token][block 4]: token col, block kg; V scales [block 4][token]
    return {col * 64 + kg * 16, col * kMxNBlk + kg, kg * 256 + col * 16, (col >> 2) * kPage + kg * 4};
  } else {
    constexpr int E = kElemBytes<FMT>;
    // K: token col, elements 32 kg ..; V: quad kg, elements 8 col .. (x 4 tokens)
    return {(col * kD + kg * 32) * E, 0, (kg * kD * 4 + col * 32) * E, 0};
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}

// Bytes per (page, head) slab of each plane of a format: K codes (or the
// comparison formats' K plane), K scales, V codes, V scales.
template <int FMT> struct SlabBytes;
template <> struct SlabBytes<kFmtNvfp4> { static constexpr uint32_t k = kSlab, ks = kScaleSlab, v = kSlab, vs = kScaleSlab; };
template <> struct SlabBytes<kFmtMxfp4> { static constexpr uint32_t k = kSlab, ks = kMxScaleSlab, v = kSlab, vs = kMxScaleSlab; };
template <> struct SlabBytes<kFmtFp8> { static constexpr uint32_t k = kPage * kD, ks = 0, v = kPage * kD, vs = 0; };
template <> struct SlabBytes<kFmtBf16> { static constexpr uint32_t k = 2 * kPage * kD, ks = 0, v = 2 * kPage * kD, vs = 0; };

// Buffer resources over whole planes: a page load then only moves the
// scalar offset (slab x slab bytes), and a load past the plane's end returns
// zeros.  Used when every plane fits 32-bit offsets (WIDE == false); larger
// caches build a resource at each slab's base instead.
struct PlaneRsrc {
  __amdgpu_buffer_rsrc_t k, ks, v, vs;
};

template <int FMT>
__device__ __forceinline__ PlaneRsrc plane_rsrc(const DecodeArgs& p) {
  using SB = SlabBytes<FMT>;
  auto mk = [&](const uint8_t* base, uint32_t slab_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0,
                                             (int)(p.num_slabs * slab_bytes), 0x00020000);
  };
  PlaneRsrc r;
  r.k = mk(p.k_codes, SB::k);
  r.v = mk(p.v_codes, SB::v);
  r.ks = SB::ks ? mk(p.k_scales, SB::ks) : r.k;
  r.vs = SB::vs ? mk(p.v_scales, SB::vs) : r.v;
  return r;
}

// Cache policy of the page loads.  A call reads every page of the cache
// once; an NVFP4 or MXFP4 page load instruction covers whole lines (1 KiB of
// codes, 128 or 64 bytes of scales, contiguous over the wave), so the lines
// have no reuse to keep, and with the non-temporal hint the same gather
// moves 6.5 TB/s instead of 5.7 (configuration-4 shape).  The FP8 and BF16
// pages are read 16 bytes per lane per instruction out of 32 or 64
// contiguous bytes per lane, so each line is touched by two or four
// instructions, and non-temporal lines were fetched again (BF16 decode of
// configuration 4: 656 us against 437): those keep the default policy.
template <int FMT>
constexpr int kPageLoadPolicy = (FMT == kFmtNvfp4 || FMT == kFmtMxfp4) ? 2 : 0;

// Buffer loads: the slab base lives in scalar registers and the lane offsets
// are fixed, so a page load needs no vector address temporaries.
template <int FMT, bool WIDE>
__device__ __forceinline__ void load_page(const DecodeArgs& p, const PlaneRsrc& pr, uint32_t slab,
                                          const LaneOffsets& o, PageRegs<FMT>& r) {
  using SB = SlabBytes<FMT>;
  // narrow planes: one resource per plane, the slab in the scalar offset
  const auto rk = WIDE ? page_rsrc(p.k_codes + (size_t)slab * SB::k) : pr.k;
  const auto rv = WIDE ? page_rsrc(p.v_codes + (size_t)slab * SB::v) : pr.v;
  const int sk = WIDE ? 0 : (int)(slab * SB::k), sv = WIDE ? 0 : (int)(slab * SB::v);
  if constexpr (FMT == kFmtNvfp4 || FMT == kFmtMxfp4) {
    const auto rks = WIDE ? page_rsrc(p.k_scales + (size_t)slab * SB::ks) : pr.ks;
    const auto rvs = WIDE ? page_rsrc(p.v_scales + (size_t)slab * SB::vs) : pr.vs;
    const int sks = WIDE ? 0 : (int)(slab * SB::ks), svs = WIDE ? 0 : (int)(slab * SB::vs);
    r.kq = __builtin_amdgcn_raw_buffer_load_b128(rk, o.k, sk, kPageLoadPolicy<FMT>);
    if constexpr (FMT == kFmtNvfp4) r.ksc = __builtin_amdgcn_raw_buffer_load_b16(rks, o.ks, sks, kPageLoadPolicy<FMT>);
    else r.ksc = __builtin_amdgcn_raw_buffer_load_b8(rks, o.ks, sks, kPageLoadPolicy<FMT>);
    r.vq = __builtin_amdgcn_raw_buffer_load_b128(rv, o.v, sv, kPageLoadPolicy<FMT>);
    r.vsc = __builtin_amdgcn_raw_buffer_load_b32(rvs, o.vs, svs, kPageLoadPolicy<FMT>);
  } else {
    constexpr int N = 2 * kElemBytes<FMT>;             // 16-byte loads per lane and operand
#pragma unroll
    for (int i = 0; i < N; ++i) r.kq[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, o.k + 16 * i, sk, kPageLoadPolicy<FMT>);
#pragma unroll
    for (int i = 0; i < N; ++i) r.vq[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, o.v + 16 * i, sv, kPageLoadPolicy<FMT>);
  }
}

struct WaveState {
  floatx4 acc_o[8];   // O^T[d = 8(4kg + r) + i][head col] in acc_o[i][r]
  float m_run;        // reference max (log2 domain) of head col
  float l_run;        // FP8 / BF16 pages: this lane's share of the running sum
  floatx4 acc_l;      // NVFP4 / MXFP4 pages: the running sum of head col in every row
};

// For the 4-bit pages the running sum of the weights is taken on the matrix
// core: a 16x16x16 product of a ones tile with P^T gives every row of head
// col the sum of its 16 weights, as rounded to FP16 for the PV product.  (The
// comparison formats keep the VALU sum: their register budget is spent on
// wider pages.)
template <int FMT> constexpr bool kSumOnMatrixCore = FMT == kFmtNvfp4 || FMT == kFmtMxfp4;

// Lazy rescaling: the accumulators are rescaled only when a head's max grows
// by more than kLazy (log2 units) over the reference, so p = 2^(s - m_run)
// stays <= 2^kLazy, well inside FP16.  The reference starts at a large
// negative finite value so that fully masked pages give p = 0, never NaN.
constexpr float kLazy = 8.0f;
constexpr float kNoMax = -1.0e30f;

__device__ __forceinline__ void reset_state(WaveState& st) {
#pragma unroll
  for (int i = 0; i < 8; ++i) st.acc_o[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  st.m_run = kNoMax;
  st.l_run = 0.0f;
  st.acc_l = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
}

// 2^(byte - 127 - ex) as an FP32, for an E8M0 byte taken relative to 2^ex:
// 0 below the FP32 normal range, and at most 2^13 so that 6 * 2^13 stays
// finite in FP16 (bytes of slots no token owns yet may hold anything, and
// their zero weights must not meet an infinity).
__device__ __forceinline__ float e8m0_rel(uint32_t byte, int ex) {
  const int f = min(127 + 13, max(0, (int)byte - ex));
  return __uint_as_float((uint32_t)f << 23);
}

// S^T = K~ Q^T of one page (before the softmax scale): lane (col, kg) gets
// the products of tokens 4kg .. 4kg + 3 with query head col.
template <bool F32Q, int FMT>
__device__ __forceinline__ floatx4 qk_page(const PageRegs<FMT>& cur, const halfx8 qh[4], const halfx8 ql[4],
                                           int kex) {
  floatx4 acc_s = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (FMT == kFmtNvfp4) {
    const halfx2 ks = e4m3x2_to_half((uint32_t)cur.ksc, false);
    const halfx2 sa = {ks[0], ks[0]}, sb = {ks[1], ks[1]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = cur.kq[i];
      const halfx2 sc = i < 2 ? sa : sb;
      const halfx2 h0 = e2m1x2_to_half<0>(w) * sc;
      const halfx2 h1 = e2m1x2_to_half<1>(w) * sc;
      const halfx2 h2 = e2m1x2_to_half<2>(w) * sc;
      const halfx2 h3 = e2m1x2_to_half<3>(w) * sc;
      const halfx8 a = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
      acc_s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qh[i], acc_s, 0, 0, 0);
      if (F32Q) acc_s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ql[i], acc_s, 0, 0, 0);
    }
  } else if constexpr (FMT == kFmtMxfp4) {
    // the conversion applies the block's power of two itself: e2m1 * 2^(e - kex)
    const float sk = e8m0_rel(cur.ksc & 0xFFu, kex);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = cur.kq[i];
      const halfx2 h0 = e2m1x2_to_half_scaled<0>(w, sk);
      const halfx2 h1 = e2m1x2_to_half_scaled<1>(w, sk);
      const halfx2 h2 = e2m1x2_to_half_scaled<2>(w, sk);
      const halfx2 h3 = e2m1x2_to_half_scaled<3>(w, sk);
      const halfx8 a = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
      acc_s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qh[i], acc_s, 0, 0, 0);
      if (F32Q) acc_s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ql[i], acc_s, 0, 0, 0);
    }
  } else if constexpr (FMT == kFmtFp8) {
    // E4M3 -> FP16 is exact; the tensor scale sits in qscale
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w0 = cur.kq[i >> 1][(2 * i) & 3], w1 = cur.kq[i >> 1][(2 * i + 1) & 3];
      const halfx2 h0 = e4m3x2_to_half(w0, false), h1 = e4m3x2_to_half(w0, true);
      const halfx2 h2 = e4m3x2_to_half(w1, false), h3 = e4m3x2_to_half(w1, true);
      const halfx8 a = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
      acc_s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qh[i], acc_s, 0, 0, 0);
      if (F32Q) acc_s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ql[i], acc_s, 0, 0, 0);
    }
  } else {
    // BF16 operands as stored (qh / ql hold bf16 bit patterns)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, cur.kq[i]);
      acc_s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, qh[i]), acc_s, 0, 0, 0);
      if (F32Q) acc_s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, ql[i]), acc_s, 0, 0, 0);
    }
  }
  return acc_s;
}

// V block scales of a page's four tokens 4kg .. 4kg + 3 as FP16 pairs:
// E4M3 (exact in FP16) or E8M0 relative to 2^vex.
template <int FMT>
__device__ __forceinline__ void v_scales(const PageRegs<FMT>& cur, int vex, halfx2& v01, halfx2& v23) {
  if constexpr (FMT == kFmtNvfp4) {
    v01 = e4m3x2_to_half(cur.vsc, false);
    v23 = e4m3x2_to_half(cur.vsc, true);
  } else {
    v01 = halfx2{(_Float16)e8m0_rel(cur.vsc & 0xFFu, vex), (_Float16)e8m0_rel((cur.vsc >> 8) & 0xFFu, vex)};
    v23 = halfx2{(_Float16)e8m0_rel((cur.vsc >> 16) & 0xFFu, vex), (_Float16)e8m0_rel(cur.vsc >> 24, vex)};
  }
}

// Element SEL of the lane's d run (d = 8 col + 4 HI + SEL) of tokens
// 4kg .. 4kg + 3, times the tokens' block scales: byte SEL of word
// 2 j + HI holds it for the token pair j (4kg + 2j, 4kg + 2j + 1).
template <int SEL, int HI, int FMT>
__device__ __forceinline__ halfx4 v_column(const PageRegs<FMT>& cur, halfx2 v01, halfx2 v23) {
  const halfx2 a0 = e2m1x2_to_half<SEL>(cur.vq[HI]) * v01;
  const halfx2 a1 = e2m1x2_to_half<SEL>(cur.vq[2 + HI]) * v23;
  return halfx4{a0[0], a0[1], a1[0], a1[1]};
}

// Clear the V bytes of the lane's tokens 4kg + r, r >= live: slots that no
// token owns may hold any bytes (NaN patterns among them), and a zero weight
// times a NaN would still be NaN.  Cleared bytes expand to exact zeros in
// every format (an E4M3 scale 0; an E8M0 scale 0 goes to 2^-127 relative to
// the offset, times a finite element).  Each word holds the four tokens in
// order: bytes for the scale words and FP8, 16-bit halves for BF16 pairs.
__device__ __forceinline__ uint32_t live_bytes(int live) {
  return live >= 4 ? 0xFFFFFFFFu : (1u << (8 * max(live, 0))) - 1u;
}

template <int FMT>
__device__ __forceinline__ void drop_v(PageRegs<FMT>& c, int live) {
  if constexpr (FMT == kFmtNvfp4 || FMT == kFmtMxfp4) {
    c.vsc &= live_bytes(live);
  } else if constexpr (FMT == kFmtFp8) {
    const uint32_t m = live_bytes(live);
#pragma unroll
    for (int i = 0; i < 2; ++i) c.vq[i] &= u32x4{m, m, m, m};
  } else {
    const uint32_t m01 = live_bytes(2 * live), m23 = live_bytes(2 * live - 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) c.vq[i] &= u32x4{m01, m23, m01, m23};
  }
}

template <bool F32Q, int FMT>
__device__ __forceinline__ void process_page(PageRegs<FMT> cur, int pg, int L, int kg, float qscale,
                                             const halfx8 qh[4], const halfx8 ql[4], WaveState& st,
                                             int kex, int vex) {
  floatx4 acc_s = qk_page<F32Q, FMT>(cur, qh, ql, kex);
  // ---- softmax (log2 domain); lane holds tokens 4kg..4kg+3 of head col.
  // Only a sequence's last page is partial (uniform test).  qscale > 0, so
  // the max is taken on the raw products and scaled once.
  if ((pg + 1) * kPage > L) {
    const int tbase = pg * kPage + kg * 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc_s[r] = (tbase + r < L) ? acc_s[r] : -INFINITY;
    drop_v<FMT>(cur, L - tbase);
  }
  // A head's page max passes the reference by more than kLazy exactly when
  // one of its four lane rows does, so the cross-row max is taken only on
  // that (rare) path.  The NaN-propagating maximum needs no quieting of the
  // accumulator values first.
  const float lmx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(acc_s[0], acc_s[1]),
                                                  __builtin_elementwise_maximum(acc_s[2], acc_s[3]));
  if (__any(lmx * qscale > st.m_run + kLazy)) {
    const float mx = max_across_rows(lmx) * qscale;
    const bool grow = mx > st.m_run + kLazy;
    const float m_new = grow ? mx : st.m_run;
    const float alpha = fast_exp2(st.m_run - m_new);
    st.m_run = m_new;
    if constexpr (kSumOnMatrixCore<FMT>) st.acc_l *= alpha;
    else st.l_run *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc_o[i] *= alpha;
  }
  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(fmaf(acc_s[r], qscale, -st.m_run));
  if constexpr (!kSumOnMatrixCore<FMT>) st.l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  if constexpr (FMT == kFmtNvfp4 || FMT == kFmtMxfp4) {
    const halfx4 bp = {(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};
    st.acc_l = __builtin_amdgcn_mfma_f32_16x16x16f16(halfx4{1.0f16, 1.0f16, 1.0f16, 1.0f16}, bp, st.acc_l, 0, 0, 0);
    // ---- O^T += V~^T P^T: one 16-token MFMA per element of the lane's
    // d run; P^T comes straight from the S^T accumulator layout
    halfx2 v01, v23;
    v_scales<FMT>(cur, vex, v01, v23);
    auto tile = [&](halfx4 a, floatx4& acc) { acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a, bp, acc, 0, 0, 0); };
    tile(v_column<0, 0>(cur, v01, v23), st.acc_o[0]);
    tile(v_column<1, 0>(cur, v01, v23), st.acc_o[1]);
    tile(v_column<2, 0>(cur, v01, v23), st.acc_o[2]);
    tile(v_column<3, 0>(cur, v01, v23), st.acc_o[3]);
    tile(v_column<0, 1>(cur, v01, v23), st.acc_o[4]);
    tile(v_column<1, 1>(cur, v01, v23), st.acc_o[5]);
    tile(v_column<2, 1>(cur, v01, v23), st.acc_o[6]);
    tile(v_column<3, 1>(cur, v01, v23), st.acc_o[7]);
  } else if constexpr (FMT == kFmtFp8) {
    // ---- O^T += V~^T P^T: word i holds element d = 8 col + i of the four
    // tokens of quad kg (the A operand's k order)
    const halfx4 bp = {(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = cur.vq[i >> 2][i & 3];
      const halfx2 lo = e4m3x2_to_half(w, false), hi = e4m3x2_to_half(w, true);
      const halfx4 a = {lo[0], lo[1], hi[0], hi[1]};
      st.acc_o[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, bp, st.acc_o[i], 0, 0, 0);
    }
  } else {
    // ---- BF16: P = hi + lo in two bf16 parts (16 significant bits, as
    // close as FP16's P; one bf16 part alone moves outputs by up to 2^-9 of
    // the weighted |v|); element d = 8 col + i of the four tokens of quad kg
    // sits in 8 bytes
    shortx4 bh, bl;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bh[r] = bf16_bits(pr[r]);
      bl[r] = bf16_bits(pr[r] - __builtin_bit_cast(float, (uint32_t)(uint16_t)bh[r] << 16));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w0 = cur.vq[i >> 1][(2 * i) & 3], w1 = cur.vq[i >> 1][(2 * i + 1) & 3];
      const shortx4 a = {(short)(w0 & 0xFFFFu), (short)(w0 >> 16), (short)(w1 & 0xFFFFu), (short)(w1 >> 16)};
      st.acc_o[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bh, st.acc_o[i], 0, 0, 0);
      st.acc_o[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bl, st.acc_o[i], 0, 0, 0);
    }
  }
}

// A lane's raw query bits (32 elements: FP32 or bf16), loaded apart from
// their conversion so that a load can be issued ahead of its use.
template <bool F32Q>
struct QRaw {
  uint4 w[F32Q ? 8 : 4];
};

template <bool F32Q>
__device__ __forceinline__ QRaw<F32Q> fetch_q(const DecodeArgs& p, int b, int kvh, int col, int kg) {
  QRaw<F32Q> r;
  if (col < p.group) {
    const size_t qoff = ((size_t)b * p.hq + kvh * p.group + col) * kD + kg * 32;
    const uint4* src = F32Q ? reinterpret_cast<const uint4*>(static_cast<const float*>(p.q) + qoff)
                            : reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + qoff);
#pragma unroll
    for (int i = 0; i < (F32Q ? 8 : 4); ++i) r.w[i] = src[i];
  } else {
#pragma unroll
    for (int i = 0; i < (F32Q ? 8 : 4); ++i) r.w[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  return r;
}

// Q of (sequence b, KV head kvh) as the B operand of S^T = K~ Q^T: lane
// (head col, group kg) holds q[32kg + 8i + j] in element j of qh[i], scaled by
// 2^shift into FP16 (the max |q| of the head lands in [2^14, 2^15)).
template <bool F32Q, int FMT>
__device__ __forceinline__ void convert_q(const DecodeArgs& p, const QRaw<F32Q>& r, int kg,
                                          halfx8 qh[4], halfx8 ql[4], float& qscale) {
  float qv[32];
  if (F32Q) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 v = r.w[i];
      qv[4 * i] = __uint_as_float(v.x); qv[4 * i + 1] = __uint_as_float(v.y);
      qv[4 * i + 2] = __uint_as_float(v.z); qv[4 * i + 3] = __uint_as_float(v.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = r.w[i];
      qv[8 * i + 0] = bf16_lo(v.x); qv[8 * i + 1] = bf16_hi(v.x);
      qv[8 * i + 2] = bf16_lo(v.y); qv[8 * i + 3] = bf16_hi(v.y);
      qv[8 * i + 4] = bf16_lo(v.z); qv[8 * i + 5] = bf16_hi(v.z);
      qv[8 * i + 6] = bf16_lo(v.w); qv[8 * i + 7] = bf16_hi(v.w);
    }
  }
  if constexpr (FMT == kFmtBf16) {
    // bf16 operands (bit patterns in the half registers): q = hi + lo, with
    // lo = 0 for bf16 queries; no range scaling (bf16 spans FP32's range)
    qscale = p.qk_scale;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = qv[8 * i + j];
        const uint16_t hb = (uint16_t)bf16_bits(v);
        qh[i][j] = __builtin_bit_cast(_Float16, hb);
        const float hv = __builtin_bit_cast(float, (uint32_t)hb << 16);
        ql[i][j] = F32Q ? __builtin_bit_cast(_Float16, (uint16_t)bf16_bits(v - hv)) : (_Float16)0.0f;
      }
    return;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(qv[i]));
  amax = max_across_rows(amax);
  int shift = amax > 0.0f ? 14 - ilogbf(amax) : 0;
  shift = max(-120, min(120, shift));
  qscale = p.qk_scale * ldexpf(1.0f, -shift);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = ldexpf(qv[8 * i + j], shift);
      const _Float16 hv = (_Float16)v;
      qh[i][j] = hv;
      ql[i][j] = F32Q ? (_Float16)(v - (float)hv) : (_Float16)0.0f;
    }
  }
}

template <bool F32Q, int FMT>
__device__ __forceinline__ void load_q(const DecodeArgs& p, int b, int kvh, int col, int kg,
                                       halfx8 qh[4], halfx8 ql[4], float& qscale) {
  convert_q<F32Q, FMT>(p, fetch_q<F32Q>(p, b, kvh, col, kg), kg, qh, ql, qscale);
}

// Write the state of (b, kvh): the final output when the piece is the whole
// segment, else a normalized partial (o / l, log2-sum-exp) in workspace slot
// (wave, slot).
template <int FMT>
__device__ __forceinline__ void flush(const DecodeArgs& p, const WaveState& st, int b, int kvh,
                                      int col, int kg, bool complete, int wave, int slot) {
  const float l_tot = kSumOnMatrixCore<FMT> ? st.acc_l[0] : sum_across_rows(st.l_run);
  if (col >= p.group) return;
  float* dst;
  float f;
  if (complete) {
    dst = p.out + ((size_t)b * p.hq + kvh * p.group + col) * kD;
    f = l_tot > 0.0f ? p.v_scale / l_tot : 0.0f;
  } else {
    const size_t piece = ((size_t)wave * 2 + slot) * p.group + col;
    dst = p.ws_o + piece * kD;
    f = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (kg == 0) p.ws_lse[piece] = l_tot > 0.0f ? st.m_run + log2f(l_tot) : -INFINITY;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[8 * (4 * kg + r) + i] = st.acc_o[i][r] * f;
}

__device__ __forceinline__ int pages_of(int len) { return (len + kPage - 1) / kPage; }

// Sequence length clamped to what its page-table row can hold, so that a
// length outside the documented range never reads past the row.
__device__ __forceinline__ int seq_len(const DecodeArgs& p, int b) {
  return min(max(p.seq_lens[b], 0), p.max_pages * kPage);
}

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  return v;
}

// Position in the (sequence, KV head, page) order: the segment (b, kvh) of a
// sequence of length L with np pages, and page pg inside it.  All fields are
// wave-uniform.
struct SegPos {
  int b, kvh, L, np, pg;
};

// Wave-uniform reads of the page table and the sequence lengths go through
// the scalar data cache: scalar loads are counted apart from vector memory,
// so waiting for one never waits for the page loads in flight (vector loads
// complete in order under one counter, and a vector load read soon after its
// issue would hold up every page behind it).  Both arrays are read-only here.
typedef __attribute__((address_space(4))) const int32_t ConstI32;

__device__ __forceinline__ int32_t scalar_load(const int32_t* base, size_t i) {
  return ((const ConstI32*)base)[i];
}

__device__ __forceinline__ int seq_len_uniform(const DecodeArgs& p, int b) {
  return min(max(scalar_load(p.seq_lens, (size_t)b), 0), p.max_pages * kPage);
}

__device__ __forceinline__ uint32_t page_id_uniform(const DecodeArgs& p, const SegPos& s) {
  return (uint32_t)scalar_load(p.page_table, (size_t)s.b * p.max_pages + s.pg);
}

// Move to the first page of the next non-empty segment.  The caller knows
// that one exists (a unit of the wave's range lies beyond).
__device__ __forceinline__ void next_segment(const DecodeArgs& p, SegPos& s) {
  s.pg = 0;
  if (++s.kvh == p.hkv) {
    s.kvh = 0;
    do {
      ++s.b;
      s.L = seq_len_uniform(p, s.b);
      s.np = pages_of(s.L);
    } while (s.np == 0);
  }
}

// Wave ranges.  The ranges follow each other in the stream in the order of
// a range index v; range v takes the units [start(v), start(v + 1)) with
//   start(v) = floor(U S(v) / S(V)),
// S the sum of the weights of the ranges before v.  Two patterns:
//   - by rounds: v = w, the first R ranges weigh A and the rest B
//     (A = B: equal ranges);
//   - interleaved (K > 0, 3K waves): waves w < K, K <= w < 2K and w >= 2K
//     (the static rounds and the tail ranges, dispatched in that order) take
//     v = 3(w mod K) + class, with weights A, B and C by class, so that the
//     small tail ranges lie spread over the whole stream.
// The range owning unit u is the largest v with start(v) <= u, which is the
// largest v with S(v) <= floor(((u + 1) S(V) - 1) / U) (S grows strictly).
// I is uint32_t when every product stays below 2^32 (the usual case: 64-bit
// division is a long software sequence), else int64_t.
template <typename I>
struct RangeMath {
  I U, T;                                  // units; T = S(V)
  int R, A, B, C, K;
  __device__ I S(int v) const {
    if (K > 0) {
      const int j = v % 3;
      return (I)(v / 3) * (I)(A + B + C) + (I)(j >= 1 ? A : 0) + (I)(j >= 2 ? B : 0);
    }
    return (I)A * (I)min(v, R) + (I)B * (I)max(0, v - R);
  }
  __device__ long long start(int v) const { return (long long)((I)((I)U * S(v)) / T); }
  __device__ int owner(long long u) const {
    const I smax = (I)((I)(u + 1) * T - 1) / U;
    if (K > 0) {
      const I P = (I)(A + B + C), r = smax % P;
      return 3 * (int)(smax / P) + (r < (I)A ? 0 : (r < (I)(A + B) ? 1 : 2));
    }
    const I ar = (I)A * (I)R;
    return smax < ar ? (int)(smax / (I)A) : R + (int)((smax - ar) / (I)B);
  }
  __device__ int v_of(int w) const { return K > 0 ? 3 * (w % K) + w / K : w; }
  __device__ int w_of(int v) const { return K > 0 ? (v % 3) * K + v / 3 : v; }
};

template <typename I>
__device__ __forceinline__ RangeMath<I> range_math(const DecodeArgs& p, long long U) {
  RangeMath<I> rm;
  rm.U = (I)U;
  rm.R = p.first_waves;
  rm.A = p.weight_first;
  rm.B = p.weight_rest;
  rm.C = p.weight_tail;
  rm.K = p.tail_start < p.num_splits ? p.first_waves : 0;
  rm.T = rm.S(rm.K > 0 ? 3 * rm.K : p.num_splits);
  return rm;
}

// Every product of the range arithmetic is at most U S(W).
__device__ __forceinline__ bool range_fits_u32(const DecodeArgs& p, long long U) {
  const long long T = p.tail_start < p.num_splits
                          ? (long long)(p.weight_first + p.weight_rest + p.weight_tail) * p.first_waves
                          : (long long)p.weight_first * p.first_waves +
                                (long long)p.weight_rest * (p.num_splits - p.first_waves);
  return U * T < (1LL << 32);
}

// Register stages of the page pipeline; the planner runs two waves per SIMD,
// so the register budget is that of two waves (a BF16 page takes three times
// the registers of an NVFP4 one).  With two waves on every SIMD the 4-bit
// formats take kShallow stages (four pages in flight per wave): against eight
// stages the configuration-4 call ran ~1 % faster (median and p10 over four
// interleaved runs on MI355X), while a lone wave per SIMD (small batches)
// keeps the deeper pipeline (configuration 3 ran ~1.5 % slower shallow).
template <int FMT> constexpr int kDepth = FMT == kFmtBf16 ? 4 : 8;
constexpr int kShallow = 5;

// PROBE: the page-gather ceiling of this kernel's access pattern.  The same
// wave ranges, page walk and page loads, but every page is consumed by an
// exclusive or instead of the attention math; nothing is written but one
// word per wave (p.out), and no merge follows.
template <bool F32Q, int FMT, bool WIDE, bool PROBE = false, int DEPTH = kDepth<FMT>>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) decode_kernel(DecodeArgs p) {
  constexpr int kD8 = DEPTH;
  const int lane = threadIdx.x;
  const int col = lane & 15, kg = lane >> 4;
  const int wave = blockIdx.x, W = gridDim.x;
  const int Hkv = p.hkv, B = p.batch;

  // ---- total work U = Hkv * sum_b pages(b), and (wave 0) the page prefix
  // sums for merge_kernel.  The page counts of the first kHeld * 64
  // sequences and their in-chunk prefix sums stay in registers: their
  // lengths are loaded together, so both passes below cost one memory round
  // trip for batches up to that size (the rest is read a chunk at a time).
  // (Lanes past the batch read the last length, B >= 1 here, and drop it.)
  constexpr int kHeld = 4;
  int np_h[kHeld], incl_h[kHeld];
#pragma unroll
  for (int i = 0; i < kHeld; ++i) np_h[i] = p.seq_lens[min(64 * i + lane, B - 1)];
#pragma unroll
  for (int i = 0; i < kHeld; ++i) {
    const int b = 64 * i + lane;
    np_h[i] = b < B ? pages_of(min(max(np_h[i], 0), p.max_pages * kPage)) : 0;
  }
  int total_pages = 0;
#pragma unroll
  for (int i = 0; i < kHeld; ++i) {
    const int b = 64 * i + lane;
    incl_h[i] = wave_scan(np_h[i], lane);
    if (!PROBE && wave == 0 && b < B) p.ws_prefix[b] = total_pages + incl_h[i] - np_h[i];
    total_pages += __builtin_amdgcn_readlane(incl_h[i], 63);
  }
  for (int c = 64 * kHeld; c < B; c += 64) {
    const int b = c + lane;
    const int np = b < B ? pages_of(seq_len(p, b)) : 0;
    const int incl = wave_scan(np, lane);
    if (!PROBE && wave == 0 && b < B) p.ws_prefix[b] = total_pages + incl - np;
    total_pages += __builtin_amdgcn_readlane(incl, 63);
  }
  if (!PROBE && wave == 0 && lane == 0) p.ws_prefix[B] = total_pages;
  const long long U = (long long)total_pages * Hkv;
  long long u0, u1;
  if (range_fits_u32(p, U)) {
    const RangeMath<uint32_t> rm = range_math<uint32_t>(p, U);
    u0 = rm.start(rm.v_of(wave));
    u1 = rm.start(rm.v_of(wave) + 1);
  } else {
    const RangeMath<long long> rm = range_math<long long>(p, U);
    u0 = rm.start(rm.v_of(wave));
    u1 = rm.start(rm.v_of(wave) + 1);
  }
  if (u0 >= u1) {                          // no units (more waves than units)
    if constexpr (PROBE) reinterpret_cast<uint32_t*>(p.out)[wave * 64 + lane] = 0u;
    return;
  }
  const int N = (int)(u1 - u0);            // units of this wave

  // ---- the segment holding u0: sequence b0 (first sequence whose prefix
  // passes u0), KV head and page inside it
  int b0 = 0;
  long long a_b0 = 0;
  {
    int carry = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < kHeld; ++i) {
      if (!found) {
        const int b = 64 * i + lane;
        const unsigned long long hit = __ballot(b < B && (long long)(carry + incl_h[i]) * Hkv > u0);
        if (hit) {
          const int idx = __ffsll((long long)hit) - 1;
          b0 = 64 * i + idx;
          a_b0 = (long long)(carry + __builtin_amdgcn_readlane(incl_h[i] - np_h[i], idx)) * Hkv;
          found = true;
        } else {
          carry += __builtin_amdgcn_readlane(incl_h[i], 63);
        }
      }
    }
    for (int c = 64 * kHeld; !found && c < B; c += 64) {
      const int b = c + lane;
      const int np = b < B ? pages_of(seq_len(p, b)) : 0;
      const int incl = wave_scan(np, lane);
      const unsigned long long hit = __ballot(b < B && (long long)(carry + incl) * Hkv > u0);
      if (hit) {
        const int idx = __ffsll((long long)hit) - 1;
        b0 = c + idx;
        a_b0 = (long long)(carry + __builtin_amdgcn_readlane(incl - np, idx)) * Hkv;
        found = true;
      } else {
        carry += __builtin_amdgcn_readlane(incl, 63);
      }
    }
  }
  SegPos start;
  start.b = __builtin_amdgcn_readfirstlane(b0);
  start.L = seq_len_uniform(p, start.b);
  start.np = pages_of(start.L);
  {
    const long long off0 = u0 - a_b0;
    start.kvh = (int)(off0 / start.np);
    start.pg = (int)(off0 % start.np);
  }

  // ---- issue side: the wave's units form one stream of pages; `iw` is
  // the unit issued next and `ipage` its page id, read one issue ahead
  SegPos iw = start;
  const ConstI32* irow = (const ConstI32*)p.page_table + (size_t)iw.b * p.max_pages;
  uint32_t ipage = (uint32_t)irow[iw.pg];
  int issued = 0;
  const LaneOffsets lo = lane_offsets<FMT>(col, kg);
  const PlaneRsrc pr = plane_rsrc<FMT>(p);
  // units past the end reload the last one (never consumed).  A page id
  // beyond the cache is clamped to its last slab, so a bad page table reads
  // wrong data but never outside the planes.
  auto issue = [&](PageRegs<FMT>& r) {
    const uint32_t slab = min(ipage * (uint32_t)Hkv + (uint32_t)iw.kvh, p.num_slabs - 1u);
    load_page<FMT, WIDE>(p, pr, slab, lo, r);
    if (issued + 1 < N) {
      ++issued;
      if (++iw.pg == iw.np) {
        next_segment(p, iw);
        irow = (const ConstI32*)p.page_table + (size_t)iw.b * p.max_pages;
      }
      ipage = (uint32_t)irow[iw.pg];
    }
  };

  // ---- process side: one piece (the wave's part of one segment) at a time
  SegPos seg = start;
  int piece_left = 0;                      // pages of the current piece still to process
  bool whole = false, first_piece = true, started = false;
  int done = 0;                            // units processed
  halfx8 qh[4], ql[4];
  float qscale = 0.0f;
  QRaw<F32Q> q_first;
  WaveState st;
  uint32_t probe_sink = 0;
  auto step = [&](const PageRegs<FMT>& r) {
    if constexpr (PROBE) {
      if constexpr (FMT == kFmtNvfp4)
        probe_sink ^= r.kq.x ^ r.kq.y ^ r.kq.z ^ r.kq.w ^ r.vq.x ^ r.vq.y ^ r.vq.z ^ r.vq.w ^ r.ksc ^ r.vsc;
      return;
    }
    if (piece_left == 0) {                 // a new piece starts with this page
      if (started) next_segment(p, seg);
      started = true;
      piece_left = min(seg.np - seg.pg, N - done);
      whole = seg.pg == 0 && piece_left == seg.np;
      if (first_piece) convert_q<F32Q, FMT>(p, q_first, kg, qh, ql, qscale);
      else load_q<F32Q, FMT>(p, seg.b, seg.kvh, col, kg, qh, ql, qscale);
      reset_state(st);
    }
    process_page<F32Q, FMT>(r, seg.pg, seg.L, kg, qscale, qh, ql, st, p.k_exp, p.v_exp);
    ++seg.pg;
    ++done;
    if (--piece_left == 0) {
      flush<FMT>(p, st, seg.b, seg.kvh, col, kg, whole, wave, first_piece ? 0 : 1);
      first_piece = false;
    }
  };

  // kD8 register stages: the loads of the next kD8 - 1 pages are in
  // flight while a page is processed.  The barriers keep the first loads in
  // stream order: the compiler derives the loop's waits from that order too,
  // and a reordered start makes every iteration wait for all but the newest
  // page.
  PageRegs<FMT> r[kD8];
  // Every stage issues, also past the end of the range (reloads of the last
  // unit), and only the loop's latch exits: every path around the back edge
  // then carries a whole iteration of page loads, which the compiler's waits
  // rely on (an exit in the middle, however rare, gives it a short path).
  // the first piece's queries load ahead of the first pages: its start then
  // waits for nothing the first page does not (a query load issued at the
  // piece start waits behind every page load in flight)
  if constexpr (!PROBE) q_first = fetch_q<F32Q>(p, start.b, start.kvh, col, kg);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kD8 - 1; ++i) {
    issue(r[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int t = 0; t < N; t += kD8) {
#pragma unroll
    for (int j = 0; j < kD8; ++j) {
      issue(r[(j + kD8 - 1) % kD8]);
      __builtin_amdgcn_sched_barrier(0);
      if (t + j < N) step(r[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (PROBE) reinterpret_cast<uint32_t*>(p.out)[wave * 64 + lane] = probe_sink;
}

// A segment cut by wave ranges is combined from its pieces:
//   o = sum_w 2^(lse_w - M) o_w / sum_w 2^(lse_w - M), times s_tV.
// The waves holding the segment's first and last units come from the same
// range arithmetic as the decode kernel (RangeMath); the piece of wave w sits
// in slot 0 when w's range starts inside the segment, else in slot 1.  Waves
// between the first and the last owner with an empty range (W > U) wrote
// nothing and are skipped.
// A query head's thread (i, e) = (tid / 32, tid % 32) takes pieces i,
// i + PL, ... and output elements 4e .. 4e + 3, so all partial loads are
// independent; the PL piece lanes are combined in LDS.  PL = 32 or 8 when
// segments have many pieces (few long sequences; more than 64 or 8 on
// average): one workgroup per query head, so that its loop over the pieces
// stays a few steps long.  Else
// PL = 2 and one workgroup holds the G query heads of a segment, 64 threads
// each (a quarter of the workgroups of one per head: their launch, not the
// merging, dominated the kernel's time).
constexpr int kMaxGroup = 16;   // query heads per KV head the decode accepts

template <int PL, bool PER_SEG, typename I>
__device__ __forceinline__ void merge_segment(const DecodeArgs& p, const RangeMath<I> rm, long long a,
                                              long long end, int g, int tid, float* out);


template <int PL, bool PER_SEG>
__global__ void __launch_bounds__(PER_SEG ? 64 * kMaxGroup : 32 * PL) merge_kernel(DecodeArgs p) {
  const int g = PER_SEG ? (int)(threadIdx.x / (32 * PL)) : (int)(blockIdx.x % p.group);
  const int seg = PER_SEG ? (int)blockIdx.x : (int)(blockIdx.x / p.group);
  const int tid = (int)(threadIdx.x % (32 * PL));
  const int b = seg / p.hkv, kvh = seg % p.hkv;
  const int pb = p.ws_prefix[b], np = p.ws_prefix[b + 1] - pb;
  const long long U = (long long)p.ws_prefix[p.batch] * p.hkv;
  float* out = p.out + ((size_t)b * p.hq + (size_t)kvh * p.group + g) * kD;
  if (np == 0) {
    if (tid < 32) reinterpret_cast<float4*>(out)[tid] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    return;
  }
  const long long a = (long long)pb * p.hkv + (long long)kvh * np;
  if (range_fits_u32(p, U))
    merge_segment<PL, PER_SEG>(p, range_math<uint32_t>(p, U), a, a + np, g, tid, out);
  else
    merge_segment<PL, PER_SEG>(p, range_math<long long>(p, U), a, a + np, g, tid, out);
}

// The exits before the workgroup barrier (empty sequence, a segment finished
// by one wave) depend only on the segment, so every head of a workgroup
// takes them together.
template <int PL, bool PER_SEG, typename I>
__device__ __forceinline__ void merge_segment(const DecodeArgs& p, const RangeMath<I> rm, long long a,
                                              long long end, int g, int tid, float* out) {
  const int pi = tid >> 5, e = tid & 31;
  const int G = p.group;
  const int v0 = rm.owner(a);
  const int v1 = rm.owner(end - 1);
  if (v0 == v1) return;                       // finished by one wave
  const int n = v1 - v0 + 1;
  // the piece of range v0 + i: its workspace index (that of the range's
  // wave), or -1 when the range is empty
  auto piece = [&](int i) -> int {
    const int v = v0 + i;
    const long long sv = rm.start(v);
    if (sv == rm.start(v + 1)) return -1;
    const int slot = sv >= a ? 0 : 1;
    return (rm.w_of(v) * 2 + slot) * G + g;
  };
  // each thread merges its pieces online (running max m, rescaling as it
  // grows); the 8 piece lanes are then combined once
  __shared__ float4 s_acc_h[PER_SEG ? kMaxGroup : 1][PL][32];
  __shared__ float s_m_h[PER_SEG ? kMaxGroup : 1][PL], s_den_h[PER_SEG ? kMaxGroup : 1][PL];
  float4 (&s_acc)[PL][32] = s_acc_h[PER_SEG ? g : 0];
  float (&s_m)[PL] = s_m_h[PER_SEG ? g : 0];
  float (&s_den)[PL] = s_den_h[PER_SEG ? g : 0];
  float m = -INFINITY, den = 0.0f;
  float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // The thread's pieces i = pi, pi + PL, ... in batches of kBatch whose loads
  // are all issued before the first is used (one memory round trip per
  // batch); a slot without a piece loads the segment's first piece, which
  // always exists (wave w0 owns the segment's first unit), and is skipped.
  constexpr int kBatch = 4;
  const int k0 = piece(0);
  for (int i0 = pi; i0 < n; i0 += kBatch * PL) {
    int ks[kBatch];
    float ls[kBatch];
    float4 vs[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * PL;
      ks[u] = i < n ? piece(i) : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int k = ks[u] >= 0 ? ks[u] : k0;
      ls[u] = p.ws_lse[k];
      vs[u] = reinterpret_cast<const float4*>(p.ws_o + (size_t)k * kD)[e];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float l = ls[u];
      if (ks[u] < 0 || l == -INFINITY) continue;   // no piece, or a piece with no weight
      if (l > m) {
        const float r = exp2f(m - l);           // 0 while m is -inf
        acc.x *= r; acc.y *= r; acc.z *= r; acc.w *= r;
        den *= r;
        m = l;
      }
      const float c = exp2f(l - m);
      acc.x = fmaf(c, vs[u].x, acc.x);
      acc.y = fmaf(c, vs[u].y, acc.y);
      acc.z = fmaf(c, vs[u].z, acc.z);
      acc.w = fmaf(c, vs[u].w, acc.w);
      den += c;
    }
  }
  s_acc[pi][e] = acc;
  if (e == 0) {
    s_m[pi] = m;
    s_den[pi] = den;
  }
  __syncthreads();
  if (tid < 32) {
    float M = s_m[0];
#pragma unroll
    for (int j = 1; j < PL; ++j) M = fmaxf(M, s_m[j]);
    float4 t = {0.0f, 0.0f, 0.0f, 0.0f};
    float d = 0.0f;
    if (M > -INFINITY) {
#pragma unroll
      for (int j = 0; j < PL; ++j) {
        if (s_m[j] == -INFINITY) continue;
        const float f = exp2f(s_m[j] - M);
        const float4 u = s_acc[j][tid];
        t.x = fmaf(f, u.x, t.x);
        t.y = fmaf(f, u.y, t.y);
        t.z = fmaf(f, u.z, t.z);
        t.w = fmaf(f, u.w, t.w);
        d = fmaf(f, s_den[j], d);
      }
    }
    const float f = d > 0.0f ? p.v_scale / d : 0.0f;
    reinterpret_cast<float4*>(out)[tid] = make_float4(t.x * f, t.y * f, t.z * f, t.w * f);
  }
}

// Resident decode waves per CU, queried once per process (every device here
// is gfx950, so the answer does not depend on the device).
template <int FMT>
static int occupancy_of(bool f32_q) {
  int n = 0;
  hipError_t e = f32_q ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<true, FMT, false>, 64, 0)
                       : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<false, FMT, false>, 64, 0);
  return e == hipSuccess ? n : 0;
}

int decode_occupancy(bool f32_q, int fmt) {
  static std::atomic<int> cached[2][4] = {};
  const int f = fmt == kFmtFp8 ? 1 : fmt == kFmtBf16 ? 2 : fmt == kFmtMxfp4 ? 3 : 0;
  int n = cached[f32_q][f].load(std::memory_order_relaxed);
  if (n > 0) return n;
  n = f == 1 ? occupancy_of<kFmtFp8>(f32_q)
      : f == 2 ? occupancy_of<kFmtBf16>(f32_q)
      : f == 3 ? occupancy_of<kFmtMxfp4>(f32_q) : occupancy_of<kFmtNvfp4>(f32_q);
  if (n <= 0) return 8;
  cached[f32_q][f].store(n, std::memory_order_relaxed);
  return n;
}

// Planes whose bytes exceed 32-bit offsets take the kernel that builds a
// buffer resource at each slab's base.
template <int FMT>
static bool wide_planes(uint32_t num_slabs) {
  using SB = SlabBytes<FMT>;
  const uint64_t m = SB::k > SB::ks ? SB::k : SB::ks;
  return (uint64_t)num_slabs * m > 0x7FFFFFFFull;
}

template <int FMT, int DEPTH>
static void launch_depth(const DecodeArgs& a, bool f32_q, hipStream_t s) {
  const bool wide = wide_planes<FMT>(a.num_slabs);
  if (f32_q) {
    if (wide) decode_kernel<true, FMT, true, false, DEPTH><<<a.num_splits, 64, 0, s>>>(a);
    else decode_kernel<true, FMT, false, false, DEPTH><<<a.num_splits, 64, 0, s>>>(a);
  } else {
    if (wide) decode_kernel<false, FMT, true, false, DEPTH><<<a.num_splits, 64, 0, s>>>(a);
    else decode_kernel<false, FMT, false, false, DEPTH><<<a.num_splits, 64, 0, s>>>(a);
  }
}

template <int FMT>
static void launch_fmt(const DecodeArgs& a, bool f32_q, hipStream_t s) {
  if constexpr (FMT == kFmtNvfp4 || FMT == kFmtMxfp4) {
    if (a.shallow) {
      launch_depth<FMT, kShallow>(a, f32_q, s);
      return;
    }
  }
  launch_depth<FMT, kDepth<FMT>>(a, f32_q, s);
}

hipError_t launch_gather_probe(const DecodeArgs& a, hipStream_t s) {
  if (wide_planes<kFmtNvfp4>(a.num_slabs)) return hipErrorInvalidValue;
  if (a.shallow) decode_kernel<false, kFmtNvfp4, false, true, kShallow><<<a.num_splits, 64, 0, s>>>(a);
  else decode_kernel<false, kFmtNvfp4, false, true><<<a.num_splits, 64, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, bool f32_q, int fmt, hipStream_t s) {
  if (fmt == kFmtFp8) launch_fmt<kFmtFp8>(a, f32_q, s);
  else if (fmt == kFmtBf16) launch_fmt<kFmtBf16>(a, f32_q, s);
  else if (fmt == kFmtMxfp4) launch_fmt<kFmtMxfp4>(a, f32_q, s);
  else launch_fmt<kFmtNvfp4>(a, f32_q, s);
  const unsigned heads = (unsigned)(a.batch * a.hkv * a.group);
  const long long segs = (long long)a.batch * a.hkv;
  if (a.num_splits > 64 * segs) merge_kernel<32, false><<<heads, 1024, 0, s>>>(a);
  else if (a.num_splits > 8 * segs) merge_kernel<8, false><<<heads, 256, 0, s>>>(a);
  else merge_kernel<2, true><<<(unsigned)segs, 64 * a.group, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace nvfp4
