// decode.hip -- decode attention over the paged NVFP4 cache, split over the
// context, plus the log-sum-exp merge of the splits.
//
// The cache is dequantized in registers right before the QK^T and PV
// products ("NVIDIA解説: NVFP4 KV Cacheで長コンテキストLLM推論を最適化",
// section 量子化・逆量子化フロー); softmax and accumulation run in FP32.
//
// Work decomposition: grid (split, kv head, sequence); a 256-thread
// workgroup (4 wave64s) owns one split of one (sequence, kv head) and its
// waves take every 4th page of the split.  Per page (16 tokens):
//   * K: lane (t = lane%16, c = lane/16) loads 16 bytes = elements
//     32c..32c+31 of token t (one coalesced 1 KiB wave load) and 2 block
//     scales; the nibbles expand to halves e2m1 * s_block (exact in FP16:
//     at most 6 significant bits, magnitudes 2^-10 .. 2688), and four
//     16x16x32 f16 MFMAs give S^T[token][head] for the G query heads of the
//     KV head (columns >= G are zero padding).  The contraction index order
//     is permuted identically on the Q side, which is loaded once.
//   * softmax: lane holds 4 tokens of one head; the page max reduces across
//     the 4 lane rows with permlane swaps; running max / sum in FP32 (log2).
//   * V: the cache stores V 4-token-interleaved so lane (m = lane%16, c)
//     loads 16 bytes = bytes 4m..4m+3 of tokens 4c..4c+3; a bit-field
//     transpose pairs the nibbles of 2 tokens per byte, which expand to the
//     A operand of eight 16x16x16 f16 MFMAs O^T[d][head] += V^T P^T with
//     d = 8m + tile.  P^T comes straight from the S^T accumulator layout.
// The 4 waves merge in LDS; with one split the workgroup writes the output,
// otherwise a normalized partial and its log2-sum-exp go to the workspace
// and merge_kernel combines them.
#include "common.h"
#include "internal.h"

namespace nvfp4 {

struct PageRegs {
  u32x4 kq;       // K codes: 32 nibbles of token lane%16
  u32x4 vq;       // V codes: 4 tokens x 8 nibbles
  uint32_t ksc;   // 2 K block scales (low 16 bits)
  uint32_t vsc;   // 4 V block scales
};

__device__ __forceinline__ void load_page(const DecodeArgs& p, int pid, int kvh, int col, int kg,
                                          PageRegs& r) {
  const size_t slab = (size_t)pid * p.hkv + kvh;
  r.kq = *reinterpret_cast<const u32x4*>(p.k_codes + slab * kSlab + col * 64 + kg * 16);
  r.ksc = *reinterpret_cast<const uint16_t*>(p.k_scales + slab * kScaleSlab + col * kNBlk + kg * 2);
  r.vq = *reinterpret_cast<const u32x4*>(p.v_codes + slab * kSlab + kg * 256 + col * 16);
  r.vsc = *reinterpret_cast<const uint32_t*>(p.v_scales + slab * kScaleSlab + (col >> 1) * kPage + kg * 4);
}

template <bool F32Q>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs p) {
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int G = p.group;
  const int L = p.seq_lens[b];
  const int npages = (L + kPage - 1) / kPage;
  const int pstart = split * p.pages_per_split;
  const int pend = min(npages, pstart + p.pages_per_split);
  const int S = p.num_splits;

  if (pstart >= pend) {       // nothing of this sequence falls in the split
    if (S > 1) {
      for (int idx = threadIdx.x; idx < G * kD; idx += 256) {
        const int g = idx / kD, d = idx % kD;
        const size_t bh = (size_t)b * p.hq + kvh * G + g;
        p.ws_o[(bh * S + split) * kD + d] = 0.0f;
        if (d == 0) p.ws_lse[bh * S + split] = -INFINITY;
      }
    } else {
      for (int idx = threadIdx.x; idx < G * kD; idx += 256) {
        const int g = idx / kD, d = idx % kD;
        p.out[((size_t)b * p.hq + kvh * G + g) * kD + d] = 0.0f;
      }
    }
    return;
  }

  // ---- Q (B operand of S^T = K~ Q^T): lane (head col, group kg) holds
  // q[32kg + 8i + j] in element j of qh[i].  Scaled by 2^shift into FP16.
  halfx8 qh[4], ql[4];
  float qscale = 0.0f;
  {
    float qv[32];
    if (col < G) {
      const size_t qoff = ((size_t)b * p.hq + kvh * G + col) * kD + kg * 32;
      if (F32Q) {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(p.q) + qoff);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float4 v = src[i];
          qv[4 * i] = v.x; qv[4 * i + 1] = v.y; qv[4 * i + 2] = v.z; qv[4 * i + 3] = v.w;
        }
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + qoff);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint4 v = src[i];
          qv[8 * i + 0] = bf16_lo(v.x); qv[8 * i + 1] = bf16_hi(v.x);
          qv[8 * i + 2] = bf16_lo(v.y); qv[8 * i + 3] = bf16_hi(v.y);
          qv[8 * i + 4] = bf16_lo(v.z); qv[8 * i + 5] = bf16_hi(v.z);
          qv[8 * i + 6] = bf16_lo(v.w); qv[8 * i + 7] = bf16_hi(v.w);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) qv[i] = 0.0f;
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
        float v = ldexpf(qv[8 * i + j], shift);
        _Float16 hv = (_Float16)v;
        qh[i][j] = hv;
        if (F32Q) ql[i][j] = (_Float16)(v - (float)hv);
      }
    }
  }

  floatx4 acc_o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc_o[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  const int32_t* pt = p.page_table + (size_t)b * p.max_pages;
  int pg = pstart + wave;
  PageRegs cur;
  if (pg < pend) load_page(p, pt[pg], kvh, col, kg, cur);
  while (pg < pend) {
    const int pgn = pg + 4;
    PageRegs nxt;
    if (pgn < pend) load_page(p, pt[pgn], kvh, col, kg, nxt);

    // ---- S^T = K~ Q^T
    halfx2 ks = e4m3x2_to_half(cur.ksc, false);
    halfx2 sa = {ks[0], ks[0]}, sb = {ks[1], ks[1]};
    floatx4 acc_s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = cur.kq[i];
      const halfx2 sc = i < 2 ? sa : sb;
      halfx2 h0 = e2m1x2_to_half<0>(w) * sc;
      halfx2 h1 = e2m1x2_to_half<1>(w) * sc;
      halfx2 h2 = e2m1x2_to_half<2>(w) * sc;
      halfx2 h3 = e2m1x2_to_half<3>(w) * sc;
      halfx8 a = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
      acc_s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qh[i], acc_s, 0, 0, 0);
      if (F32Q) acc_s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ql[i], acc_s, 0, 0, 0);
    }

    // ---- online softmax (log2 domain); lane holds tokens 4kg..4kg+3 of head col
    const int tbase = pg * kPage + kg * 4;
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = (tbase + r < L) ? acc_s[r] * qscale : -INFINITY;
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = max_across_rows(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = exp2f(s[r] - m_new);
    l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc_o[i] *= alpha;
    halfx4 bp = {(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};

    // ---- O^T += V~^T P^T
    const halfx2 v01 = e4m3x2_to_half(cur.vsc, false);
    const halfx2 v23 = e4m3x2_to_half(cur.vsc, true);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t W = cur.vq[k];
      const uint32_t lo = (W & 0x000F000Fu) | ((W >> 4) & 0x00F000F0u);
      const uint32_t hi = ((W >> 4) & 0x000F000Fu) | ((W >> 8) & 0x00F000F0u);
      halfx2 a0 = e2m1x2_to_half<0>(lo) * v01, a1 = e2m1x2_to_half<2>(lo) * v23;
      halfx2 b0 = e2m1x2_to_half<0>(hi) * v01, b1 = e2m1x2_to_half<2>(hi) * v23;
      halfx4 alo = {a0[0], a0[1], a1[0], a1[1]};
      halfx4 ahi = {b0[0], b0[1], b1[0], b1[1]};
      acc_o[2 * k] = __builtin_amdgcn_mfma_f32_16x16x16f16(alo, bp, acc_o[2 * k], 0, 0, 0);
      acc_o[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(ahi, bp, acc_o[2 * k + 1], 0, 0, 0);
    }
    cur = nxt;
    pg = pgn;
  }

  // ---- merge the 4 waves in LDS
  __shared__ float sm_o[4][16][kD];
  __shared__ float sm_m[4][16], sm_l[4][16];
  const float l_tot = sum_across_rows(l_run);
  if (col < G) {
    if (kg == 0) { sm_m[wave][col] = m_run; sm_l[wave][col] = l_tot; }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm_o[wave][col][8 * (4 * kg + r) + i] = acc_o[i][r];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kD; idx += 256) {
    const int g = idx / kD, d = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][g]);
    float o = 0.0f, l = 0.0f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float c = exp2f(sm_m[w][g] - M);
        o += c * sm_o[w][g][d];
        l += c * sm_l[w][g];
      }
    }
    const size_t bh = (size_t)b * p.hq + kvh * G + g;
    if (S == 1) {
      p.out[bh * kD + d] = l > 0.0f ? o / l * p.v_scale : 0.0f;
    } else {
      p.ws_o[(bh * S + split) * kD + d] = l > 0.0f ? o / l : 0.0f;
      if (d == 0) p.ws_lse[bh * S + split] = l > 0.0f ? M + log2f(l) : -INFINITY;
    }
  }
}

// One workgroup per (sequence, query head); thread d combines the splits:
// o = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), times s_tV.
__global__ void __launch_bounds__(128) merge_kernel(DecodeArgs p) {
  const size_t bh = blockIdx.x;
  const int d = threadIdx.x;
  const int S = p.num_splits;
  const float* lse = p.ws_lse + bh * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, lse[s]);
  float num = 0.0f, den = 0.0f;
  if (M > -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float w = exp2f(lse[s] - M);
      num += w * p.ws_o[(bh * S + s) * kD + d];
      den += w;
    }
  }
  p.out[bh * kD + d] = den > 0.0f ? num / den * p.v_scale : 0.0f;
}

hipError_t launch_decode(const DecodeArgs& a, bool f32_q, hipStream_t s) {
  dim3 grid(a.num_splits, a.hkv, a.batch);
  if (f32_q) decode_kernel<true><<<grid, 256, 0, s>>>(a);
  else decode_kernel<false><<<grid, 256, 0, s>>>(a);
  if (a.num_splits > 1) merge_kernel<<<(unsigned)(a.batch * a.hq), 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace nvfp4
