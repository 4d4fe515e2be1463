// convert.hip -- NVFP4 -> FP8 (E4M3) conversion of a row-major tensor.
//
// "一個 Triton FP8 繞道補丁，為 DGX Spark 的 GB10 擠出多 17% 的 NVFP4 速度"
// (section 這個 80 行的 Triton 繞道): NVFP4 weights are turned into FP8 when
// the model loads so that the GEMM runs on FP8 matrix cores, and the
// dequantization divides by the global scale.  Element value
// e2m1 * s_block (exact in FP32) / g (IEEE division), written as the E4M3
// code of that value / s8 (IEEE division), nearest, ties to even, clamped to
// 448.  The rule is stated in include/nvfp4kv.h.
//
// An element's output depends only on its E2M1 magnitude (8 values), its
// sign and its block scale (127 codes), so each workgroup first fills a
// 1 KiB LDS table of the 128 x 8 magnitude codes (two IEEE divisions per
// entry) and the stream then costs a table row per block and one byte
// permute per four elements: the kernel is bound by HBM (0.5625 bytes in and
// 1 byte out per element), not by the divisions.  Every byte is read or
// written once, so the loads and stores carry the non-temporal hint.
#include "common.h"
#include "internal.h"

namespace nvfp4 {

constexpr int kConvThreads = 256;
constexpr int kPer = 4;           // blocks per lane per step

// Four nibbles (bits 0..15 of x, element j in bits 4j..4j+3) spread to the
// low nibbles of four bytes.
__device__ __forceinline__ uint32_t spread4(uint32_t x) {
  return (x & 0xFu) | ((x & 0xF0u) << 4) | ((x & 0xF00u) << 8) | ((x & 0xF000u) << 12);
}

// FP8 codes of 8 elements (nibbles of w) whose magnitudes index the table
// row (lo: magnitudes 0..3, hi: 4..7); the sign nibble bit becomes bit 7.
__device__ __forceinline__ uint2 convert8(uint32_t w, uint32_t lo, uint32_t hi) {
  const uint32_t a = spread4(w & 0xFFFFu), b = spread4(w >> 16);
  // v_perm_b32: selector byte k (0..7) picks byte k of {hi:lo}
  const uint32_t ra = __builtin_amdgcn_perm(hi, lo, a & 0x07070707u) | ((a & 0x08080808u) << 4);
  const uint32_t rb = __builtin_amdgcn_perm(hi, lo, b & 0x07070707u) | ((b & 0x08080808u) << 4);
  return make_uint2(ra, rb);
}

__global__ void __launch_bounds__(kConvThreads) to_fp8_kernel(ToFp8Args a) {
  __shared__ uint32_t table[128][2];
  uint8_t* tb = reinterpret_cast<uint8_t*>(&table[0][0]);
  for (int i = threadIdx.x; i < 1024; i += kConvThreads) {
    const uint32_t sb = (uint32_t)i >> 3, m = (uint32_t)i & 7u;
    const float e = m < 4u ? 0.5f * (float)m : (m == 7u ? 6.0f : (float)m - 2.0f);
    const float v = e * e4m3_to_float(sb);                   // exact
    const float xh = v / a.g;                                 // divide by the global scale
    const float q = fminf(xh / a.s8, 448.0f);                 // non-negative
    tb[i] = (uint8_t)((uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xFFu);
  }
  __syncthreads();
  // wave w takes blocks [kPer*64*w, kPer*64*(w+1)) of each stride: lane l
  // converts blocks base + 64j + l, so every load and store instruction of
  // the wave covers one contiguous run (512 B of codes, 1 KiB of output);
  // the kPer loads of a lane are issued before any conversion
  const int lane = threadIdx.x & 63;
  const long long wave = ((long long)blockIdx.x * kConvThreads + threadIdx.x) >> 6;
  const long long stride = ((long long)gridDim.x * kConvThreads >> 6) * (kPer * 64);
  for (long long base = wave * (kPer * 64); base < a.n_blocks; base += stride) {
    uint2 w[kPer];
    uint32_t sc[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const long long b = base + 64 * j + lane;
      w[j] = make_uint2(0u, 0u);
      sc[j] = 0u;
      if (b < a.n_blocks) {
        w[j] = load_once8(a.codes + 8 * b);
        sc[j] = __builtin_nontemporal_load(a.scales + b) & 0x7Fu;
      }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const long long b = base + 64 * j + lane;
      if (b < a.n_blocks) {
        const uint32_t lo = table[sc[j]][0], hi = table[sc[j]][1];
        const uint2 r0 = convert8(w[j].x, lo, hi), r1 = convert8(w[j].y, lo, hi);
        store_once16(a.out + 16 * b, make_uint4(r0.x, r0.y, r1.x, r1.y));
      }
    }
  }
}

hipError_t launch_to_fp8(const ToFp8Args& a, hipStream_t s) {
  const long long waves = (a.n_blocks + kPer * 64 - 1) / (kPer * 64);
  long long blocks = (waves + kConvThreads / 64 - 1) / (kConvThreads / 64);
  // a grid-stride loop over at most 8 workgroups per CU; each fills its
  // table once
  blocks = blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks);
  to_fp8_kernel<<<(unsigned)blocks, kConvThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace nvfp4
