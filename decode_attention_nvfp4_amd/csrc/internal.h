// internal.h -- argument blocks and launchers shared by the C-ABI layer
// (api.cpp) and the kernels.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kPrefillTile = 64;   // keys per prefill tile
constexpr int kFmtNvfp4 = 0;       // cache formats of the decode kernel: NVFP4,
constexpr int kFmtFp8 = 1;         // and the comparison formats (values of
constexpr int kFmtBf16 = 2;        // nvfp4_cmp_format)
constexpr int kFmtMxfp4 = 3;       // the MXFP4 cache
// block-scale rules of the append kernel
constexpr int kAppendAmax6 = 0;    // NVFP4, E4M3 nearest to amax / (6 s_t)
constexpr int kAppendMse = 1;      // NVFP4, MSE-searched E4M3 scale
constexpr int kAppendMx = 2;       // MXFP4, E8M0 floor(log2 amax) - 2
constexpr int kPrefillFP8 = 0;     // operand precisions of the prefill path
constexpr int kPrefillF16 = 1;
constexpr int kPrefillMx = 2;      // MXFP4 cache: FP4 K operand, FP8 V~, Q', P

struct AppendArgs {
  uint8_t* k_codes;
  uint8_t* k_scales;
  uint8_t* v_codes;
  uint8_t* v_scales;
  float k_scale, v_scale;     // tensor scales s_t
  double k_six_st, v_six_st;  // 6 * s_t, exact in double
  float k_inv6, v_inv6;       // 1 / (6 * s_t) rounded to FP32 (fast block-scale path)
  const void* k_new;
  const void* v_new;
  const int32_t* tok_seq;
  const int32_t* tok_pos;
  const int32_t* page_table;
  int32_t max_pages;
  int32_t n_tok;
  int32_t hkv;
  int32_t num_pages;          // page ids beyond the cache are clamped to its last page
};

// Append to a comparison-format cache: k / v planes of E4M3 codes of
// x / s_t, or of bf16 values.
struct CmpAppendArgs {
  uint8_t* k;
  uint8_t* v;
  float k_scale, v_scale;
  const void* k_new;
  const void* v_new;
  const int32_t* tok_seq;
  const int32_t* tok_pos;
  const int32_t* page_table;
  int32_t max_pages;
  int32_t n_tok;
  int32_t hkv;
  int32_t fmt;
  int32_t num_pages;
};

// NVFP4 -> FP8 conversion of a flat run of 16-element blocks.
struct ToFp8Args {
  const uint8_t* codes;     // 8 bytes per block, 16-byte aligned
  const uint8_t* scales;    // 1 byte per block
  uint8_t* out;             // 16 bytes per block, 16-byte aligned
  long long n_blocks;
  float g;                  // global encode scale (divides)
  float s8;                 // output scale (divides)
};

struct DequantArgs {
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  float k_scale, v_scale;
  const int32_t* page_table_row;
  int32_t pos0, n, hkv;
  int32_t num_pages;
  void* k_out;
  void* v_out;
};

struct DecodeArgs {
  const uint8_t* k_codes;     // comparison formats: the k plane
  const uint8_t* k_scales;    // (unused by the comparison formats)
  const uint8_t* v_codes;     // comparison formats: the v plane
  const uint8_t* v_scales;
  const void* q;              // [B][Hq][128]
  const int32_t* page_table;  // [B][max_pages]
  const int32_t* seq_lens;    // [B]
  float* out;                 // [B][Hq][128]
  float* ws_o;                // partials [W][2][G][128]
  float* ws_lse;              // partial log2-sum-exp [W][2][G]
  int32_t* ws_prefix;         // [B+1] exclusive prefix of pages per sequence
  float qk_scale;             // s_tK * softmax_scale * log2(e)
  float v_scale;              // s_tV
  int32_t max_pages;
  int32_t batch, hq, hkv, group;
  int32_t num_splits;         // W: number of waves (work ranges)
  uint32_t num_slabs;         // num_pages * hkv: (page, head) slabs of each plane
  int32_t k_exp, v_exp;       // MXFP4: values are taken relative to 2^k_exp, 2^v_exp
  // work weights of the waves: the first first_waves weigh weight_first,
  // the rest weight_rest (equal weights: equal ranges); or, when tail_start <
  // num_splits (= 3 first_waves), the three classes of first_waves waves weigh
  // weight_first, weight_rest and weight_tail with their ranges interleaved
  // in the stream (RangeMath)
  int32_t first_waves, weight_first, weight_rest;
  int32_t tail_start, weight_tail;
  // more than one wave per SIMD: the 4-bit formats take the shallower page
  // pipeline
  int32_t shallow;
};

struct PrefillArgs {
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  const void* q;              // [T][Hq][128]
  const int32_t* page_table_row;
  float* out;                 // [T][Hq][128]
  uint8_t* kx;                // workspace: expanded K  [Hkv][tiles*64][128]
  uint8_t* vx;                // workspace: expanded V^T [Hkv][tiles][128][64]
  float k_scale, v_scale;     // tensor scales
  float softmax_scale;
  int32_t T, hq, hkv, group;
  int32_t prefix, causal;
  int32_t total;              // prefix + T
  int32_t num_tiles;          // ceil(total / 64)
  int32_t mode;               // kPrefillFP8, kPrefillF16 or kPrefillMx
  int32_t num_pages;
  int32_t v_ref;              // MXFP4: V~ holds values relative to 2^v_ref (v_scale = 2^v_ref)
};

// A page id read from a page table, clamped into the cache (ids outside
// [0, num_pages) are a caller error; clamping keeps every access inside the
// planes).
__host__ __device__ __forceinline__ int clamp_page(int page, int num_pages) {
  return (unsigned)page < (unsigned)num_pages ? page : num_pages - 1;
}

hipError_t launch_append(const AppendArgs& a, bool f32_in, int mode, hipStream_t s);
hipError_t launch_dequant(const DequantArgs& a, bool f32_out, hipStream_t s);
hipError_t launch_to_fp8(const ToFp8Args& a, hipStream_t s);
hipError_t launch_absmax(const void* x, bool f32_in, int64_t n, float* out, hipStream_t s);
hipError_t launch_cmp_append(const CmpAppendArgs& a, bool f32_in, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, bool f32_q, int fmt, hipStream_t s);
hipError_t launch_gather_probe(const DecodeArgs& a, hipStream_t s);
int decode_occupancy(bool f32_q, int fmt);   // resident decode waves per CU
hipError_t launch_prefill(const PrefillArgs& a, bool f32_q, hipStream_t s);

// Bytes of the fixed device scratch that nvfp4_decode_attn_noalloc uses as
// its decode workspace (NVFP4_DECODE_NOALLOC_SCRATCH_BYTES in the header).
constexpr size_t kScratchBytes = size_t(40) << 20;
// Device address of the current device's scratch (taken once per device).
hipError_t scratch_address(void** out);

}  // namespace nvfp4
