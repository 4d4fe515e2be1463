// api.cpp -- the C ABI declared in include/nvfp4kv.h: argument validation,
// the decode split planner, workspace sizing and kernel launches.
#include "nvfp4kv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.h"

using namespace nvfp4;

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int32_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return NVFP4_OK;
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool good_scale(float s) { return std::isfinite(s) && s > 0.0f; }

int32_t check_cache(const nvfp4_kv_cache* c) {
  if (!c) return fail(NVFP4_ERR_INVALID_ARG, "cache is NULL");
  if (c->head_dim != NVFP4_HEAD_DIM)
    return fail(NVFP4_ERR_UNSUPPORTED, "head_dim %d is not supported (only 128)", c->head_dim);
  if (c->page_size != NVFP4_PAGE_SIZE)
    return fail(NVFP4_ERR_UNSUPPORTED, "page_size %d is not supported (only 16)", c->page_size);
  if (c->num_pages <= 0 || c->num_kv_heads <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "num_pages (%d) and num_kv_heads (%d) must be > 0",
                c->num_pages, c->num_kv_heads);
  if (!c->k_codes || !c->k_scales || !c->v_codes || !c->v_scales)
    return fail(NVFP4_ERR_INVALID_ARG, "a cache plane pointer is NULL");
  if (!aligned16(c->k_codes) || !aligned16(c->k_scales) || !aligned16(c->v_codes) ||
      !aligned16(c->v_scales))
    return fail(NVFP4_ERR_INVALID_ARG, "cache planes must be 16-byte aligned");
  if (!good_scale(c->k_tensor_scale) || !good_scale(c->v_tensor_scale))
    return fail(NVFP4_ERR_INVALID_ARG, "tensor scales must be finite and > 0 (k %g, v %g)",
                (double)c->k_tensor_scale, (double)c->v_tensor_scale);
  return NVFP4_OK;
}

bool dtype_ok(int32_t d) { return d == NVFP4_DTYPE_F32 || d == NVFP4_DTYPE_BF16; }

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Decode work plan: the number of waves W that split the (sequence, KV head,
// page) work into equal contiguous ranges.  Automatic: at most 8 waves per
// CU (two per SIMD: with more, the oldest waves take the issue slots and the
// younger ones only stretch the tail, measured on MI355X), and at least
// kMinPagesPerWave pages per wave for the longest batch max_seq_len allows, so
// that each wave's fixed cost (query load, partial write and merge) stays
// small next to its page stream, and at most about kMaxPiecesPerSegment waves
// per (sequence, KV head) segment, since the merge of a segment's partials
// grows with their number (few long sequences).  Work too small to give every
// SIMD a wave of 16 pages is spread over up to one wave per SIMD with at least
// kMinPagesSmall pages each instead: such a call is bound by a wave's latency,
// not by the machine (configuration 1, 64 pages: 16.3 us at 4 waves, 12.1 us
// at 32; configuration 2, 16384 pages: 20.4 us at 1024 waves against 24.7 at
// 2048 and 24.1 at 512, measured on MI355X).  A requested count is used as
// given.
constexpr int64_t kMinPagesPerWave = 16;
constexpr int64_t kMinPagesSmall = 2;
constexpr int64_t kWavesPerCu = 8;
constexpr int64_t kSimdsPerCu = 4;
constexpr int64_t kMaxPiecesPerSegment = 128;
// A full launch of the 4-bit formats (two waves per SIMD) gets one more range
// per SIMD of weight 1 (~9 % of the work, ~26 pages each), interleaved with
// the static ranges in the stream.  These tail waves come last in the grid,
// so each is dispatched when a slot frees up: per-wave timestamps of the
// static launch showed a mean end of 104 us against a span of 114 us
// (configuration 4).  In interleaved calls 1024 tail ranges (one per SIMD)
// ran 8-11 % faster than none; 512, 768 and 1536 gained less, and 2048-4096
// finer ranges lost (each range pays the prologue and a partial).  With the
// tail ranges at the end of the stream instead, the last sequences' segments
// were cut into up to 20 pieces and the merge took 9.4 us instead of 6.2.

int32_t plan_waves(int32_t num_splits, bool f32_q, int32_t batch, int32_t hkv, int32_t max_seq_len,
                   int fmt = kFmtNvfp4) {
  if (num_splits > 0) return num_splits;
  const int64_t slots = (int64_t)cu_count() * std::min<int64_t>(kWavesPerCu, decode_occupancy(f32_q, fmt));
  const int64_t units = (int64_t)batch * hkv * ((max_seq_len + NVFP4_PAGE_SIZE - 1) / NVFP4_PAGE_SIZE);
  const int64_t simds = kSimdsPerCu * cu_count();
  int64_t want = (units + kMinPagesPerWave - 1) / kMinPagesPerWave;
  if (want < simds) want = std::min(simds, (units + kMinPagesSmall - 1) / kMinPagesSmall);
  want = std::min(want, std::max<int64_t>(cu_count(), kMaxPiecesPerSegment * batch * hkv));
  want = std::max<int64_t>(1, std::min(slots, want));
  if ((fmt == kFmtNvfp4 || fmt == kFmtMxfp4) && want == 2 * simds) want += simds;
  return (int32_t)want;
}

// Work weights of the decode waves.  A launch of exactly two waves per SIMD
// is placed one wave per SIMD for the first 4 x CUs workgroups and a second
// wave per SIMD for the rest (measured on MI355X).  The SIMD's issue
// arbitration favours the older wave, which then runs about 1.6 times as
// fast as its partner on NVFP4 and MXFP4 pages (their expansion makes the
// SIMD, not HBM, the limit; FP8 and BF16 pages are bound by HBM and gain
// nothing), so equal ranges leave each SIMD's second wave finishing alone,
// some 40 us after its partner on a 700 MB cache.  The first round's ranges
// are weighted 8 : 5 instead (12 : 7 and 3 : 2 were measured too), and the
// two waves of a SIMD finish within a few us of each other.  Every other
// wave count keeps equal ranges.  The results do not depend on the
// placement: the decode and the merge kernels derive the same ranges from
// these weights.
constexpr int32_t kWeightFirst = 8, kWeightRest = 5;
// With the tail ranges below the static ranges are equal (5 : 5, the tail
// ranges weighing 1, ~9 % of the work): the dispatcher does not always place
// the first round one wave per SIMD (per-wave hardware ids on one box: 91 of
// 1024 SIMDs held two first-round waves and no second-round one, and their
// waves ended last), and equal ranges give every SIMD the same static work
// whatever the placement, while the tail ranges even out the rest.  In
// interleaved calls on MI355X: 5 : 5 128.9 us, 6 : 5 132.0 us, 4 : 5 133.3 us,
// 8 : 5 142-144 us; 3 : 3, 4 : 4 and 6 : 6 (tail shares 14, 11 and 8 %) within
// 1 % of 5 : 5.
constexpr int32_t kTailWeightFirst = 5, kTailWeightRest = 5;

void set_wave_weights(DecodeArgs& a, int fmt, int64_t max_units) {
  const int64_t simds = kSimdsPerCu * cu_count();
  a.shallow = a.num_splits > simds ? 1 : 0;
  a.first_waves = a.num_splits;
  a.tail_start = a.num_splits;
  a.weight_first = 1;
  a.weight_rest = 1;
  a.weight_tail = 1;
  if (fmt != kFmtNvfp4 && fmt != kFmtMxfp4) return;
  if (a.num_splits == 2 * simds) {
    const int64_t T = (kWeightFirst + kWeightRest) * simds;   // sum of the weights
    if (max_units <= (INT64_MAX / 4) / T) {
      a.first_waves = (int32_t)simds;
      a.weight_first = kWeightFirst;
      a.weight_rest = kWeightRest;
    }
  } else if (a.num_splits == 3 * simds) {
    const int64_t T = (int64_t)(kTailWeightFirst + kTailWeightRest + 1) * simds;
    if (max_units <= (INT64_MAX / 4) / T) {
      a.first_waves = (int32_t)simds;
      a.tail_start = (int32_t)(2 * simds);
      a.weight_first = kTailWeightFirst;
      a.weight_rest = kTailWeightRest;
      a.weight_tail = 1;
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

extern "C" {

const char* nvfp4_status_string(int32_t status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID_ARG: return "invalid argument";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported configuration";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* nvfp4_last_error(void) { return g_err; }

size_t nvfp4_kv_plane_bytes(int32_t num_pages, int32_t num_kv_heads, int32_t plane) {
  if (num_pages <= 0 || num_kv_heads <= 0) return 0;
  const size_t slabs = (size_t)num_pages * num_kv_heads;
  switch (plane) {
    case 0: case 2: return slabs * (NVFP4_PAGE_SIZE * NVFP4_HEAD_DIM / 2);
    case 1: case 3: return slabs * (NVFP4_PAGE_SIZE * NVFP4_HEAD_DIM / NVFP4_BLOCK);
    default: return 0;
  }
}

size_t nvfp4_kv_cache_bytes(int32_t num_pages, int32_t num_kv_heads) {
  size_t t = 0;
  for (int p = 0; p < 4; ++p) t += nvfp4_kv_plane_bytes(num_pages, num_kv_heads, p);
  return t;
}

float nvfp4_tensor_scale_from_amax(float amax) {
  if (!std::isfinite(amax) || !(amax > 0.0f)) return 0.0f;
  volatile float den = 2688.0f;   // 6 * 448, IEEE division
  return amax / den;
}

int32_t nvfp4_abs_max(const void* x, int32_t dtype, int64_t n, float* amax_out, void* stream) {
  g_err[0] = 0;
  if (!dtype_ok(dtype)) return fail(NVFP4_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (n < 0) return fail(NVFP4_ERR_INVALID_ARG, "n < 0");
  if (!amax_out || (n > 0 && !x)) return fail(NVFP4_ERR_INVALID_ARG, "NULL pointer");
  return hip_status(launch_absmax(x, dtype == NVFP4_DTYPE_F32, n, amax_out, (hipStream_t)stream),
                    "abs_max launch");
}

int32_t nvfp4_to_fp8(const void* codes, const void* scales, int64_t n, float global_scale,
                     float out_scale, void* fp8_out, void* stream) {
  g_err[0] = 0;
  if (n < 0 || n % 16 != 0) return fail(NVFP4_ERR_INVALID_ARG, "n must be a non-negative multiple of 16");
  if (!good_scale(global_scale))
    return fail(NVFP4_ERR_INVALID_ARG, "global_scale must be finite and > 0");
  if (!good_scale(out_scale))
    return fail(NVFP4_ERR_INVALID_ARG, "out_scale must be finite and > 0");
  if (n == 0) return NVFP4_OK;
  if (!codes || !scales || !fp8_out) return fail(NVFP4_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(codes) || !aligned16(fp8_out))
    return fail(NVFP4_ERR_INVALID_ARG, "codes / fp8_out must be 16-byte aligned");
  ToFp8Args a;
  a.codes = static_cast<const uint8_t*>(codes);
  a.scales = static_cast<const uint8_t*>(scales);
  a.out = static_cast<uint8_t*>(fp8_out);
  a.n_blocks = n / 16;
  a.g = global_scale;
  a.s8 = out_scale;
  return hip_status(launch_to_fp8(a, (hipStream_t)stream), "to_fp8 launch");
}

// Validation of the row arguments and launch shared by the NVFP4 and MXFP4
// appends; a holds the cache planes and scales, hkv the cache's heads.
static int32_t append_rows(AppendArgs a, int mode, const void* k_new, const void* v_new,
                           int32_t dtype, int32_t n_tok, const int32_t* tok_seq,
                           const int32_t* tok_pos, const int32_t* page_table,
                           int32_t max_pages_per_seq, void* stream) {
  if (!dtype_ok(dtype)) return fail(NVFP4_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (n_tok < 0) return fail(NVFP4_ERR_INVALID_ARG, "n_tok < 0");
  if (max_pages_per_seq <= 0) return fail(NVFP4_ERR_INVALID_ARG, "max_pages_per_seq must be > 0");
  if (n_tok == 0) return NVFP4_OK;
  if (!k_new || !v_new || !tok_seq || !tok_pos || !page_table)
    return fail(NVFP4_ERR_INVALID_ARG, "NULL input pointer");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(NVFP4_ERR_INVALID_ARG, "k_new / v_new must be 16-byte aligned");
  a.k_new = k_new; a.v_new = v_new;
  a.tok_seq = tok_seq; a.tok_pos = tok_pos; a.page_table = page_table;
  a.max_pages = max_pages_per_seq; a.n_tok = n_tok;
  return hip_status(launch_append(a, dtype == NVFP4_DTYPE_F32, mode, (hipStream_t)stream), "append launch");
}

static int32_t append_call(const nvfp4_kv_cache* cache, const void* k_new, const void* v_new,
                           int32_t dtype, int32_t n_tok, const int32_t* tok_seq,
                           const int32_t* tok_pos, const int32_t* page_table,
                           int32_t max_pages_per_seq, int mode, void* stream) {
  g_err[0] = 0;
  int32_t st = check_cache(cache);
  if (st) return st;
  AppendArgs a;
  a.k_codes = cache->k_codes; a.k_scales = cache->k_scales;
  a.v_codes = cache->v_codes; a.v_scales = cache->v_scales;
  a.k_scale = cache->k_tensor_scale; a.v_scale = cache->v_tensor_scale;
  a.k_six_st = 6.0 * (double)cache->k_tensor_scale;
  a.v_six_st = 6.0 * (double)cache->v_tensor_scale;
  // the FP32 fast path of the block scale needs 6 s_t well inside the
  // normal FP32 range; 0 turns it off (the exact path then decides)
  auto inv6 = [](double six) { return (six > 0x1p-100 && six < 0x1p100) ? (float)(1.0 / six) : 0.0f; };
  a.k_inv6 = inv6(a.k_six_st);
  a.v_inv6 = inv6(a.v_six_st);
  a.hkv = cache->num_kv_heads;
  a.num_pages = cache->num_pages;
  return append_rows(a, mode, k_new, v_new, dtype, n_tok, tok_seq, tok_pos, page_table, max_pages_per_seq,
                     stream);
}

int32_t nvfp4_kv_append(const nvfp4_kv_cache* cache, const void* k_new, const void* v_new,
                        int32_t dtype, int32_t n_tok, const int32_t* tok_seq,
                        const int32_t* tok_pos, const int32_t* page_table,
                        int32_t max_pages_per_seq, void* stream) {
  return append_call(cache, k_new, v_new, dtype, n_tok, tok_seq, tok_pos, page_table, max_pages_per_seq,
                     kAppendAmax6, stream);
}

int32_t nvfp4_kv_append_mse(const nvfp4_kv_cache* cache, const void* k_new, const void* v_new,
                            int32_t dtype, int32_t n_tok, const int32_t* tok_seq,
                            const int32_t* tok_pos, const int32_t* page_table,
                            int32_t max_pages_per_seq, void* stream) {
  return append_call(cache, k_new, v_new, dtype, n_tok, tok_seq, tok_pos, page_table, max_pages_per_seq,
                     kAppendMse, stream);
}

int32_t nvfp4_kv_dequant(const nvfp4_kv_cache* cache, const int32_t* page_table_row,
                         int32_t pos0, int32_t n, void* k_out, void* v_out,
                         int32_t out_dtype, void* stream) {
  g_err[0] = 0;
  int32_t st = check_cache(cache);
  if (st) return st;
  if (!dtype_ok(out_dtype)) return fail(NVFP4_ERR_UNSUPPORTED, "dtype %d", out_dtype);
  if (pos0 < 0 || n < 0) return fail(NVFP4_ERR_INVALID_ARG, "pos0 and n must be >= 0");
  if (n == 0) return NVFP4_OK;
  if (!page_table_row) return fail(NVFP4_ERR_INVALID_ARG, "page_table_row is NULL");
  if (!k_out && !v_out) return NVFP4_OK;
  if ((k_out && !aligned16(k_out)) || (v_out && !aligned16(v_out)))
    return fail(NVFP4_ERR_INVALID_ARG, "outputs must be 16-byte aligned");
  DequantArgs a;
  a.k_codes = cache->k_codes; a.k_scales = cache->k_scales;
  a.v_codes = cache->v_codes; a.v_scales = cache->v_scales;
  a.k_scale = cache->k_tensor_scale; a.v_scale = cache->v_tensor_scale;
  a.page_table_row = page_table_row; a.pos0 = pos0; a.n = n; a.hkv = cache->num_kv_heads;
  a.num_pages = cache->num_pages;
  a.k_out = k_out; a.v_out = v_out;
  return hip_status(launch_dequant(a, out_dtype == NVFP4_DTYPE_F32, (hipStream_t)stream),
                    "dequant launch");
}

int32_t nvfp4_decode_num_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len,
                                int32_t num_splits) {
  if (batch <= 0 || num_kv_heads <= 0 || max_seq_len < 0 || num_splits < 0) return 0;
  return plan_waves(num_splits, false, batch, num_kv_heads, max_seq_len);
}

static size_t decode_ws(int32_t batch, int32_t group, int32_t waves) {
  const size_t pieces = (size_t)waves * 2 * group;
  return align256(pieces * NVFP4_HEAD_DIM * sizeof(float)) + align256(pieces * sizeof(float)) +
         align256(((size_t)batch + 1) * sizeof(int32_t));
}

size_t nvfp4_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t max_seq_len, int32_t num_splits) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 || num_splits < 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  // sized for the FP32-query kernel too (its occupancy is never higher)
  const int32_t w = std::max(plan_waves(num_splits, false, batch, num_kv_heads, max_seq_len),
                             plan_waves(num_splits, true, batch, num_kv_heads, max_seq_len));
  return decode_ws(batch, num_q_heads / num_kv_heads, w);
}

// Validation and launch shared by the NVFP4 and comparison-format decodes
// (the cache itself has been checked by the caller).
static int32_t decode_call(int fmt, const uint8_t* kplane, const uint8_t* kscales, const uint8_t* vplane,
                           const uint8_t* vscales, float k_scale, float v_scale, int32_t hkv, int32_t num_pages,
                           const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                           const int32_t* page_table, int32_t max_pages_per_seq,
                           const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                           int32_t num_splits, void* workspace, size_t workspace_bytes, float* out,
                           void* stream, int32_t k_exp = 0, int32_t v_exp = 0,
                           bool fixed_scratch = false) {
  if (!dtype_ok(q_dtype)) return fail(NVFP4_ERR_UNSUPPORTED, "q dtype %d", q_dtype);
  const int64_t num_slabs = (int64_t)num_pages * hkv;
  if (num_slabs > (int64_t)UINT32_MAX) return fail(NVFP4_ERR_INVALID_ARG, "num_pages x num_kv_heads too large");
  if (batch < 0 || num_q_heads <= 0 || max_seq_len < 0 || num_splits < 0 || max_pages_per_seq <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "bad sizes (batch %d, heads %d, max_seq_len %d, splits %d, "
                "max_pages %d)", batch, num_q_heads, max_seq_len, num_splits, max_pages_per_seq);
  if (num_q_heads % hkv != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, hkv);
  const int32_t G = num_q_heads / hkv;
  if (G > 16) return fail(NVFP4_ERR_UNSUPPORTED, "more than 16 query heads per KV head (%d)", G);
  if ((int64_t)(max_seq_len + NVFP4_PAGE_SIZE - 1) / NVFP4_PAGE_SIZE > max_pages_per_seq)
    return fail(NVFP4_ERR_INVALID_ARG, "max_seq_len %d needs more than max_pages_per_seq %d pages",
                max_seq_len, max_pages_per_seq);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f))
    return fail(NVFP4_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (batch == 0) return NVFP4_OK;
  if (!q || !page_table || !seq_lens || !out) return fail(NVFP4_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(q) || !aligned16(out)) return fail(NVFP4_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
  const bool f32q = q_dtype == NVFP4_DTYPE_F32;
  const int32_t W = plan_waves(num_splits, f32q, batch, hkv, max_seq_len, fmt);
  const size_t need = decode_ws(batch, G, W);
  if (fixed_scratch) {
    if (need > kScratchBytes)
      return fail(NVFP4_ERR_WORKSPACE, "decode needs %zu workspace bytes, more than the fixed scratch of %zu "
                  "(use nvfp4_decode_attn with a workspace)", need, kScratchBytes);
    hipError_t e = scratch_address(&workspace);
    if (e != hipSuccess) return hip_status(e, "scratch address");
    workspace_bytes = kScratchBytes;
  }
  if (!workspace || workspace_bytes < need)
    return fail(NVFP4_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(NVFP4_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  DecodeArgs a;
  a.k_codes = kplane; a.k_scales = kscales;
  a.v_codes = vplane; a.v_scales = vscales;
  a.q = q; a.page_table = page_table; a.seq_lens = seq_lens; a.out = out;
  const size_t pieces = (size_t)W * 2 * G;
  char* ws = static_cast<char*>(workspace);
  a.ws_o = reinterpret_cast<float*>(ws);
  a.ws_lse = reinterpret_cast<float*>(ws + align256(pieces * NVFP4_HEAD_DIM * sizeof(float)));
  a.ws_prefix = reinterpret_cast<int32_t*>(ws + align256(pieces * NVFP4_HEAD_DIM * sizeof(float)) +
                                           align256(pieces * sizeof(float)));
  a.qk_scale = (float)((double)k_scale * (double)softmax_scale * 1.4426950408889634);
  a.v_scale = v_scale;
  a.k_exp = k_exp;
  a.v_exp = v_exp;
  a.max_pages = max_pages_per_seq;
  a.batch = batch; a.hq = num_q_heads; a.hkv = hkv; a.group = G;
  a.num_splits = W;
  a.num_slabs = (uint32_t)num_slabs;
  set_wave_weights(a, fmt, (int64_t)batch * hkv * max_pages_per_seq);
  return hip_status(launch_decode(a, f32q, fmt, (hipStream_t)stream), "decode launch");
}

int32_t nvfp4_decode_attn(const nvfp4_kv_cache* cache, const void* q, int32_t q_dtype,
                          int32_t batch, int32_t num_q_heads, const int32_t* page_table,
                          int32_t max_pages_per_seq, const int32_t* seq_lens,
                          int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, float* out, void* stream) {
  g_err[0] = 0;
  int32_t st = check_cache(cache);
  if (st) return st;
  return decode_call(kFmtNvfp4, cache->k_codes, cache->k_scales, cache->v_codes, cache->v_scales,
                     cache->k_tensor_scale, cache->v_tensor_scale, cache->num_kv_heads, cache->num_pages, q, q_dtype,
                     batch, num_q_heads, page_table, max_pages_per_seq, seq_lens, max_seq_len,
                     softmax_scale, num_splits, workspace, workspace_bytes, out, stream);
}

int32_t nvfp4_decode_gather_probe(const nvfp4_kv_cache* cache, int32_t batch, const int32_t* page_table,
                                  int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                  int32_t num_splits, void* sink, size_t sink_bytes, void* stream) {
  g_err[0] = 0;
  int32_t st = check_cache(cache);
  if (st) return st;
  if (batch < 0 || max_seq_len < 0 || num_splits < 0 || max_pages_per_seq <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "bad sizes");
  if ((int64_t)(max_seq_len + NVFP4_PAGE_SIZE - 1) / NVFP4_PAGE_SIZE > max_pages_per_seq)
    return fail(NVFP4_ERR_INVALID_ARG, "max_seq_len %d needs more than max_pages_per_seq %d pages",
                max_seq_len, max_pages_per_seq);
  if (batch == 0) return NVFP4_OK;
  if (!page_table || !seq_lens || !sink) return fail(NVFP4_ERR_INVALID_ARG, "NULL pointer");
  const int64_t num_slabs = (int64_t)cache->num_pages * cache->num_kv_heads;
  if (num_slabs * (NVFP4_PAGE_SIZE * NVFP4_HEAD_DIM / 2) > 0x7FFFFFFFll)
    return fail(NVFP4_ERR_UNSUPPORTED, "the probe takes caches whose planes fit 31-bit offsets");
  const int32_t W = plan_waves(num_splits, false, batch, cache->num_kv_heads, max_seq_len);
  if (sink_bytes < (size_t)W * 64 * sizeof(uint32_t))
    return fail(NVFP4_ERR_WORKSPACE, "the probe needs %zu sink bytes", (size_t)W * 64 * sizeof(uint32_t));
  DecodeArgs a = {};
  a.k_codes = cache->k_codes; a.k_scales = cache->k_scales;
  a.v_codes = cache->v_codes; a.v_scales = cache->v_scales;
  a.page_table = page_table; a.seq_lens = seq_lens;
  a.out = static_cast<float*>(sink);
  a.max_pages = max_pages_per_seq;
  a.batch = batch; a.hkv = cache->num_kv_heads; a.group = 1; a.hq = cache->num_kv_heads;
  a.num_splits = W;
  a.num_slabs = (uint32_t)num_slabs;
  set_wave_weights(a, kFmtNvfp4, (int64_t)batch * a.hkv * max_pages_per_seq);
  return hip_status(launch_gather_probe(a, (hipStream_t)stream), "probe launch");
}

int32_t nvfp4_decode_attn_noalloc(const nvfp4_kv_cache* cache, const void* q, int32_t q_dtype,
                                  int32_t batch, int32_t num_q_heads, const int32_t* page_table,
                                  int32_t max_pages_per_seq, const int32_t* seq_lens,
                                  int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                                  float* out, void* stream) {
  g_err[0] = 0;
  int32_t st = check_cache(cache);
  if (st) return st;
  return decode_call(kFmtNvfp4, cache->k_codes, cache->k_scales, cache->v_codes, cache->v_scales,
                     cache->k_tensor_scale, cache->v_tensor_scale, cache->num_kv_heads, cache->num_pages, q, q_dtype,
                     batch, num_q_heads, page_table, max_pages_per_seq, seq_lens, max_seq_len,
                     softmax_scale, num_splits, nullptr, 0, out, stream, 0, 0, true);
}

// ------------------------------------------------ comparison formats

static int32_t cmp_elem_bytes(int32_t format) {
  return format == NVFP4_CMP_FP8 ? 1 : format == NVFP4_CMP_BF16 ? 2 : 0;
}

static int32_t check_cmp_cache(const nvfp4_cmp_cache* c) {
  if (!c) return fail(NVFP4_ERR_INVALID_ARG, "cache is NULL");
  if (!cmp_elem_bytes(c->format)) return fail(NVFP4_ERR_UNSUPPORTED, "cache format %d", c->format);
  if (c->head_dim != NVFP4_HEAD_DIM)
    return fail(NVFP4_ERR_UNSUPPORTED, "head_dim %d is not supported (only 128)", c->head_dim);
  if (c->page_size != NVFP4_PAGE_SIZE)
    return fail(NVFP4_ERR_UNSUPPORTED, "page_size %d is not supported (only 16)", c->page_size);
  if (c->num_pages <= 0 || c->num_kv_heads <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "num_pages (%d) and num_kv_heads (%d) must be > 0",
                c->num_pages, c->num_kv_heads);
  if (!c->k || !c->v) return fail(NVFP4_ERR_INVALID_ARG, "a cache plane pointer is NULL");
  if (!aligned16(c->k) || !aligned16(c->v))
    return fail(NVFP4_ERR_INVALID_ARG, "cache planes must be 16-byte aligned");
  if (c->format == NVFP4_CMP_FP8 && (!good_scale(c->k_scale) || !good_scale(c->v_scale)))
    return fail(NVFP4_ERR_INVALID_ARG, "FP8 tensor scales must be finite and > 0 (k %g, v %g)",
                (double)c->k_scale, (double)c->v_scale);
  return NVFP4_OK;
}

size_t nvfp4_cmp_plane_bytes(int32_t num_pages, int32_t num_kv_heads, int32_t format) {
  if (num_pages <= 0 || num_kv_heads <= 0 || !cmp_elem_bytes(format)) return 0;
  return (size_t)num_pages * num_kv_heads * NVFP4_PAGE_SIZE * NVFP4_HEAD_DIM * cmp_elem_bytes(format);
}

float nvfp4_cmp_fp8_scale_from_amax(float amax) {
  if (!std::isfinite(amax) || !(amax > 0.0f)) return 0.0f;
  return amax / 448.0f;
}

int32_t nvfp4_cmp_append(const nvfp4_cmp_cache* cache, const void* k_new, const void* v_new,
                         int32_t dtype, int32_t n_tok, const int32_t* tok_seq,
                         const int32_t* tok_pos, const int32_t* page_table,
                         int32_t max_pages_per_seq, void* stream) {
  g_err[0] = 0;
  int32_t st = check_cmp_cache(cache);
  if (st) return st;
  if (!dtype_ok(dtype)) return fail(NVFP4_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (n_tok < 0) return fail(NVFP4_ERR_INVALID_ARG, "n_tok < 0");
  if (max_pages_per_seq <= 0) return fail(NVFP4_ERR_INVALID_ARG, "max_pages_per_seq must be > 0");
  if (n_tok == 0) return NVFP4_OK;
  if (!k_new || !v_new || !tok_seq || !tok_pos || !page_table)
    return fail(NVFP4_ERR_INVALID_ARG, "NULL input pointer");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(NVFP4_ERR_INVALID_ARG, "k_new / v_new must be 16-byte aligned");
  CmpAppendArgs a;
  a.k = static_cast<uint8_t*>(cache->k);
  a.v = static_cast<uint8_t*>(cache->v);
  a.k_scale = cache->k_scale; a.v_scale = cache->v_scale;
  a.k_new = k_new; a.v_new = v_new;
  a.tok_seq = tok_seq; a.tok_pos = tok_pos; a.page_table = page_table;
  a.max_pages = max_pages_per_seq; a.n_tok = n_tok; a.hkv = cache->num_kv_heads;
  a.fmt = cache->format == NVFP4_CMP_FP8 ? kFmtFp8 : kFmtBf16;
  a.num_pages = cache->num_pages;
  return hip_status(launch_cmp_append(a, dtype == NVFP4_DTYPE_F32, (hipStream_t)stream), "append launch");
}

size_t nvfp4_cmp_decode_workspace_bytes(int32_t format, int32_t batch, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t max_seq_len,
                                        int32_t num_splits) {
  if (!cmp_elem_bytes(format) || batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      max_seq_len < 0 || num_splits < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  const int fmt = format == NVFP4_CMP_FP8 ? kFmtFp8 : kFmtBf16;
  const int32_t w = std::max(plan_waves(num_splits, false, batch, num_kv_heads, max_seq_len, fmt),
                             plan_waves(num_splits, true, batch, num_kv_heads, max_seq_len, fmt));
  return decode_ws(batch, num_q_heads / num_kv_heads, w);
}

int32_t nvfp4_cmp_decode_attn(const nvfp4_cmp_cache* cache, const void* q, int32_t q_dtype,
                              int32_t batch, int32_t num_q_heads, const int32_t* page_table,
                              int32_t max_pages_per_seq, const int32_t* seq_lens,
                              int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                              void* workspace, size_t workspace_bytes, float* out, void* stream) {
  g_err[0] = 0;
  int32_t st = check_cmp_cache(cache);
  if (st) return st;
  const bool fp8 = cache->format == NVFP4_CMP_FP8;
  return decode_call(fp8 ? kFmtFp8 : kFmtBf16, static_cast<const uint8_t*>(cache->k), nullptr,
                     static_cast<const uint8_t*>(cache->v), nullptr, fp8 ? cache->k_scale : 1.0f,
                     fp8 ? cache->v_scale : 1.0f, cache->num_kv_heads, cache->num_pages, q, q_dtype, batch,
                     num_q_heads,
                     page_table, max_pages_per_seq, seq_lens, max_seq_len, softmax_scale, num_splits,
                     workspace, workspace_bytes, out, stream);
}

// ------------------------------------------------------------------ MXFP4

static int32_t check_mx_cache(const nvfp4_mx_cache* c) {
  if (!c) return fail(NVFP4_ERR_INVALID_ARG, "cache is NULL");
  if (c->head_dim != NVFP4_HEAD_DIM)
    return fail(NVFP4_ERR_UNSUPPORTED, "head_dim %d is not supported (only 128)", c->head_dim);
  if (c->page_size != NVFP4_PAGE_SIZE)
    return fail(NVFP4_ERR_UNSUPPORTED, "page_size %d is not supported (only 16)", c->page_size);
  if (c->num_pages <= 0 || c->num_kv_heads <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "num_pages (%d) and num_kv_heads (%d) must be > 0",
                c->num_pages, c->num_kv_heads);
  if (!c->k_codes || !c->k_scales || !c->v_codes || !c->v_scales)
    return fail(NVFP4_ERR_INVALID_ARG, "a cache plane pointer is NULL");
  if (!aligned16(c->k_codes) || !aligned16(c->k_scales) || !aligned16(c->v_codes) ||
      !aligned16(c->v_scales))
    return fail(NVFP4_ERR_INVALID_ARG, "cache planes must be 16-byte aligned");
  if (c->k_exp_offset < -126 || c->k_exp_offset > 127 || c->v_exp_offset < -126 || c->v_exp_offset > 127)
    return fail(NVFP4_ERR_INVALID_ARG, "exp offsets must lie in [-126, 127] (k %d, v %d)", c->k_exp_offset,
                c->v_exp_offset);
  return NVFP4_OK;
}

size_t nvfp4_mx_plane_bytes(int32_t num_pages, int32_t num_kv_heads, int32_t plane) {
  if (num_pages <= 0 || num_kv_heads <= 0) return 0;
  const size_t slabs = (size_t)num_pages * num_kv_heads;
  switch (plane) {
    case 0: case 2: return slabs * (NVFP4_PAGE_SIZE * NVFP4_HEAD_DIM / 2);
    case 1: case 3: return slabs * (NVFP4_PAGE_SIZE * NVFP4_HEAD_DIM / 32);   // one E8M0 byte per 32
    default: return 0;
  }
}

int32_t nvfp4_mx_exp_offset_from_amax(float amax) {
  if (!std::isfinite(amax) || !(amax > 0.0f)) return 0;
  return std::ilogb(amax) - 10;
}

int32_t nvfp4_mx_append(const nvfp4_mx_cache* cache, const void* k_new, const void* v_new,
                        int32_t dtype, int32_t n_tok, const int32_t* tok_seq,
                        const int32_t* tok_pos, const int32_t* page_table,
                        int32_t max_pages_per_seq, void* stream) {
  g_err[0] = 0;
  int32_t st = check_mx_cache(cache);
  if (st) return st;
  AppendArgs a = {};
  a.k_codes = cache->k_codes; a.k_scales = cache->k_scales;
  a.v_codes = cache->v_codes; a.v_scales = cache->v_scales;
  a.k_scale = a.v_scale = 1.0f;
  a.hkv = cache->num_kv_heads;
  a.num_pages = cache->num_pages;
  return append_rows(a, kAppendMx, k_new, v_new, dtype, n_tok, tok_seq, tok_pos, page_table,
                     max_pages_per_seq, stream);
}

size_t nvfp4_mx_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t max_seq_len, int32_t num_splits) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 || num_splits < 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  const int32_t w = std::max(plan_waves(num_splits, false, batch, num_kv_heads, max_seq_len, kFmtMxfp4),
                             plan_waves(num_splits, true, batch, num_kv_heads, max_seq_len, kFmtMxfp4));
  return decode_ws(batch, num_q_heads / num_kv_heads, w);
}

int32_t nvfp4_mx_decode_attn(const nvfp4_mx_cache* cache, const void* q, int32_t q_dtype,
                             int32_t batch, int32_t num_q_heads, const int32_t* page_table,
                             int32_t max_pages_per_seq, const int32_t* seq_lens,
                             int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                             void* workspace, size_t workspace_bytes, float* out, void* stream) {
  g_err[0] = 0;
  int32_t st = check_mx_cache(cache);
  if (st) return st;
  return decode_call(kFmtMxfp4, cache->k_codes, cache->k_scales, cache->v_codes, cache->v_scales,
                     std::ldexp(1.0f, cache->k_exp_offset), std::ldexp(1.0f, cache->v_exp_offset),
                     cache->num_kv_heads, cache->num_pages, q, q_dtype, batch, num_q_heads, page_table, max_pages_per_seq,
                     seq_lens, max_seq_len, softmax_scale, num_splits, workspace, workspace_bytes, out,
                     stream, cache->k_exp_offset, cache->v_exp_offset);
}

static size_t prefill_ws(int32_t total, int32_t hkv, int32_t mode) {
  const size_t tiles = (size_t)(total + kPrefillTile - 1) / kPrefillTile;
  const size_t eb = mode == NVFP4_PREFILL_F16 ? 2 : 1;
  const size_t one = align256(tiles * kPrefillTile * NVFP4_HEAD_DIM * (size_t)hkv * eb);
  return mode == kPrefillMx ? one : 2 * one;    // MXFP4: V~ only (K is read from the cache)
}

size_t nvfp4_prefill_workspace_bytes(int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t prefix_len, int32_t mode) {
  (void)num_q_heads;
  if (num_tokens < 0 || num_kv_heads <= 0 || prefix_len < 0) return 0;
  if (mode != NVFP4_PREFILL_FP8 && mode != NVFP4_PREFILL_F16) return 0;
  return prefill_ws(prefix_len + num_tokens, num_kv_heads, mode);
}

size_t nvfp4_mx_prefill_workspace_bytes(int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t prefix_len) {
  (void)num_q_heads;
  if (num_tokens < 0 || num_kv_heads <= 0 || prefix_len < 0) return 0;
  return prefill_ws(prefix_len + num_tokens, num_kv_heads, kPrefillMx);
}

// Shared checks and launch of the prefill entry points; the planes and
// scales of the cache are in a (its mode set), the rest is checked here.
static int32_t prefill_call(PrefillArgs a, int32_t hkv, const void* q, int32_t q_dtype, int32_t num_tokens,
                            int32_t num_q_heads, const int32_t* page_table_row, int32_t prefix_len,
                            int32_t causal, float softmax_scale, void* workspace, size_t workspace_bytes,
                            float* out, void* stream) {
  if (!dtype_ok(q_dtype)) return fail(NVFP4_ERR_UNSUPPORTED, "q dtype %d", q_dtype);
  if (num_tokens < 0 || prefix_len < 0 || num_q_heads <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "bad sizes (tokens %d, prefix %d, heads %d)", num_tokens,
                prefix_len, num_q_heads);
  if (num_q_heads % hkv != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, hkv);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f))
    return fail(NVFP4_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if ((int64_t)prefix_len + num_tokens > (int64_t)1 << 30)
    return fail(NVFP4_ERR_INVALID_ARG, "context too long");
  if (num_tokens == 0) return NVFP4_OK;
  if (!q || !page_table_row || !out) return fail(NVFP4_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(q) || !aligned16(out)) return fail(NVFP4_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
  const int32_t total = prefix_len + num_tokens;
  const size_t need = prefill_ws(total, hkv, a.mode);
  if (!workspace || workspace_bytes < need)
    return fail(NVFP4_ERR_WORKSPACE, "prefill needs %zu workspace bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(NVFP4_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  a.q = q; a.page_table_row = page_table_row; a.out = out;
  if (a.mode == kPrefillMx) {
    a.kx = nullptr;
    a.vx = static_cast<uint8_t*>(workspace);
  } else {
    a.kx = static_cast<uint8_t*>(workspace);
    a.vx = static_cast<uint8_t*>(workspace) + need / 2;
  }
  a.softmax_scale = softmax_scale;
  a.T = num_tokens; a.hq = num_q_heads; a.hkv = hkv; a.group = num_q_heads / hkv;
  a.prefix = prefix_len; a.causal = causal ? 1 : 0; a.total = total;
  a.num_tiles = (total + kPrefillTile - 1) / kPrefillTile;
  return hip_status(launch_prefill(a, q_dtype == NVFP4_DTYPE_F32, (hipStream_t)stream),
                    "prefill launch");
}

int32_t nvfp4_prefill_attn(const nvfp4_kv_cache* cache, const void* q, int32_t q_dtype,
                           int32_t num_tokens, int32_t num_q_heads,
                           const int32_t* page_table_row, int32_t prefix_len, int32_t causal,
                           int32_t mode, float softmax_scale, void* workspace,
                           size_t workspace_bytes, float* out, void* stream) {
  g_err[0] = 0;
  int32_t st = check_cache(cache);
  if (st) return st;
  if (mode != NVFP4_PREFILL_FP8 && mode != NVFP4_PREFILL_F16)
    return fail(NVFP4_ERR_UNSUPPORTED, "prefill mode %d", mode);
  PrefillArgs a = {};
  a.k_codes = cache->k_codes; a.k_scales = cache->k_scales;
  a.v_codes = cache->v_codes; a.v_scales = cache->v_scales;
  a.mode = mode;
  a.k_scale = cache->k_tensor_scale; a.v_scale = cache->v_tensor_scale;
  a.num_pages = cache->num_pages;
  return prefill_call(a, cache->num_kv_heads, q, q_dtype, num_tokens, num_q_heads, page_table_row, prefix_len,
                      causal, softmax_scale, workspace, workspace_bytes, out, stream);
}

int32_t nvfp4_mx_prefill_attn(const nvfp4_mx_cache* cache, const void* q, int32_t q_dtype,
                              int32_t num_tokens, int32_t num_q_heads,
                              const int32_t* page_table_row, int32_t prefix_len, int32_t causal,
                              float softmax_scale, void* workspace, size_t workspace_bytes, float* out,
                              void* stream) {
  g_err[0] = 0;
  int32_t st = check_mx_cache(cache);
  if (st) return st;
  PrefillArgs a = {};
  a.k_codes = cache->k_codes; a.k_scales = cache->k_scales;
  a.v_codes = cache->v_codes; a.v_scales = cache->v_scales;
  a.mode = kPrefillMx;
  // K values are the codes times their E8M0 scales (no tensor scale); V~
  // holds values relative to 2^v_ref, with the largest block of a tensor
  // quantized under v_exp_offset (at v_exp_offset + 8) reaching 6 * 2^6
  a.k_scale = 1.0f;
  a.v_ref = std::min(cache->v_exp_offset + 2, 125);
  a.v_scale = std::ldexp(1.0f, a.v_ref);
  a.num_pages = cache->num_pages;
  return prefill_call(a, cache->num_kv_heads, q, q_dtype, num_tokens, num_q_heads, page_table_row, prefix_len,
                      causal, softmax_scale, workspace, workspace_bytes, out, stream);
}

}  // extern "C"
