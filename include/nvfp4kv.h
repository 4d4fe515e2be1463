/*
 * nvfp4kv.h -- C ABI of the NVFP4 KV-cache library for AMD Instinct MI355X
 * (gfx950).  Plain C; no HIP, PyTorch or C++ types in any signature.
 *
 * The operations follow these source pages (cited by title and section):
 *  [EXPL] "NVIDIA解説: NVFP4 KV Cacheで長コンテキストLLM推論を最適化 —
 *          メモリ50%削減・TTFT 3倍高速化"
 *  [GB10] "一個 Triton FP8 繞道補丁，為 DGX Spark 的 GB10 擠出多 17% 的 NVFP4 速度"
 *  [RC17] "TensorRT-LLM rc17 が SM121（DGX Spark）向けに NVFP4 MoE バックエンドと
 *          NVFP4 KV キャッシュを追加"
 *  [TRTL] "Compilation d'inferences spécialisées en matériel FP8 et NVFP4 sur
 *          Blackwell"
 *
 * Format ([EXPL] §E2M1 + 2レベルスケーリング): every K or V element is a 4-bit
 * E2M1 code (1 sign, 2 exponent, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5,
 * 2, 3, 4, 6); every 16 consecutive elements of one token's 128-wide head
 * vector share one E4M3 (OCP E4M3FN) block scale; each of K and V has one
 * FP32 tensor scale s_t, so x ~= e2m1 * s_block * s_t.
 *
 * Quantization rule (the pages leave it open; this library fixes it):
 *   s_block = the E4M3 value nearest to amax16 / (6 * s_t), ties to the even
 *             code, clamped to 448;
 *   code    = the E2M1 value nearest to x / (s_block * s_t) in exact
 *             arithmetic, ties to the even code, clamped to 6; the sign bit is
 *             the sign of x; a zero block scale gives magnitude 0.
 *   s_t is calibrated offline, e.g. amax(|X|) / (6 * 448)
 *   (nvfp4_tensor_scale_from_amax); NVFP4 KV needs a calibrated scale rather
 *   than a runtime switch ([RC17] §実務メモ).
 * Dequantization multiplies by s_t, i.e. divides by the global encode scale
 * 1/s_t ([GB10] §這個 80 行的 Triton 繞道).
 *
 * ---------------------------------------------------------------- layout
 * The cache is paged: a page holds 16 consecutive tokens of one sequence for
 * every KV head.  Four device planes, each [num_pages][num_kv_heads][slab]:
 *
 *   k_codes  slab 1024 B: [token 16][byte 64]; byte j of a token row holds
 *            element 2j in its low nibble and element 2j+1 in its high nibble.
 *   k_scales slab  128 B: [token 16][block 8]; block j covers elements
 *            16j..16j+15.
 *   v_codes  slab 1024 B: [token quad 4][element group 16][token pair 2]
 *            [element 8]; the byte at (t/4)*256 + (d/8)*16 + ((t/2)%2)*8 + d%8
 *            holds element d of the token pair (t & ~1, t | 1): the even
 *            token in the low nibble, the odd token in the high nibble.
 *   v_scales slab  128 B: [block 8][token 16].
 *
 * Bytes per element: 0.5 (code) + 1/16 (scale) = 0.5625, i.e. 3.56x fewer
 * than FP16 and 1.78x fewer than FP8 ([EXPL] §メモリ削減効果).
 *
 * ---------------------------------------------------------- conventions
 *  - Every buffer is caller-owned device memory unless marked host.  The
 *    library allocates nothing, keeps no pointer after a call returns and
 *    holds no global state except a thread-local error string and the fixed
 *    per-device scratch of nvfp4_decode_attn_noalloc.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  All
 *    work is enqueued on it; no call synchronizes.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    failed call enqueues nothing.  Device-resident indices (page tables,
 *    sequence ids, positions, lengths) are not checked: they must lie within
 *    the bounds stated below.  Every page id read from a page table must lie
 *    in [0, num_pages); the kernels clamp an id outside that range to the
 *    last page, so a bad page table gives wrong results but no access
 *    outside the cache planes.
 *  - Every entry returns an nvfp4_status.  nvfp4_last_error() describes the
 *    most recent failure on the calling thread.
 */
#ifndef NVFP4KV_H
#define NVFP4KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARG = 1,  /* null pointer, bad size, bad scale, misaligned plane */
  NVFP4_ERR_UNSUPPORTED = 2,  /* head_dim != 128, page_size != 16, unknown dtype */
  NVFP4_ERR_WORKSPACE = 3,    /* workspace missing or too small */
  NVFP4_ERR_HIP = 4           /* the HIP runtime reported an error */
} nvfp4_status;

typedef enum nvfp4_dtype {
  NVFP4_DTYPE_F32 = 0,
  NVFP4_DTYPE_BF16 = 1
} nvfp4_dtype;

#define NVFP4_HEAD_DIM 128
#define NVFP4_PAGE_SIZE 16
#define NVFP4_BLOCK 16

/* Host description of a paged NVFP4 cache (one layer).  The four plane
 * pointers are device memory laid out as in the header comment and must be
 * 16-byte aligned.  Tensor scales must be finite and > 0. */
typedef struct nvfp4_kv_cache {
  uint8_t* k_codes;
  uint8_t* k_scales;
  uint8_t* v_codes;
  uint8_t* v_scales;
  float k_tensor_scale;
  float v_tensor_scale;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t page_size;   /* must be 16 */
  int32_t head_dim;    /* must be 128 */
} nvfp4_kv_cache;

/* Text of a status code (static storage). */
const char* nvfp4_status_string(int32_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* nvfp4_last_error(void);

/* Bytes of one plane: plane 0 k_codes, 1 k_scales, 2 v_codes, 3 v_scales.
 * Returns 0 for invalid arguments. */
size_t nvfp4_kv_plane_bytes(int32_t num_pages, int32_t num_kv_heads, int32_t plane);

/* Bytes of all four planes: 2 * num_pages * 16 * num_kv_heads * 128 * 0.5625
 * (the KV-memory formula of [EXPL] §KV Cacheのメモリボトルネック for one layer,
 * 0.5625 bytes per element). */
size_t nvfp4_kv_cache_bytes(int32_t num_pages, int32_t num_kv_heads);

/* Tensor-scale calibration (step A0, host): amax / (6 * 448) in FP32.
 * Returns 0 when amax is not finite or not > 0. */
float nvfp4_tensor_scale_from_amax(float amax);

/* amax_out[0] = max |x_i| over n elements of x (device), computed exactly on
 * the device.  amax_out is one device float, overwritten.  n >= 0. */
int32_t nvfp4_abs_max(const void* x, int32_t dtype, int64_t n, float* amax_out, void* stream);

/* Quantize-on-append (step A1; [EXPL] §量子化・逆量子化フロー: new K/V are
 * quantized in 16-element blocks and appended to the NVFP4 cache).
 *   k_new, v_new : device [n_tok][num_kv_heads][128] of `dtype` (F32 or BF16)
 *   tok_seq      : device int32 [n_tok], sequence index of each row, in
 *                  [0, number of page-table rows)
 *   tok_pos      : device int32 [n_tok], token position within its sequence;
 *                  page_table[seq * max_pages_per_seq + pos / 16] must be a
 *                  valid page (< num_pages), slot pos % 16
 *   page_table   : device int32 [rows][max_pages_per_seq]
 * Writes the 128 codes and 8 block scales of each (token, head) row of K and
 * of V; nothing else in the cache changes (the V codes of the other token of
 * a pair, which share bytes with this token's, are kept).  Two rows of one
 * call must not target the same (page, slot).  n_tok == 0 is a no-op. */
int32_t nvfp4_kv_append(const nvfp4_kv_cache* cache, const void* k_new, const void* v_new,
                        int32_t dtype, int32_t n_tok, const int32_t* tok_seq,
                        const int32_t* tok_pos, const int32_t* page_table,
                        int32_t max_pages_per_seq, void* stream);

/* Quantize-on-append with a searched block scale ([EXPL] §E2M1 + 2レベル
 * スケーリング describes the NVFP4 block scale as chosen for least squared
 * error, without a procedure).  Arguments, layout, ownership and errors are
 * those of nvfp4_kv_append; only the block scale differs: among the E4M3
 * codes within 8 of the amax/6 code (code 0 excluded), the one whose element
 * codes (the usual nearest-even rounding) give the smallest squared error
 * sum_e (x_e - e2m1_e * s_block * s_t)^2 over the block, summed in double in
 * element order with every operation rounded once; ties go to the candidate
 * nearest the amax/6 code, then to the smaller code.  A block whose amax/6
 * code is 0 keeps scale 0.  The cache is read by the same decode and prefill
 * calls. */
int32_t nvfp4_kv_append_mse(const nvfp4_kv_cache* cache, const void* k_new, const void* v_new,
                            int32_t dtype, int32_t n_tok, const int32_t* tok_seq,
                            const int32_t* tok_pos, const int32_t* page_table,
                            int32_t max_pages_per_seq, void* stream);

/* NVFP4 -> FP8 conversion for an FP8 GEMM ([GB10] §這個 80 行的 Triton 繞道:
 * NVFP4 weights are converted to FP8 when a model loads, and dequantization
 * divides by the global scale).  Converts n elements of a row-major NVFP4
 * tensor [rows][cols] (cols a multiple of 16, so the tensor is a flat run
 * of n/16 blocks), e.g. a weight matrix or a cache's K codes and K scales
 * planes (whose slabs are row-major [token][128]; the V planes are not).
 *   codes       : device, n/2 bytes, element 2j in the low nibble of byte j,
 *                 16-byte aligned
 *   scales      : device, n/16 bytes, E4M3 block scales 0x00..0x7E (the
 *                 sign bit is ignored; 0x7F gives unspecified output)
 *   global_scale: the global encode scale g (finite, > 0); NVFP4 values are
 *                 e2m1 * s_block / g, so g = 1 / s_t of this library's caches
 *   out_scale   : s8 (finite, > 0); the output dequantizes as e4m3 * s8.
 *                 6 / g maps the largest NVFP4 magnitude (2688 / g) onto 448;
 *                 a power of two such as 8 / g keeps more values exact
 *   fp8_out     : device, n bytes of OCP E4M3FN codes, 16-byte aligned
 * Element: x = FP32(e2m1 * s_block) / g, then the E4M3 code nearest to
 * FP32(x / s8), ties to the even code, clamped to 448, sign of x (both
 * divisions IEEE FP32).  Reads codes and scales, writes fp8_out only.
 * n == 0 is a no-op; n < 0 or not a multiple of 16 is invalid. */
int32_t nvfp4_to_fp8(const void* codes, const void* scales, int64_t n, float global_scale,
                     float out_scale, void* fp8_out, void* stream);

/* Dequantization (step A10, for checks and fallbacks): positions
 * pos0 .. pos0+n-1 of the sequence whose page-table row is page_table_row
 * (device int32, at least ceil((pos0+n)/16) page ids in [0, num_pages))
 * into k_out and v_out,
 * each device [n][num_kv_heads][128] of out_dtype.  F32 output is
 * FP32(e2m1 * s_block * s_t); BF16 output is that value rounded to nearest
 * even.  Either output pointer may be NULL to skip it.  n == 0 is a no-op. */
int32_t nvfp4_kv_dequant(const nvfp4_kv_cache* cache, const int32_t* page_table_row,
                         int32_t pos0, int32_t n, void* k_out, void* v_out,
                         int32_t out_dtype, void* stream);

/* Number of work ranges (waves) the decode planner uses on the current
 * device: num_splits when > 0, else, with U = batch * num_kv_heads *
 * ceil(max_seq_len/16) pages and S = 4 * (compute units) SIMDs,
 * W = ceil(U / 16) (at least 16 pages per wave), or when that is below S,
 * min(S, ceil(U / 2)) (latency-bound work: up to one wave per SIMD, at least
 * 2 pages each); then at most max(compute units, 128 * batch * num_kv_heads)
 * and at most the device's resident decode wave slots, and at least 1; a
 * launch of exactly two waves per SIMD (S * 2) of an NVFP4 or MXFP4 cache
 * adds 1024 small tail ranges that the device dispatches as slots free up.
 * 0 for invalid arguments. */
int32_t nvfp4_decode_num_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len,
                                int32_t num_splits);

/* Workspace bytes nvfp4_decode_attn needs for these arguments on the
 * current device (partial results of the work ranges; 0 for invalid
 * arguments). */
size_t nvfp4_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t max_seq_len, int32_t num_splits);

/* Decode attention over the NVFP4 cache (steps A2-A8).  For each sequence b
 * and query head h (KV head h / (num_q_heads / num_kv_heads)):
 *   out[b][h] = softmax_t(q[b][h] . k_hat_t * softmax_scale) . v_hat_t,
 *   t = 0 .. seq_lens[b]-1, with k_hat, v_hat the dequantized cache
 * ([EXPL] §量子化・逆量子化フロー: dequantize, then attention; FP32
 * accumulation as in [TRTL] §Pourquoi FP8 est toujours le sol pour KV cache).
 *   q          : device [batch][num_q_heads][128], F32 or BF16
 *   page_table : device int32 [batch][max_pages_per_seq]; the first
 *                ceil(seq_lens[b]/16) entries of row b are page ids in
 *                [0, num_pages)
 *   seq_lens   : device int32 [batch], each in [0, max_seq_len];
 *                ceil(seq_lens[b]/16) <= max_pages_per_seq
 *   max_seq_len: host bound on seq_lens, used by the split planner
 *   softmax_scale: > 0 and finite (1/sqrt(128) is the usual value)
 *   num_splits : 0 = automatic, else the number of work ranges: the
 *                (sequence, KV head, page) work is cut into that many
 *                contiguous ranges, one per wave; equal ranges, except that
 *                exactly two waves per SIMD (2 x 4 x CUs) give the first
 *                4 x CUs waves 8/5 of the others' share (the SIMD favours
 *                its older wave).  The split changes rounding only within
 *                the stated tolerance, and a given split is deterministic.
 *   workspace  : device, >= nvfp4_decode_workspace_bytes(...) bytes,
 *                256-byte aligned
 *   out        : device FP32 [batch][num_q_heads][128]
 * A sequence of length 0 yields zeros.  Results do not depend on the run:
 * no atomics, fixed reduction order. */
int32_t nvfp4_decode_attn(const nvfp4_kv_cache* cache, const void* q, int32_t q_dtype,
                          int32_t batch, int32_t num_q_heads, const int32_t* page_table,
                          int32_t max_pages_per_seq, const int32_t* seq_lens,
                          int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, float* out, void* stream);

/* Page-gather ceiling of the NVFP4 decode (a measurement aid beside the hot
 * path): runs the decode kernel's wave ranges, page walk and page loads over
 * the cache exactly as nvfp4_decode_attn with bf16 queries and these
 * arguments would, but consumes each page with an exclusive or instead of
 * the attention math, and runs no merge.  Its time is what the decode's own
 * access pattern costs without the math.
 *   page_table, max_pages_per_seq, seq_lens, max_seq_len, num_splits: as for
 *                nvfp4_decode_attn (same wave ranges)
 *   sink       : device, >= 256 * (wave count) bytes; one 32-bit word per
 *                lane is written: the exclusive or of the words the lane
 *                loaded (0 for waves without units), so the exclusive or of
 *                all words is that of every (page, KV head) slab the
 *                sequences own (K codes and V codes as 32-bit words, K
 *                scales as 16-bit words; V scales are loaded by lane pairs
 *                and cancel)
 * Planes beyond 2^31 bytes are not supported (NVFP4_ERR_UNSUPPORTED). */
int32_t nvfp4_decode_gather_probe(const nvfp4_kv_cache* cache, int32_t batch, const int32_t* page_table,
                                  int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                  int32_t num_splits, void* sink, size_t sink_bytes, void* stream);

/* Bytes of the fixed device scratch of nvfp4_decode_attn_noalloc (40 MiB:
 * every automatic split of up to 8 waves per CU on 256 CUs with up to 16
 * query heads per KV head fits). */
#define NVFP4_DECODE_NOALLOC_SCRATCH_BYTES 41943040

/* Decode attention that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation).  The operation, arguments, work split, results and
 * errors are those of nvfp4_decode_attn without the workspace: the partial
 * results live in a fixed scratch of NVFP4_DECODE_NOALLOC_SCRATCH_BYTES bytes
 * that the library keeps in each device's memory from the first call on that
 * device until the process ends.  A call whose partial results need more
 * than that (the size nvfp4_decode_workspace_bytes reports for the same
 * arguments) fails with NVFP4_ERR_WORKSPACE before enqueueing anything.
 * Every call on one device uses that device's one scratch, which keeps the
 * last call's contents: calls that may overlap on one device (other streams,
 * other threads) race, and the caller must serialize them.  The call makes
 * no hipMalloc or hipFree and no allocating library call. */
int32_t nvfp4_decode_attn_noalloc(const nvfp4_kv_cache* cache, const void* q, int32_t q_dtype,
                                  int32_t batch, int32_t num_q_heads, const int32_t* page_table,
                                  int32_t max_pages_per_seq, const int32_t* seq_lens,
                                  int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                                  float* out, void* stream);

/* Operand precision of the prefill path. */
typedef enum nvfp4_prefill_mode {
  NVFP4_PREFILL_FP8 = 0,  /* the pages' flow: FP8 operands (E4M3 rounding of
                             the dequantized cache, of Q and of P) */
  NVFP4_PREFILL_F16 = 1   /* exact 16-bit operands (the dequantized cache is
                             exact in FP16); half the FP8 MFMA rate */
} nvfp4_prefill_mode;

/* Workspace bytes nvfp4_prefill_attn needs (0 for invalid arguments): the
 * expanded K and V of the sequence, 1 (FP8) or 2 (F16) bytes per element. */
size_t nvfp4_prefill_workspace_bytes(int32_t num_tokens, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t prefix_len, int32_t mode);

/* Chunked-prefill attention (step A9; [EXPL] §量子化・逆量子化フロー: the
 * NVFP4 cache is dequantized to FP8 and attention runs on FP8 operands with
 * an FP32 accumulator; mode NVFP4_PREFILL_F16 keeps the dequantized values
 * exact instead).  The chunk's own K/V must already be appended.
 *   q             : device [num_tokens][num_q_heads][128], F32 or BF16
 *   page_table_row: device int32, ceil((prefix_len+num_tokens)/16) page ids
 *                   in [0, num_pages)
 *   causal != 0   : query i (absolute position prefix_len + i) attends to
 *                   tokens 0 .. prefix_len + i; causal == 0: to all
 *                   prefix_len + num_tokens tokens
 *   mode          : an nvfp4_prefill_mode
 *   workspace     : device, >= nvfp4_prefill_workspace_bytes(...), 256-byte
 *                   aligned
 *   out           : device FP32 [num_tokens][num_q_heads][128]
 * num_tokens == 0 is a no-op. */
int32_t nvfp4_prefill_attn(const nvfp4_kv_cache* cache, const void* q, int32_t q_dtype,
                           int32_t num_tokens, int32_t num_q_heads,
                           const int32_t* page_table_row, int32_t prefix_len, int32_t causal,
                           int32_t mode, float softmax_scale, void* workspace,
                           size_t workspace_bytes, float* out, void* stream);

/* ------------------------------------------------ comparison KV formats
 * The formats NVFP4 is measured against ([EXPL] §なぜ4ビット量子化が必要か and
 * §メモリ削減効果: FP8 caches are in wide use and NVFP4 halves their bytes;
 * FP16/BF16 is the unquantized baseline; [TRTL] §Pourquoi FP8 est toujours le
 * sol pour KV cache), stored in the same paging and decoded by the same
 * decode kernel, so that the speed ratio of the formats can be measured.
 *
 *   NVFP4_CMP_FP8 : each element is an OCP E4M3FN byte, the value nearest to
 *                   x / s_t (FP32 quotient), ties to the even code, clamped
 *                   to 448; one FP32 tensor scale s_t per K and per V, e.g.
 *                   amax(|X|) / 448 (nvfp4_cmp_fp8_scale_from_amax); a
 *                   value is e4m3 * s_t.  1 byte per element.
 *   NVFP4_CMP_BF16: each element is the bf16 value (F32 input rounded to
 *                   nearest even, BF16 input copied); the scales are unused.
 *                   2 bytes per element.
 * Layout: two planes k and v, each [num_pages][num_kv_heads][slab] with E
 * bytes per element (1 or 2):
 *   k slab 16 * 128 * E: [token 16][element 128];
 *   v slab 16 * 128 * E: [token quad 4][element 128][token 4], i.e. element
 *                        d of token t at ((t/4) * 128 + d) * 4 + t%4 (in
 *                        elements), so that the four tokens of a quad at one
 *                        element are adjacent (the operand order of PV).
 */
typedef enum nvfp4_cmp_format {
  NVFP4_CMP_FP8 = 1,
  NVFP4_CMP_BF16 = 2
} nvfp4_cmp_format;

/* Host description of a paged comparison-format cache (one layer).  k and v
 * are 16-byte aligned device planes; for FP8 the scales must be finite and
 * > 0. */
typedef struct nvfp4_cmp_cache {
  void* k;
  void* v;
  float k_scale;
  float v_scale;
  int32_t format;      /* an nvfp4_cmp_format */
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t page_size;   /* must be 16 */
  int32_t head_dim;    /* must be 128 */
} nvfp4_cmp_cache;

/* Bytes of one plane (k or v): num_pages * num_kv_heads * 16 * 128 * E.
 * 0 for invalid arguments. */
size_t nvfp4_cmp_plane_bytes(int32_t num_pages, int32_t num_kv_heads, int32_t format);

/* FP8 tensor scale: amax / 448 in FP32; 0 when amax is not finite or not > 0. */
float nvfp4_cmp_fp8_scale_from_amax(float amax);

/* Append rows to a comparison-format cache; the arguments and index rules
 * are those of nvfp4_kv_append.  Writes each (token, head) row of K and V;
 * nothing else changes.  n_tok == 0 is a no-op. */
int32_t nvfp4_cmp_append(const nvfp4_cmp_cache* cache, const void* k_new, const void* v_new,
                         int32_t dtype, int32_t n_tok, const int32_t* tok_seq,
                         const int32_t* tok_pos, const int32_t* page_table,
                         int32_t max_pages_per_seq, void* stream);

/* Workspace bytes of nvfp4_cmp_decode_attn (0 for invalid arguments). */
size_t nvfp4_cmp_decode_workspace_bytes(int32_t format, int32_t batch, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t max_seq_len,
                                        int32_t num_splits);

/* Decode attention over a comparison-format cache: the operation, arguments
 * and work split of nvfp4_decode_attn (with equal ranges at every wave
 * count: these pages are bound by HBM, not by the SIMD), with the cached
 * values of the format (FP8: e4m3 * s_t, exact in FP16 and expanded to it;
 * BF16: the bf16 values, multiplied in bf16 with P carried as two bf16
 * parts). */
int32_t nvfp4_cmp_decode_attn(const nvfp4_cmp_cache* cache, const void* q, int32_t q_dtype,
                              int32_t batch, int32_t num_q_heads, const int32_t* page_table,
                              int32_t max_pages_per_seq, const int32_t* seq_lens,
                              int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                              void* workspace, size_t workspace_bytes, float* out, void* stream);

/* ---------------------------------------------------------------- MXFP4
 *
 * An MXFP4 KV cache, the OCP format set against NVFP4 in [EXPL]
 * §MXFP4との比較 (table: 32-element blocks, E8M0 power-of-two scales, no
 * tensor scale), with the same paging and decode as NVFP4.
 * Codec (per (token, head) row of 128 elements, 4 blocks of 32): block
 * exponent e = floor(log2(block amax)) - 2, clamped to [-127, 127], -127 for
 * a zero block; scale byte e + 127 (E8M0); element code = the E2M1
 * magnitude nearest to |x| / 2^e, ties to the even code, clamped to 6, sign
 * bit from x.  Value = e2m1 * 2^(scale - 127).
 * Layout: the code planes are those of the NVFP4 cache (K [token][64 B],
 * V token pairs sharing bytes); the scale planes hold 64 bytes per
 * (page, head) slab:
 *   k_scales slab 64 B: [token 16][block 4];
 *   v_scales slab 64 B: [block 4][token 16].
 * 0.53125 bytes per element; K and V of one (page, head) are 2176 bytes.
 *
 * Decode multiplies exact FP16 operands: K and V values are taken relative
 * to 2^exp_offset (the cache's k_exp_offset, v_exp_offset) and the power of
 * two is applied to the scores and the output.  Values are exact when the
 * block exponents lie within [exp_offset - 23, exp_offset + 13];
 * nvfp4_mx_exp_offset_from_amax gives the offset that puts a tensor's
 * largest block at exp_offset + 8, so a block loses exactness only when its
 * amax is below about 2^-31 of the tensor's (a negligible contribution).
 */
typedef struct nvfp4_mx_cache {
  uint8_t* k_codes;
  uint8_t* k_scales;
  uint8_t* v_codes;
  uint8_t* v_scales;
  int32_t k_exp_offset;  /* in [-126, 127] */
  int32_t v_exp_offset;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t page_size;     /* must be 16 */
  int32_t head_dim;      /* must be 128 */
} nvfp4_mx_cache;

/* Bytes of one plane: plane 0 k_codes, 1 k_scales, 2 v_codes, 3 v_scales
 * (codes num_pages * num_kv_heads * 1024, scales num_pages * num_kv_heads *
 * 64).  0 for invalid arguments. */
size_t nvfp4_mx_plane_bytes(int32_t num_pages, int32_t num_kv_heads, int32_t plane);

/* floor(log2(amax)) - 10 for a tensor's amax (finite, > 0), else 0. */
int32_t nvfp4_mx_exp_offset_from_amax(float amax);

/* Quantize rows to MXFP4 and append them; arguments, index rules and
 * ownership are those of nvfp4_kv_append (the exp offsets are not used).
 * Writes the 128 codes and 4 block scales of each (token, head) row of K and
 * of V; nothing else changes. */
int32_t nvfp4_mx_append(const nvfp4_mx_cache* cache, const void* k_new, const void* v_new,
                        int32_t dtype, int32_t n_tok, const int32_t* tok_seq,
                        const int32_t* tok_pos, const int32_t* page_table,
                        int32_t max_pages_per_seq, void* stream);

/* Workspace bytes of nvfp4_mx_decode_attn (0 for invalid arguments). */
size_t nvfp4_mx_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t max_seq_len, int32_t num_splits);

/* Decode attention over an MXFP4 cache: the operation, arguments and work
 * split of nvfp4_decode_attn, with the MXFP4 values of the cache. */
int32_t nvfp4_mx_decode_attn(const nvfp4_mx_cache* cache, const void* q, int32_t q_dtype,
                             int32_t batch, int32_t num_q_heads, const int32_t* page_table,
                             int32_t max_pages_per_seq, const int32_t* seq_lens,
                             int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                             void* workspace, size_t workspace_bytes, float* out, void* stream);

/* Workspace bytes of nvfp4_mx_prefill_attn (0 for invalid arguments): the
 * expanded V of the sequence, 1 byte per element (K is not expanded). */
size_t nvfp4_mx_prefill_workspace_bytes(int32_t num_tokens, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t prefix_len);

/* Chunked-prefill attention over an MXFP4 cache: the operation and arguments
 * of nvfp4_prefill_attn on FP8-class matrix products ([EXPL]
 * §量子化・逆量子化フロー; §MXFP4との比較 for the format).  K enters the score
 * products as the cache's own E2M1 codes with their E8M0 block scales (the
 * block-scaled FP4 x FP8 matrix instruction; exact K), Q as E4M3 with a
 * power-of-two scale per (row, head), P as E4M3, and V as E4M3 of
 * e2m1 * 2^(e - r) with r = min(v_exp_offset + 2, 125): exact for blocks
 * within [v_exp_offset - 12, v_exp_offset + 8] (the range
 * nvfp4_mx_exp_offset_from_amax sets for the tensor it was computed from),
 * rounded below, saturated at 448 * 2^r above.  The chunk's own K/V must
 * already be appended (nvfp4_mx_append).  Accumulation in FP32.
 *   page_table_row, causal, q, out: as in nvfp4_prefill_attn
 *   workspace: device, >= nvfp4_mx_prefill_workspace_bytes(...), 256-byte
 *              aligned
 * num_tokens == 0 is a no-op. */
int32_t nvfp4_mx_prefill_attn(const nvfp4_mx_cache* cache, const void* q, int32_t q_dtype,
                              int32_t num_tokens, int32_t num_q_heads,
                              const int32_t* page_table_row, int32_t prefix_len, int32_t causal,
                              float softmax_scale, void* workspace, size_t workspace_bytes,
                              float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4KV_H */
