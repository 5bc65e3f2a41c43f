/*
 * bdfp4 — NVFP4 / MXFP4 KV-cache page quantization and paged FP4 decode
 * attention for AMD MI355X (gfx950).
 *
 * C ABI. Every pointer argument is a plain device pointer (allocated by the
 * caller, for example as a torch tensor) unless the comment says "host".
 * The library never allocates or frees memory and keeps no pointer after a
 * call returns. Its one piece of state is the fixed workspace array of
 * bdfp4_decode_attention_noalloc (one per GPU, in the library's static device
 * memory). Launches are asynchronous on the given stream (a hipStream_t
 * passed as void*; NULL is the null stream).
 *
 * Errors: every entry point validates its recipe, shapes, pointers and
 * alignment on the host before enqueuing anything. On any error it returns a
 * negative bdfp4_status and enqueues nothing; bdfp4_last_error() then
 * describes the failure (thread-local, valid until the next call on the same
 * thread). A failed launch returns BDFP4_E_HIP.
 *
 * Sources of the method (three web pages): "BitDecoding-FP4
 * evaluation/config.py" (OpenBitSys/BitDecoding-FP4: RECIPE,
 * recipe_additional_config, probability_environment, KV_MODES,
 * PARITY_ENGINE_KWARGS), "kv-landlords scripts/quant_ab.py" (module
 * docstring, mem_ratio, PageSim) and the gitdiagram summary "How
 * openbitsys/bitdecoding-fp4 works" (components KV cache writer, KV
 * quantization, Decode interface, Paged attention kernel, Block scaling,
 * Scale modes). The pages name the scale modes and constants but print no
 * formulas; the readings this library implements are stated at each entry.
 *
 * Shapes are fixed by the method: head_dim = 128 and block_size (tokens per
 * page) = 128 ("block_size": 128 in PARITY_ENGINE_KWARGS).
 */
#ifndef BDFP4_H
#define BDFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BDFP4_OK = 0,
  BDFP4_E_INVALID = -1,      /* bad argument, shape, pointer or alignment     */
  BDFP4_E_UNCALIBRATED = -2, /* tau is still "calibrate" (NaN)                */
  BDFP4_E_UNSUPPORTED = -3,  /* valid for the method, not built here          */
  BDFP4_E_WORKSPACE = -4,    /* workspace missing or too small                */
  BDFP4_E_HIP = -5           /* a HIP launch or runtime call failed           */
} bdfp4_status;

/* Scale modes (names from recipe_additional_config and probability_environment):
 *   AMAX6          one E4M3 scale per 16 elements, s = E4M3(amax / 6)
 *   FOUR_SIX       per 16 elements, the better (lower float32 squared error,
 *                  ties keep 6) of s = E4M3(amax/6) and s = E4M3(amax/4)
 *   MXFP4_SEARCH   one E8M0 scale 2^E per 32 elements, the better of E_hi
 *                  (least E with amax <= 6 * 2^E) and E_hi - 1
 *   AMAX2_OR_AMAX6 probabilities only: on p' = c * p per 16-token block,
 *                  s = E4M3(a/2) if a < tau else E4M3(a/6), a = max p'
 *   NONE           not quantized (debug/oracle use; decode rejects it)
 * E4M3 rounding is to nearest, ties to even, saturating at 448. E2M1 codes are
 * the nearest grid point of the exact ratio |x|/s (grid 0, .5, 1, 1.5, 2, 3,
 * 4, 6; ties to the even code; saturating at 6), sign = sign bit of x; a zero
 * scale gives all-zero codes. */
enum {
  BDFP4_SCALE_NONE = 0,
  BDFP4_SCALE_AMAX6 = 1,
  BDFP4_SCALE_FOUR_SIX = 2,
  BDFP4_SCALE_MXFP4_SEARCH = 3,
  BDFP4_SCALE_AMAX2_OR_AMAX6 = 4
};

/* The BitDecoding recipe ("BitDecoding-FP4 evaluation/config.py": RECIPE,
 * recipe_additional_config, probability_environment, KV_MODES). */
typedef struct {
  int32_t sink_tokens;   /* BF16 sink length: multiple of 16 in [0, 112]; 16 in
                            the bitdecoding-nvfp4 / -mxfp4 modes                */
  int32_t rotation;      /* 1: 128-point Hadamard rotation of keys and query;
                            0: none                                            */
  int32_t key_smoothing; /* 1: subtract the static per-channel key mean before
                            rotation (key_shift argument required)            */
  int32_t scale_mode_k;  /* FOUR_SIX | AMAX6 | MXFP4_SEARCH                    */
  int32_t scale_mode_v;  /* AMAX6 | MXFP4_SEARCH                               */
  int32_t scale_mode_q;  /* AMAX6 | MXFP4_SEARCH                               */
  int32_t scale_mode_p;  /* AMAX2_OR_AMAX6 (scaling enabled) | AMAX6 (disabled)*/
  int32_t query_terms;   /* 2: q ~ Q1 + Q2 (residual); 1: Q1 only              */
  int32_t c;             /* probability multiplier, 1 or 8                     */
  float tau;             /* threshold, finite in [0, 448]; NaN = "calibrate"  */
  int32_t rotate_v;      /* recipe variant, 0 in both modes: 1 rotates values
                            with the same Hadamard rotation before they are
                            quantized, and the decode rotates its output back */
  int32_t p_running_max; /* recipe variant, 0 in both modes: 1 normalises the
                            P of each 16-token block by the running maximum
                            over the partition's blocks up to it (one-pass
                            softmax) instead of the partition maximum, and
                            weights it back; NVFP4 K/V, two query terms and
                            AMAX2_OR_AMAX6 only (else E_UNSUPPORTED)          */
  int32_t key_scale_geometry; /* BDFP4_KEY_GEOMETRY_LOCAL (default of both
                            modes: a key block is 16 channels of one token)
                            or BDFP4_KEY_GEOMETRY_CHANNEL (16 tokens of one
                            channel, KV_MODES key_scale_geometry; quant_ab.py
                            SCHEMES per-channel keys): NVFP4 keys (FOUR_SIX
                            or AMAX6) and no p_running_max, else
                            E_UNSUPPORTED                                     */
} bdfp4_recipe;

enum { BDFP4_KEY_GEOMETRY_LOCAL = 0, BDFP4_KEY_GEOMETRY_CHANNEL = 1 };

/* The quantized paged cache. Each of the four arrays is dense
 * [num_pages][num_kv_heads][bytes per page-head]; the block of (page p, head h)
 * starts at (p * num_kv_heads + h) * bytes. Sizes from bdfp4_cache_bytes().
 * Byte order inside a block (t = token in page 0..127, d = element 0..127,
 * j = scale block; two codes per byte):
 *   K codes (8192 B; elements d, d+1 of token t, d even in bits 3..0):
 *     (t>>4)*1024 + (d>>5)*256 + (t&15)*16 + ((d&31)>>1)
 *   V codes, NVFP4 (8192 B; tokens t, t+1 of element d, t even in bits 3..0):
 *     (t>>5)*2048 + (((t>>3)&3)*16 + (d>>3))*32 + (d&7)*4 + ((t&7)>>1)
 *   V codes, MXFP4 (8192 B; elements d, d+1 of token t, d even in bits 3..0):
 *     ((((t>>5)*4 + ((t>>3)&3))*16 + (d>>3))*8 + (t&7))*4 + ((d&7)>>1)
 *   K scales, NVFP4 (1024 B, j = d>>4): (((j>>1)*16 + (t&15))*8 + (t>>4))*2 + (j&1)
 *   K scales, MXFP4 (512 B, j = d>>5):  (j*16 + (t&15))*8 + (t>>4)
 *   K scales, NVFP4, channel key geometry (1024 B, token block b = t>>4):
 *     b*128 + d
 *   V scales, NVFP4 (1024 B): (((t>>5)*4 + ((t>>3)&3))*8 + j)*8 + (t&7)
 *   V scales, MXFP4 (512 B):  (((t>>5)*4 + ((t>>3)&3))*4 + j)*8 + (t&7)
 * All four pointers 16-byte aligned. */
typedef struct {
  void* k_codes;
  void* k_scales;
  void* v_codes;
  void* v_scales;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t head_dim;   /* must be 128 */
  int32_t block_size; /* must be 128 */
} bdfp4_cache;

/* Fill *r with the bitdecoding-nvfp4 recipe (sink 16, Hadamard, key
 * smoothing, K four_six, V/Q amax6, P amax2_or_amax6, 2 query terms, c = 8,
 * tau = NaN i.e. still to be calibrated). */
bdfp4_status bdfp4_recipe_default_nvfp4(bdfp4_recipe* r);

/* Same for bitdecoding-mxfp4 (K, V and Q mxfp4_search). */
bdfp4_status bdfp4_recipe_default_mxfp4(bdfp4_recipe* r);

/* Host-only check of a recipe, mirroring probability_environment: c not in
 * {1, 8} -> E_INVALID; tau NaN ("calibrate") -> E_UNCALIBRATED; tau not finite
 * or outside [0, 448] -> E_INVALID; other fields outside their ranges ->
 * E_INVALID; combinations this library has no kernel for (mixed NVFP4/MXFP4
 * tensors, NONE modes) -> E_UNSUPPORTED. */
bdfp4_status bdfp4_recipe_validate(const bdfp4_recipe* r);

/* Bytes of each cache array for num_pages pages (host outputs). */
bdfp4_status bdfp4_cache_bytes(const bdfp4_recipe* r, int32_t num_pages,
                               int32_t num_kv_heads, size_t* k_codes,
                               size_t* k_scales, size_t* v_codes,
                               size_t* v_scales);

/* KV page writer ("KV cache writer -> KV quantization" in the gitdiagram;
 * freeze-at-fill pages as in PageSim of quant_ab.py): quantize n_pages whole
 * pages of BF16 keys and values into the cache.
 *   k_bf16, v_bf16: [n_pages * 128][num_kv_heads][128] bf16, row-major; input
 *                   page i is rows [128 i, 128 i + 128). 16-byte aligned.
 *   page_ids:       int32 [n_pages], destination physical page of input page
 *                   i; entries outside [0, num_pages) are skipped.
 *   key_shift:      float32 [num_kv_heads][128] static key means mu; required
 *                   iff recipe->key_smoothing (NULL otherwise).
 * Keys: x = float32(k) - mu, y = H x / sqrt(128) (fast Walsh-Hadamard,
 * stages h = 1..64, float32), then scale_mode_k. Values: scale_mode_v on
 * float32(v), no rotation. Codes and scales are bit-exact functions of the
 * inputs. n_pages = 0 is a no-op; n_pages * num_kv_heads >= 2^24 (more than
 * one call's grid holds) -> E_INVALID. */
bdfp4_status bdfp4_quantize_pages(const bdfp4_recipe* r, const bdfp4_cache* cache,
                                  const void* k_bf16, const void* v_bf16,
                                  const int32_t* page_ids, int32_t n_pages,
                                  const float* key_shift, void* stream);

/* Decode-time append with freeze-at-fill ("kv-landlords scripts/quant_ab.py"
 * PageSim: the hot page stays BF16 and is quantized once, when it fills;
 * "BitDecoding-FP4 evaluation/config.py" KV_MODES "sink_tokens": 16). One new
 * token per sequence, at 0-based position positions[b] (device int32 [batch]):
 *   k_new, v_new:  bf16 [batch][num_kv_heads][128], 16-byte aligned.
 *   tail_k/v:      bf16 [batch][num_kv_heads][128][128] (the buffers
 *                  bdfp4_decode_attention reads); the token goes to slot
 *                  positions[b] mod 128.
 *   sink_k/v:      bf16 [batch][num_kv_heads][sink_tokens][128]; a token with
 *                  position < sink_tokens is also written at that index.
 *                  May be NULL when sink_tokens = 0.
 *   block_tables:  int32 [batch][max_pages_per_seq], as for the decode.
 *   key_shift:     as for bdfp4_quantize_pages.
 * The token that fills slot 127 freezes the page: its 128 tail rows (slots
 * 0..126 written by earlier calls, slot 127 this one) are quantized exactly
 * as bdfp4_quantize_pages quantizes a whole page, into physical page
 * block_tables[b][positions[b] / 128]; a page outside [0, num_pages) is
 * skipped (the tail is still written). Rows with positions[b] < 0 (padding)
 * or >= 128 * max_pages_per_seq are skipped entirely. The caller advances
 * its sequence lengths afterwards (the decode after this call uses
 * L = positions[b] + 1). Sequences of one call must not share tail, sink or
 * destination pages. batch = 0 is a no-op. */
bdfp4_status bdfp4_append_tokens(const bdfp4_recipe* r, const bdfp4_cache* cache,
                                 const void* k_new, const void* v_new, int32_t batch,
                                 const int32_t* positions, const int32_t* block_tables,
                                 int32_t max_pages_per_seq, void* sink_k, void* sink_v,
                                 void* tail_k, void* tail_v, const float* key_shift,
                                 void* stream);

/* Calibration of the key means ("BitDecoding-FP4 evaluation/config.py",
 * RECIPE outlier_aware_key_quantization: key smoothing with a static key
 * shift, created by a calibration pass when missing). mu_out[h][c] (float32
 * [num_kv_heads][128], device) = the mean over the calibration tokens of
 * float32(k[t][h][c]), summed in float64 in a fixed order (results do not
 * depend on scheduling; the sum starts from +0.0, so zeros of either sign
 * give +0.0) and rounded to float32 once.
 *   k_bf16:    [tokens][num_kv_heads][128] bf16, the rows bdfp4_quantize_pages
 *              takes; 16-byte aligned.
 *   workspace: device scratch of bdfp4_key_means_workspace_size bytes (no
 *              initialization needed; contents undefined afterwards).
 * E_INVALID for tokens < 1, num_kv_heads outside [1, 65535], NULL or
 * misaligned pointers; E_WORKSPACE for a short workspace. */
bdfp4_status bdfp4_key_means_workspace_size(int32_t tokens, int32_t num_kv_heads, size_t* bytes);
bdfp4_status bdfp4_key_means(const void* k_bf16, int32_t tokens, int32_t num_kv_heads,
                             void* workspace, size_t workspace_bytes, float* mu_out,
                             void* stream);

/* Error sums for calibration and diagnostics: sums_out[0] = sum over i < n
 * of (got[i] - ref[i])^2 and sums_out[1] = sum of ref[i]^2, in float64 in a
 * fixed order (device pointers; sums_out 8-byte aligned, two doubles). The
 * tau search ("calibrate" in probability_environment) compares decode
 * outputs for candidate taus with exact attention through these sums.
 * n in [0, 2^31] (got and ref may be NULL when n = 0, which writes two
 * zeros); one workgroup, meant for outputs and small tensors. */
bdfp4_status bdfp4_error_sums(const float* got, const float* ref, int64_t n, double* sums_out,
                              void* stream);

/* The tau choice of the calibration search (host only; config.py
 * probability_environment leaves tau to calibration and states no
 * objective): candidate i's error is the relative L2 error
 * sqrt(sums[2i] / sums[2i + 1]) of its decode output against exact
 * attention (the two sums of bdfp4_error_sums, copied to the host; a zero
 * reference sum gives 0 for a zero error, else +inf; a NaN error counts as
 * +inf). The smallest error wins and ties keep the earlier candidate.
 *   sums: host double [n][2]; candidates: host float [n]; n >= 1;
 *   best_tau: host, the chosen candidate; best_index: host or NULL;
 *   rel_errors: host double [n] or NULL, each candidate's error.
 * E_INVALID for n < 1, NULL inputs, negative sums, or when every error is
 * NaN. */
bdfp4_status bdfp4_select_tau(const double* sums, const float* candidates, int32_t n, float* best_tau,
                              int32_t* best_index, double* rel_errors);

/* Quantization diagnostics ("kv-landlords scripts/quant_ab.py" compares
 * cache schemes by reconstruction error; the recipe ablations of
 * "BitDecoding-FP4 evaluation/config.py"): for n_pages pages written from
 * k_bf16 / v_bf16 / page_ids / key_shift (the arguments bdfp4_quantize_pages
 * took), sums_out (device double[4]) = [sum (k_hat - y)^2, sum y^2,
 * sum (v_hat - v)^2, sum v^2] over every element, where y are the keys as
 * quantized (centered and rotated in float32 exactly as the writer does)
 * and k_hat, v_hat the values the cache holds (codes times scales, read
 * through the layout above). Float64, fixed summation order. Pages whose
 * destination is outside [0, num_pages) contribute nothing. workspace:
 * bdfp4_page_errors_workspace_size bytes, 16-byte aligned, no
 * initialization needed. */
bdfp4_status bdfp4_page_errors_workspace_size(int32_t n_pages, int32_t num_kv_heads, size_t* bytes);
bdfp4_status bdfp4_page_errors(const bdfp4_recipe* r, const bdfp4_cache* cache,
                               const void* k_bf16, const void* v_bf16,
                               const int32_t* page_ids, int32_t n_pages,
                               const float* key_shift, void* workspace,
                               size_t workspace_bytes, double* sums_out, void* stream);

/* Split plan of bdfp4_decode_attention (host). pages_per_partition (1 .. 4)
 * is the number of consecutive full pages one FP4 partition covers; 0 picks
 * it from (batch, num_kv_heads, max_seq_len) for the MI355X's 256 compute
 * units: the smallest value that keeps the workgroups of four partitions
 * within 256 when one of up to 4 pages does (the launch then also gives
 * the BF16 partitions workgroups of their own), else about 512. The chosen
 * value and the number of FP4 partitions of the longest sequence are
 * returned. */
bdfp4_status bdfp4_decode_plan(int32_t batch, int32_t num_kv_heads,
                               int32_t max_seq_len, int32_t pages_per_partition,
                               int32_t* pages_per_partition_out,
                               int32_t* max_partitions_out);

/* Split plan of bdfp4_bf16_decode_attention (host). pages_per_partition
 * (1 .. 16) is the number of consecutive pages, the partial last one
 * included, that one workgroup covers (its 4 waves share them); 0 picks
 * ceil(batch * num_kv_heads * ceil(max_seq_len / 128) / 512), at most 16:
 * about 512 workgroups, the fastest grid measured on the MI355X (one
 * resident round). The chosen value and the number of partitions of the
 * longest sequence are returned. */
bdfp4_status bdfp4_bf16_decode_plan(int32_t batch, int32_t num_kv_heads,
                                    int32_t max_seq_len, int32_t pages_per_partition,
                                    int32_t* pages_per_partition_out,
                                    int32_t* max_partitions_out);

/* Workspace bytes for bdfp4_decode_attention / bdfp4_bf16_decode_attention
 * with these sizes (host output): a fixed ticket region of
 * 16384 * 128 bytes (one 128-byte line per ticket; the same for every call
 * shape), then
 * batch * num_kv_heads * S partial slots of 2080 bytes, S = P + 2 rounded up
 * to even (the slots are stored in pairs), where
 * P = ceil(ceil(max_seq_len / 128) / pages_per_partition).
 * pages_per_partition 0 sizes for the larger of the two decodes' automatic
 * plans, 1 .. 4 for that value (either decode), 5 .. 16 for the BF16 decode
 * with that value. The workspace must
 * be zero-filled once after it is allocated; every call leaves its ticket
 * words zero again, so a buffer can be reused by calls of any shape (and
 * captured in a graph) without clearing. After a call that did not complete
 * (process killed, device error) zero it again. Calls that share one
 * workspace must not overlap in time. */
bdfp4_status bdfp4_decode_workspace_size(int32_t batch, int32_t num_q_heads,
                                         int32_t num_kv_heads,
                                         int32_t max_seq_len,
                                         int32_t pages_per_partition,
                                         size_t* bytes);

/* Paged FP4 decode attention ("Decode interface -> Paged attention kernel").
 *   q_bf16:        [batch][num_q_heads][128] bf16; query head g reads KV head
 *                  g / (num_q_heads / num_kv_heads). num_q_heads / num_kv_heads
 *                  must be 4 (the GQA group this library supports).
 *   block_tables:  int32 [batch][max_pages_per_seq] physical page of each
 *                  logical page.
 *   seq_lens:      int32 [batch] context length L (tokens), device memory.
 *   max_seq_len:   host upper bound of seq_lens (sizes the grid).
 *   sink_k/v:      bf16 [batch][num_kv_heads][sink_tokens][128]: tokens
 *                  [0, sink_tokens), kept in BF16 (KV_MODES "sink_tokens": 16).
 *   tail_k/v:      bf16 [batch][num_kv_heads][128][128]: the partial page;
 *                  slot j holds token 128 * floor(L / 128) + j.
 *   key_shift:     float32 [num_kv_heads][128], the means the keys were
 *                  centered with (required iff key_smoothing).
 *   softmax_scale: sigma, applied to the float32 logits.
 *   out:           float32 [batch][num_q_heads][128].
 * Tokens [sink, 128 * floor(L/128)) are read from the FP4 pages, the sink and
 * tokens [max(sink, 128 floor(L/128)), L) from the BF16 buffers. The query is
 * rotated and quantized as Q1 + Q2 (scale_mode_q); an FP4 token's logit is
 * sigma * (q_hat . k_hat + q . mu). Partition 0 holds the BF16 tokens (exact
 * float32 attention); partitions 1..S hold pages_per_partition (1 .. 4)
 * consecutive full pages each (the last may hold fewer).
 * Per partition: m = max logit, p = exp(t - m), l = sum p; FP4 partitions
 * quantize p' = c p per 16-token block (scale_mode_p, tau) and accumulate
 * P_hat = s e2m1 / c times v_hat. Partitions are merged by log-sum-exp.
 * A sequence with L < 1 or L > max_seq_len or more full pages than
 * max_pages_per_seq, or whose block table names a page outside
 * [0, num_pages), gets NaN outputs. */
bdfp4_status bdfp4_decode_attention(
    const bdfp4_recipe* r, const bdfp4_cache* cache, const void* q_bf16,
    int32_t batch, int32_t num_q_heads, const int32_t* block_tables,
    int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
    const void* sink_k, const void* sink_v, const void* tail_k,
    const void* tail_v, const float* key_shift, float softmax_scale,
    int32_t pages_per_partition, void* workspace, size_t workspace_bytes,
    float* out, void* stream);

/* bdfp4_decode_attention without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. Arguments, results and errors are
 * those of bdfp4_decode_attention (the same kernels). The tickets and
 * partials live in a static device array of the library,
 * bdfp4_decode_noalloc_max_workspace() bytes (16 MiB) per GPU, held until the
 * process ends; its address on the current device is looked up on the first
 * call there, which also enqueues the zeroing of its ticket words on
 * `stream`. The call allocates nothing. A call whose plan needs more
 * workspace than the array holds (bdfp4_decode_workspace_size) returns
 * BDFP4_E_WORKSPACE and enqueues nothing. Every call on one GPU shares that
 * array: calls that may overlap in time on one GPU (two streams, two host
 * threads) race and must be serialized by the caller. */
bdfp4_status bdfp4_decode_attention_noalloc(
    const bdfp4_recipe* r, const bdfp4_cache* cache, const void* q_bf16,
    int32_t batch, int32_t num_q_heads, const int32_t* block_tables,
    int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
    const void* sink_k, const void* sink_v, const void* tail_k,
    const void* tail_v, const float* key_shift, float softmax_scale,
    int32_t pages_per_partition, float* out, void* stream);

/* Size in bytes of the allocation-free decode's workspace array. */
size_t bdfp4_decode_noalloc_max_workspace(void);

/* Debug entry: bdfp4_decode_attention that also writes the raw logit
 * q . mu + q_hat . k_hat (float32, before sigma) of every FP4 token, as the
 * decode computes it before the partition maximum and P quantization:
 *   logits: float32 [batch][num_kv_heads][4][128 * max_pages_per_seq], token
 *           at its logical position; the sink slots of page 0 hold -inf;
 *           BF16 tokens and positions past the full pages are not written.
 * Used to count how often float32 logits change a P code or scale. */
bdfp4_status bdfp4_decode_attention_logits(
    const bdfp4_recipe* r, const bdfp4_cache* cache, const void* q_bf16,
    int32_t batch, int32_t num_q_heads, const int32_t* block_tables,
    int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
    const void* sink_k, const void* sink_v, const void* tail_k,
    const void* tail_v, const float* key_shift, float softmax_scale,
    int32_t pages_per_partition, void* workspace, size_t workspace_bytes,
    float* out, float* logits, void* stream);

/* BF16-KV paged decode (the unquantized baseline arm, kv_cache_dtype "auto"
 * in KV_MODES): exact softmax attention over all L tokens of BF16 pages
 * k_pages / v_pages [num_pages][num_kv_heads][128][128], split as
 * bdfp4_bf16_decode_plan says (pages_per_partition 0 .. 16), with the
 * workspace rules of bdfp4_decode_attention. */
bdfp4_status bdfp4_bf16_decode_attention(
    const void* q_bf16, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
    const void* k_pages, const void* v_pages, int32_t num_pages,
    const int32_t* block_tables, int32_t max_pages_per_seq,
    const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
    int32_t pages_per_partition, void* workspace, size_t workspace_bytes,
    float* out, void* stream);

/* Debug/codec entry: quantize n_rows independent rows of 128 elements with
 * the key or query path and write logical codes and scales.
 *   rows_bf16:  bf16 [n_rows][128]; shift: float32 [128] subtracted first, or
 *               NULL; rotation: 0/1; mode: AMAX6 | FOUR_SIX | MXFP4_SEARCH;
 *               terms: 1, or 2 for the residual second term.
 *   codes:      uint8 [n_rows][terms][64], element 2i in bits 3..0 of byte i.
 *   scales:     uint8 [n_rows][terms][nb], nb = 8 (E4M3) or 4 (E8M0). */
bdfp4_status bdfp4_quantize_rows(const void* rows_bf16, int32_t n_rows,
                                 const float* shift, int32_t rotation,
                                 int32_t mode, int32_t terms, uint8_t* codes,
                                 uint8_t* scales, void* stream);

/* Debug entry: the query quantization exactly as bdfp4_decode_attention
 * performs it (the decode's own prologue: 128-point rotation when the recipe
 * has it, then Q1 and, with two terms, Q2 of the residual; amax6 per 16 for
 * NVFP4 pages, mxfp4_search per 32 for MXFP4 pages), for every query row.
 *   q_bf16: [batch][num_q_heads][128]; num_q_heads = 4 * num_kv_heads.
 *   codes:  uint8 [batch * num_q_heads][query_terms][64], element 2i in
 *           bits 3..0 of byte i; scales: uint8 [batch * num_q_heads]
 *           [query_terms][nb], nb = 8 (E4M3) or 4 (E8M0).
 * The recipe is validated as for the decode (tau included). */
bdfp4_status bdfp4_decode_query_codes(const bdfp4_recipe* r, const void* q_bf16,
                                      int32_t batch, int32_t num_q_heads,
                                      int32_t num_kv_heads, uint8_t* codes,
                                      uint8_t* scales, void* stream);

/* Debug/codec entry: the probability quantizer on n_blocks blocks of 16
 * non-negative float32 values p' (already multiplied by c).
 *   mode: AMAX2_OR_AMAX6 (with tau) | AMAX6; codes uint8 [n_blocks][8];
 *   scales uint8 [n_blocks] (E4M3). */
bdfp4_status bdfp4_quantize_p_blocks(const float* pp, int32_t n_blocks,
                                     int32_t mode, float tau, uint8_t* codes,
                                     uint8_t* scales, void* stream);

/* Diagnostic: a plain streaming read of `bytes` (a multiple of 16) at `src`
 * (device, 16-byte aligned) by `workgroups` workgroups of 256 threads (1 ..
 * 65536), grid-stride over 16-byte words with four loads in flight per
 * thread. Every thread stores one uint32 fold (xor) of what it read to
 * `sink` (device, at least workgroups * 256 * 4 bytes), so the reads cannot
 * be elided. It measures the practical HBM read bandwidth for a byte count,
 * the ceiling the decode's roofline fraction is read against. Asynchronous
 * on `stream`; E_INVALID for bad sizes, alignment or NULL pointers. */
bdfp4_status bdfp4_stream_read(const void* src, size_t bytes, void* sink,
                               size_t sink_bytes, int32_t workgroups,
                               void* stream);

/* Name of a status code (static string). */
const char* bdfp4_status_string(int32_t status);

/* Description of the last error on this thread ("" if none). */
const char* bdfp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BDFP4_H */
