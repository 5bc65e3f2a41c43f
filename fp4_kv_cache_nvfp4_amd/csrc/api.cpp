// Host side of the bdfp4 C ABI: recipe defaults and validation, sizes, the
// decode split plan, and the launches. Every check runs before anything is
// enqueued; a failing check returns its status and records a message.
//
// The constraints enforced on the probability settings come from
// "BitDecoding-FP4 evaluation/config.py", section probability_environment:
// the P multiplier c takes the values 1 and 8, an uncalibrated tau cannot be
// used to decode, and a calibrated tau lies in the E4M3 range [0, 448]. The
// KV_MODES entries bitdecoding-nvfp4 / bitdecoding-mxfp4 give the sink, the
// scale modes and the query terms. Checks and messages are this library's.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/bdfp4.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

bdfp4_status fail(bdfp4_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

bdfp4_status ok() {
  g_err[0] = '\0';
  return BDFP4_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_nv_kv(const bdfp4_recipe* r) {
  return (r->scale_mode_k == BDFP4_SCALE_FOUR_SIX || r->scale_mode_k == BDFP4_SCALE_AMAX6) &&
         r->scale_mode_v == BDFP4_SCALE_AMAX6;
}

bool is_mx_kv(const bdfp4_recipe* r) {
  return r->scale_mode_k == BDFP4_SCALE_MXFP4_SEARCH && r->scale_mode_v == BDFP4_SCALE_MXFP4_SEARCH;
}

// The fields the page writer uses: rotation, smoothing, K and V modes.
bdfp4_status check_kv_recipe(const bdfp4_recipe* r) {
  if (r == nullptr) return fail(BDFP4_E_INVALID, "recipe is NULL");
  if (r->rotation != 0 && r->rotation != 1) return fail(BDFP4_E_INVALID, "rotation must be 0 or 1");
  if (r->rotate_v != 0 && r->rotate_v != 1) return fail(BDFP4_E_INVALID, "rotate_v must be 0 or 1");
  if (r->key_smoothing != 0 && r->key_smoothing != 1)
    return fail(BDFP4_E_INVALID, "key_smoothing must be 0 or 1");
  const int km = r->scale_mode_k, vm = r->scale_mode_v;
  if (km != BDFP4_SCALE_FOUR_SIX && km != BDFP4_SCALE_AMAX6 && km != BDFP4_SCALE_MXFP4_SEARCH &&
      km != BDFP4_SCALE_NONE)
    return fail(BDFP4_E_INVALID, "scale_mode_k %d is not a key scale mode", km);
  if (vm != BDFP4_SCALE_AMAX6 && vm != BDFP4_SCALE_MXFP4_SEARCH && vm != BDFP4_SCALE_NONE)
    return fail(BDFP4_E_INVALID, "scale_mode_v %d is not a value scale mode", vm);
  if (!is_nv_kv(r) && !is_mx_kv(r))
    return fail(BDFP4_E_UNSUPPORTED,
                "K/V scale modes (%d, %d): this library has kernels for (four_six|amax6, amax6) and "
                "(mxfp4_search, mxfp4_search)", km, vm);
  if (r->key_scale_geometry != BDFP4_KEY_GEOMETRY_LOCAL && r->key_scale_geometry != BDFP4_KEY_GEOMETRY_CHANNEL)
    return fail(BDFP4_E_INVALID, "key_scale_geometry must be 0 (local) or 1 (channel), got %d",
                r->key_scale_geometry);
  if (r->key_scale_geometry == BDFP4_KEY_GEOMETRY_CHANNEL && !is_nv_kv(r))
    return fail(BDFP4_E_UNSUPPORTED, "the channel key geometry has kernels for NVFP4 keys (four_six or amax6) only");
  return BDFP4_OK;
}

// tau of the amax2_or_amax6 P mode: NaN is the "still to be calibrated"
// placeholder (refused with its own status), anything else must be a finite
// threshold inside the E4M3 range.
bdfp4_status check_tau(float tau) {
  if (isnan(tau))
    return fail(BDFP4_E_UNCALIBRATED,
                "tau is NaN (the placeholder for a threshold not yet calibrated); run the tau search first");
  if (!(tau >= 0.0f && tau <= 448.0f))
    return fail(BDFP4_E_INVALID, "tau = %g: the amax2/amax6 threshold must be finite and within [0, 448]",
                (double)tau);
  return BDFP4_OK;
}

// P settings: the mode, then (amax2_or_amax6 only) tau, then the multiplier
// c, which every quantized P mode applies.
bdfp4_status check_probability(const bdfp4_recipe* r) {
  const int pm = r->scale_mode_p;
  if (pm == BDFP4_SCALE_NONE) return fail(BDFP4_E_UNSUPPORTED, "unquantized probabilities have no FP4 decode kernel");
  if (pm != BDFP4_SCALE_AMAX2_OR_AMAX6 && pm != BDFP4_SCALE_AMAX6)
    return fail(BDFP4_E_INVALID, "scale_mode_p %d is not a probability scale mode", pm);
  if (pm == BDFP4_SCALE_AMAX2_OR_AMAX6) {
    const bdfp4_status s = check_tau(r->tau);
    if (s != BDFP4_OK) return s;
  }
  if (r->c != 1 && r->c != 8)
    return fail(BDFP4_E_INVALID, "c = %d: P is multiplied by 1 or by 8 before quantization, nothing else", r->c);
  return BDFP4_OK;
}

bdfp4_status check_recipe(const bdfp4_recipe* r) {
  bdfp4_status s = check_kv_recipe(r);
  if (s != BDFP4_OK) {
    // an invalid K/V field outranks an unsupported combination only if the
    // probability settings are themselves fine; report the first problem
    if (s == BDFP4_E_INVALID) return s;
  }
  if (r->sink_tokens < 0 || r->sink_tokens > 112 || (r->sink_tokens % 16) != 0)
    return fail(BDFP4_E_INVALID, "sink_tokens must be a multiple of 16 in [0, 112], got %d",
                r->sink_tokens);
  if (r->query_terms != 1 && r->query_terms != 2)
    return fail(BDFP4_E_INVALID, "query_terms must be 1 or 2, got %d", r->query_terms);
  if (r->p_running_max != 0 && r->p_running_max != 1)
    return fail(BDFP4_E_INVALID, "p_running_max must be 0 or 1");
  const int qm = r->scale_mode_q, pm = r->scale_mode_p;
  if (qm != BDFP4_SCALE_AMAX6 && qm != BDFP4_SCALE_MXFP4_SEARCH && qm != BDFP4_SCALE_NONE)
    return fail(BDFP4_E_INVALID, "scale_mode_q %d is not a query scale mode", qm);
  const bdfp4_status ps = check_probability(r);
  if (ps != BDFP4_OK) return ps;
  if (s != BDFP4_OK) return s;
  if (qm == BDFP4_SCALE_NONE)
    return fail(BDFP4_E_UNSUPPORTED, "an unquantized query has no FP4 decode kernel");
  if (is_nv_kv(r) && qm != BDFP4_SCALE_AMAX6)
    return fail(BDFP4_E_UNSUPPORTED, "NVFP4 pages take an amax6 query in this library");
  if (is_mx_kv(r) && qm != BDFP4_SCALE_MXFP4_SEARCH)
    return fail(BDFP4_E_UNSUPPORTED, "MXFP4 pages take an mxfp4_search query in this library");
  if (r->p_running_max && (!is_nv_kv(r) || r->query_terms != 2 || pm != BDFP4_SCALE_AMAX2_OR_AMAX6))
    return fail(BDFP4_E_UNSUPPORTED,
                "p_running_max has a kernel for NVFP4 pages, two query terms and amax2_or_amax6 P only");
  if (r->p_running_max && r->key_scale_geometry == BDFP4_KEY_GEOMETRY_CHANNEL)
    return fail(BDFP4_E_UNSUPPORTED, "p_running_max has no kernel for the channel key geometry");
  return BDFP4_OK;
}

bdfp4_status check_cache(const bdfp4_cache* c) {
  if (c == nullptr) return fail(BDFP4_E_INVALID, "cache is NULL");
  if (c->head_dim != 128 || c->block_size != 128)
    return fail(BDFP4_E_UNSUPPORTED, "head_dim and block_size must be 128 (got %d, %d)", c->head_dim,
                c->block_size);
  if (c->num_pages < 1 || c->num_kv_heads < 1)
    return fail(BDFP4_E_INVALID, "num_pages and num_kv_heads must be positive");
  if (!c->k_codes || !c->k_scales || !c->v_codes || !c->v_scales)
    return fail(BDFP4_E_INVALID, "cache array pointer is NULL");
  if (!aligned16(c->k_codes) || !aligned16(c->k_scales) || !aligned16(c->v_codes) || !aligned16(c->v_scales))
    return fail(BDFP4_E_INVALID, "cache arrays must be 16-byte aligned");
  return BDFP4_OK;
}

// Pages per partition for the MI355X's 256 compute units. The smallest that
// keeps the FP4 workgroups (four partitions each) within one per compute
// unit, when one of up to 4 pages does: the grid then has room for the BF16
// partitions' own workgroups. Longer contexts take about two FP4 workgroups
// per compute unit (measured best from 8K to 128K tokens at batch 1, 8 KV
// heads: 1 page up to 16K, 2 at 32K, 3 at 48K, 4 at 64K, 3 at 96K, 4 at 128K).
int32_t auto_ppp(int32_t batch, int32_t hkv, int32_t max_seq_len) {
  const int64_t n_full = max_seq_len / 128;
  const int64_t work = (int64_t)batch * hkv * n_full;     // full page-heads
  int64_t ppp = (work + 1023) / 1024;                     // <= 256 workgroups
  if (ppp > 4) ppp = (work + 2047) / 2048;                // about 512 workgroups
  if (ppp < 1) ppp = 1;
  if (ppp > 4) ppp = 4;
  return (int32_t)ppp;
}

constexpr int32_t kMaxPpp = 4;   // a partition is one wave's pages; its logits sit in LDS

// The BF16-KV decode's plan: every page of a sequence is read (the partial
// last one included) and a workgroup's partition is split over its 4 waves,
// up to 16 pages (its logits sit in LDS). Measured on the MI355X for one
// sequence x 8 KV heads, the best value is the one that gives about 512
// workgroups (8K: 1-2 pages, 32K: 4, 64K: 8, 128K: 16; at 128K 16 pages take
// 108 us against 129 us for 4, whose 2,048 workgroups run in 2.7 rounds and
// merge 256 partials per head).
constexpr int32_t kMaxPppBf16 = 16;

int32_t auto_ppp_bf16(int32_t batch, int32_t hkv, int32_t max_seq_len) {
  const int64_t pages = ((int64_t)max_seq_len + 127) / 128;
  const int64_t work = (int64_t)batch * hkv * pages;      // page-heads
  int64_t ppp = (work + 511) / 512;                       // about 512 workgroups
  if (ppp < 1) ppp = 1;
  if (ppp > kMaxPppBf16) ppp = kMaxPppBf16;
  return (int32_t)ppp;
}

bdfp4_status plan_checks(int32_t batch, int32_t hkv, int32_t max_seq_len, int32_t ppp_in, int32_t max_ppp) {
  if (batch < 1 || hkv < 1) return fail(BDFP4_E_INVALID, "batch and num_kv_heads must be positive");
  if (max_seq_len < 1) return fail(BDFP4_E_INVALID, "max_seq_len must be positive");
  if (ppp_in < 0 || ppp_in > max_ppp)
    return fail(BDFP4_E_INVALID, "pages_per_partition must be in [0, %d], got %d", max_ppp, ppp_in);
  if ((int64_t)batch * hkv > bdfp4::kMaxSeqHeads)
    return fail(BDFP4_E_UNSUPPORTED, "batch * num_kv_heads must be <= %d", bdfp4::kMaxSeqHeads);
  return BDFP4_OK;
}

// FP4 decode plan: partitions of full pages.
bdfp4_status plan(int32_t batch, int32_t hkv, int32_t max_seq_len, int32_t ppp_in, int32_t* ppp,
                  int32_t* parts) {
  const bdfp4_status s = plan_checks(batch, hkv, max_seq_len, ppp_in, kMaxPpp);
  if (s != BDFP4_OK) return s;
  *ppp = ppp_in ? ppp_in : auto_ppp(batch, hkv, max_seq_len);
  const int32_t n_full = max_seq_len / 128;
  *parts = (n_full + *ppp - 1) / *ppp;
  return BDFP4_OK;
}

// BF16-KV decode plan: partitions of all pages.
bdfp4_status plan_bf16(int32_t batch, int32_t hkv, int32_t max_seq_len, int32_t ppp_in, int32_t* ppp,
                       int32_t* parts) {
  const bdfp4_status s = plan_checks(batch, hkv, max_seq_len, ppp_in, kMaxPppBf16);
  if (s != BDFP4_OK) return s;
  *ppp = ppp_in ? ppp_in : auto_ppp_bf16(batch, hkv, max_seq_len);
  const int32_t pages = (max_seq_len + 127) / 128;
  *parts = (pages + *ppp - 1) / *ppp;
  return BDFP4_OK;
}

// Partitions the workspace is sized for: those of the longest sequence
// counting its partial last page (the BF16 decode reads it as a page).
int32_t workspace_parts(int32_t max_seq_len, int32_t ppp) { return ((max_seq_len + 127) / 128 + ppp - 1) / ppp; }

size_t workspace_bytes(int32_t batch, int32_t hkv, int32_t max_seq_len, int32_t ppp) {
  return bdfp4::workspace_bytes_for(batch, hkv, workspace_parts(max_seq_len, ppp));
}

bdfp4_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BDFP4_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* bdfp4_status_string(int32_t s) {
  switch (s) {
    case BDFP4_OK: return "BDFP4_OK";
    case BDFP4_E_INVALID: return "BDFP4_E_INVALID";
    case BDFP4_E_UNCALIBRATED: return "BDFP4_E_UNCALIBRATED";
    case BDFP4_E_UNSUPPORTED: return "BDFP4_E_UNSUPPORTED";
    case BDFP4_E_WORKSPACE: return "BDFP4_E_WORKSPACE";
    case BDFP4_E_HIP: return "BDFP4_E_HIP";
    default: return "BDFP4_E_UNKNOWN";
  }
}

const char* bdfp4_last_error(void) { return g_err; }

bdfp4_status bdfp4_recipe_default_nvfp4(bdfp4_recipe* r) {
  if (r == nullptr) return fail(BDFP4_E_INVALID, "recipe is NULL");
  r->sink_tokens = 16;
  r->rotation = 1;
  r->rotate_v = 0;
  r->p_running_max = 0;
  r->key_smoothing = 1;
  r->scale_mode_k = BDFP4_SCALE_FOUR_SIX;
  r->scale_mode_v = BDFP4_SCALE_AMAX6;
  r->scale_mode_q = BDFP4_SCALE_AMAX6;
  r->scale_mode_p = BDFP4_SCALE_AMAX2_OR_AMAX6;
  r->query_terms = 2;
  r->c = 8;
  r->tau = NAN;
  r->key_scale_geometry = BDFP4_KEY_GEOMETRY_LOCAL;
  return ok();
}

bdfp4_status bdfp4_recipe_default_mxfp4(bdfp4_recipe* r) {
  bdfp4_status s = bdfp4_recipe_default_nvfp4(r);
  if (s != BDFP4_OK) return s;
  r->scale_mode_k = r->scale_mode_v = r->scale_mode_q = BDFP4_SCALE_MXFP4_SEARCH;
  return ok();
}

bdfp4_status bdfp4_recipe_validate(const bdfp4_recipe* r) {
  if (r == nullptr) return fail(BDFP4_E_INVALID, "recipe is NULL");
  bdfp4_status s = check_recipe(r);
  return s == BDFP4_OK ? ok() : s;
}

bdfp4_status bdfp4_cache_bytes(const bdfp4_recipe* r, int32_t num_pages, int32_t num_kv_heads,
                               size_t* k_codes, size_t* k_scales, size_t* v_codes, size_t* v_scales) {
  bdfp4_status s = check_kv_recipe(r);
  if (s != BDFP4_OK) return s;
  if (num_pages < 0 || num_kv_heads < 1) return fail(BDFP4_E_INVALID, "bad page or head count");
  if (!k_codes || !k_scales || !v_codes || !v_scales) return fail(BDFP4_E_INVALID, "NULL output");
  const size_t ph = (size_t)num_pages * num_kv_heads;
  const bool kmx = r->scale_mode_k == BDFP4_SCALE_MXFP4_SEARCH;
  const bool vmx = r->scale_mode_v == BDFP4_SCALE_MXFP4_SEARCH;
  *k_codes = ph * 8192;
  *v_codes = ph * 8192;
  *k_scales = ph * (kmx ? 512 : 1024);
  *v_scales = ph * (vmx ? 512 : 1024);
  return ok();
}

bdfp4_status bdfp4_quantize_pages(const bdfp4_recipe* r, const bdfp4_cache* cache, const void* k_bf16,
                                  const void* v_bf16, const int32_t* page_ids, int32_t n_pages,
                                  const float* key_shift, void* stream) {
  bdfp4_status s = check_kv_recipe(r);
  if (s != BDFP4_OK) return s;
  if ((s = check_cache(cache)) != BDFP4_OK) return s;
  if (n_pages < 0) return fail(BDFP4_E_INVALID, "n_pages must be >= 0");
  if (n_pages == 0) return ok();
  if (!k_bf16 || !v_bf16 || !page_ids) return fail(BDFP4_E_INVALID, "NULL input pointer");
  if (!aligned16(k_bf16) || !aligned16(v_bf16)) return fail(BDFP4_E_INVALID, "k/v must be 16-byte aligned");
  if (r->key_smoothing && key_shift == nullptr)
    return fail(BDFP4_E_INVALID, "key_smoothing needs key_shift (the key-mean sidecar)");
  if (!r->key_smoothing && key_shift != nullptr)
    return fail(BDFP4_E_INVALID, "key_shift given but key_smoothing is off");
  if (key_shift && !aligned16(key_shift)) return fail(BDFP4_E_INVALID, "key_shift must be 16-byte aligned");
  // one 256-thread workgroup per (page, KV head): the grid's work-items
  // along x must stay below 2^32
  if ((int64_t)n_pages * cache->num_kv_heads >= ((int64_t)1 << 24))
    return fail(BDFP4_E_INVALID, "too many pages in one call (n_pages * num_kv_heads must be < 2^24)");
  bdfp4::WriterLaunch L;
  L.k = k_bf16;
  L.v = v_bf16;
  L.page_ids = page_ids;
  L.key_shift = key_shift;
  L.k_codes = cache->k_codes;
  L.k_scales = cache->k_scales;
  L.v_codes = cache->v_codes;
  L.v_scales = cache->v_scales;
  L.num_pages = cache->num_pages;
  L.hkv = cache->num_kv_heads;
  L.n_pages = n_pages;
  L.rotation = r->rotation;
  L.rotate_v = r->rotate_v;
  L.k_mode = r->scale_mode_k == BDFP4_SCALE_FOUR_SIX ? 2 : (r->scale_mode_k == BDFP4_SCALE_AMAX6 ? 1 : 3);
  L.v_mode = r->scale_mode_v == BDFP4_SCALE_AMAX6 ? 1 : 3;
  L.k_chan = r->key_scale_geometry == BDFP4_KEY_GEOMETRY_CHANNEL;
  return hip_status(bdfp4::launch_writer(L, static_cast<hipStream_t>(stream)), "page writer launch");
}

bdfp4_status bdfp4_append_tokens(const bdfp4_recipe* r, const bdfp4_cache* cache, const void* k_new,
                                 const void* v_new, int32_t batch, const int32_t* positions,
                                 const int32_t* block_tables, int32_t max_pages_per_seq, void* sink_k,
                                 void* sink_v, void* tail_k, void* tail_v, const float* key_shift,
                                 void* stream) {
  bdfp4_status s = check_kv_recipe(r);
  if (s != BDFP4_OK) return s;
  if ((s = check_cache(cache)) != BDFP4_OK) return s;
  if (batch < 0) return fail(BDFP4_E_INVALID, "batch must be >= 0");
  if (batch == 0) return ok();
  if (max_pages_per_seq < 1 || max_pages_per_seq > (1 << 23))
    return fail(BDFP4_E_INVALID, "max_pages_per_seq must be in [1, 2^23]");
  if ((int64_t)batch * cache->num_kv_heads > 0x7FFFFFFF) return fail(BDFP4_E_INVALID, "batch too large");
  if (!k_new || !v_new || !positions || !block_tables || !tail_k || !tail_v)
    return fail(BDFP4_E_INVALID, "NULL input pointer");
  if (r->sink_tokens > 0 && (!sink_k || !sink_v))
    return fail(BDFP4_E_INVALID, "sink buffers required when sink_tokens > 0");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(tail_k) || !aligned16(tail_v) ||
      (r->sink_tokens > 0 && (!aligned16(sink_k) || !aligned16(sink_v))))
    return fail(BDFP4_E_INVALID, "token, tail and sink buffers must be 16-byte aligned");
  if (r->key_smoothing && key_shift == nullptr)
    return fail(BDFP4_E_INVALID, "key_smoothing needs key_shift (the key-mean sidecar)");
  if (!r->key_smoothing && key_shift != nullptr)
    return fail(BDFP4_E_INVALID, "key_shift given but key_smoothing is off");
  if (key_shift && !aligned16(key_shift)) return fail(BDFP4_E_INVALID, "key_shift must be 16-byte aligned");
  bdfp4::AppendLaunch L;
  L.w.k = nullptr;
  L.w.v = nullptr;
  L.w.page_ids = nullptr;
  L.w.key_shift = key_shift;
  L.w.k_codes = cache->k_codes;
  L.w.k_scales = cache->k_scales;
  L.w.v_codes = cache->v_codes;
  L.w.v_scales = cache->v_scales;
  L.w.num_pages = cache->num_pages;
  L.w.hkv = cache->num_kv_heads;
  L.w.n_pages = 0;
  L.w.rotation = r->rotation;
  L.w.rotate_v = r->rotate_v;
  L.w.k_mode = r->scale_mode_k == BDFP4_SCALE_FOUR_SIX ? 2 : (r->scale_mode_k == BDFP4_SCALE_AMAX6 ? 1 : 3);
  L.w.v_mode = r->scale_mode_v == BDFP4_SCALE_AMAX6 ? 1 : 3;
  L.w.k_chan = r->key_scale_geometry == BDFP4_KEY_GEOMETRY_CHANNEL;
  L.k_new = k_new;
  L.v_new = v_new;
  L.positions = positions;
  L.block_tables = block_tables;
  L.sink_k = r->sink_tokens > 0 ? sink_k : nullptr;
  L.sink_v = r->sink_tokens > 0 ? sink_v : nullptr;
  L.tail_k = tail_k;
  L.tail_v = tail_v;
  L.batch = batch;
  L.max_pages_per_seq = max_pages_per_seq;
  L.sink_tokens = r->sink_tokens;
  return hip_status(bdfp4::launch_append(L, static_cast<hipStream_t>(stream)), "append launch");
}

bdfp4_status bdfp4_key_means_workspace_size(int32_t tokens, int32_t num_kv_heads, size_t* bytes) {
  if (!bytes) return fail(BDFP4_E_INVALID, "NULL output");
  if (tokens < 1) return fail(BDFP4_E_INVALID, "tokens must be >= 1");
  if (num_kv_heads < 1 || num_kv_heads > 65535) return fail(BDFP4_E_INVALID, "num_kv_heads must be in [1, 65535]");
  *bytes = bdfp4::key_means_workspace_bytes(tokens, num_kv_heads);
  return ok();
}

bdfp4_status bdfp4_key_means(const void* k_bf16, int32_t tokens, int32_t num_kv_heads, void* workspace,
                             size_t workspace_bytes, float* mu_out, void* stream) {
  size_t need = 0;
  bdfp4_status s = bdfp4_key_means_workspace_size(tokens, num_kv_heads, &need);
  if (s != BDFP4_OK) return s;
  if (!k_bf16 || !workspace || !mu_out) return fail(BDFP4_E_INVALID, "NULL pointer");
  if (!aligned16(k_bf16) || !aligned16(workspace) || !aligned16(mu_out))
    return fail(BDFP4_E_INVALID, "keys, workspace and output must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(BDFP4_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  return hip_status(bdfp4::launch_key_means(k_bf16, tokens, num_kv_heads, workspace, mu_out,
                                            static_cast<hipStream_t>(stream)),
                    "key means launch");
}

bdfp4_status bdfp4_error_sums(const float* got, const float* ref, int64_t n, double* sums_out, void* stream) {
  if (n < 0 || n > ((int64_t)1 << 31)) return fail(BDFP4_E_INVALID, "n must be in [0, 2^31]");
  if (!sums_out || (n > 0 && (!got || !ref))) return fail(BDFP4_E_INVALID, "NULL pointer");
  if (((uintptr_t)got & 3) || ((uintptr_t)ref & 3) || ((uintptr_t)sums_out & 7))
    return fail(BDFP4_E_INVALID, "misaligned pointer");
  return hip_status(bdfp4::launch_error_sums(got, ref, n, sums_out, static_cast<hipStream_t>(stream)),
                    "error sums launch");
}

bdfp4_status bdfp4_select_tau(const double* sums, const float* candidates, int32_t n, float* best_tau,
                              int32_t* best_index, double* rel_errors) {
  if (n < 1) return fail(BDFP4_E_INVALID, "n must be >= 1");
  if (!sums || !candidates || !best_tau) return fail(BDFP4_E_INVALID, "NULL pointer");
  int best = -1;
  double best_err = 0.0;
  bool any = false;
  for (int32_t i = 0; i < n; ++i) {
    const double e = sums[2 * i], r = sums[2 * i + 1];
    if (e < 0.0 || r < 0.0) return fail(BDFP4_E_INVALID, "error sums of candidate %d are negative", i);
    double rel;
    if (isnan(e) || isnan(r)) rel = NAN;
    else if (r == 0.0) rel = e == 0.0 ? 0.0 : INFINITY;
    else rel = sqrt(e / r);
    if (rel_errors) rel_errors[i] = rel;
    if (isnan(rel)) continue;
    any = true;
    if (best < 0 || rel < best_err) {   // strict: a tie keeps the earlier candidate
      best = i;
      best_err = rel;
    }
  }
  if (!any) return fail(BDFP4_E_INVALID, "every candidate's error is NaN");
  *best_tau = candidates[best];
  if (best_index) *best_index = best;
  return ok();
}

bdfp4_status bdfp4_page_errors_workspace_size(int32_t n_pages, int32_t num_kv_heads, size_t* bytes) {
  if (!bytes) return fail(BDFP4_E_INVALID, "NULL output");
  if (n_pages < 1 || num_kv_heads < 1 || (int64_t)n_pages * num_kv_heads > 0x7FFFFFFF)
    return fail(BDFP4_E_INVALID, "n_pages and num_kv_heads must be >= 1 (product < 2^31)");
  *bytes = bdfp4::page_errors_workspace_bytes(n_pages, num_kv_heads);
  return ok();
}

bdfp4_status bdfp4_page_errors(const bdfp4_recipe* r, const bdfp4_cache* cache, const void* k_bf16,
                               const void* v_bf16, const int32_t* page_ids, int32_t n_pages,
                               const float* key_shift, void* workspace, size_t workspace_bytes,
                               double* sums_out, void* stream) {
  bdfp4_status s = check_kv_recipe(r);
  if (s != BDFP4_OK) return s;
  if ((s = check_cache(cache)) != BDFP4_OK) return s;
  size_t need = 0;
  if ((s = bdfp4_page_errors_workspace_size(n_pages, cache->num_kv_heads, &need)) != BDFP4_OK) return s;
  if (!k_bf16 || !v_bf16 || !page_ids || !workspace || !sums_out) return fail(BDFP4_E_INVALID, "NULL pointer");
  if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(workspace) || ((uintptr_t)sums_out & 7))
    return fail(BDFP4_E_INVALID, "misaligned pointer");
  if (r->key_smoothing && key_shift == nullptr)
    return fail(BDFP4_E_INVALID, "key_smoothing needs key_shift (the key-mean sidecar)");
  if (!r->key_smoothing && key_shift != nullptr)
    return fail(BDFP4_E_INVALID, "key_shift given but key_smoothing is off");
  if (workspace_bytes < need)
    return fail(BDFP4_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  bdfp4::WriterLaunch L;
  L.k = k_bf16;
  L.v = v_bf16;
  L.page_ids = page_ids;
  L.key_shift = key_shift;
  L.k_codes = cache->k_codes;
  L.k_scales = cache->k_scales;
  L.v_codes = cache->v_codes;
  L.v_scales = cache->v_scales;
  L.num_pages = cache->num_pages;
  L.hkv = cache->num_kv_heads;
  L.n_pages = n_pages;
  L.rotation = r->rotation;
  L.rotate_v = r->rotate_v;
  L.k_mode = r->scale_mode_k == BDFP4_SCALE_FOUR_SIX ? 2 : (r->scale_mode_k == BDFP4_SCALE_AMAX6 ? 1 : 3);
  L.v_mode = r->scale_mode_v == BDFP4_SCALE_AMAX6 ? 1 : 3;
  L.k_chan = r->key_scale_geometry == BDFP4_KEY_GEOMETRY_CHANNEL;
  return hip_status(bdfp4::launch_page_errors(L, workspace, sums_out, static_cast<hipStream_t>(stream)),
                    "page errors launch");
}

bdfp4_status bdfp4_decode_plan(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len,
                               int32_t pages_per_partition, int32_t* ppp_out, int32_t* parts_out) {
  if (!ppp_out || !parts_out) return fail(BDFP4_E_INVALID, "NULL output");
  bdfp4_status s = plan(batch, num_kv_heads, max_seq_len, pages_per_partition, ppp_out, parts_out);
  return s == BDFP4_OK ? ok() : s;
}

bdfp4_status bdfp4_bf16_decode_plan(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len,
                                    int32_t pages_per_partition, int32_t* ppp_out, int32_t* parts_out) {
  if (!ppp_out || !parts_out) return fail(BDFP4_E_INVALID, "NULL output");
  bdfp4_status s = plan_bf16(batch, num_kv_heads, max_seq_len, pages_per_partition, ppp_out, parts_out);
  return s == BDFP4_OK ? ok() : s;
}

bdfp4_status bdfp4_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t max_seq_len, int32_t pages_per_partition, size_t* bytes) {
  if (!bytes) return fail(BDFP4_E_INVALID, "NULL output");
  if (num_q_heads != bdfp4::kGroup * num_kv_heads)
    return fail(BDFP4_E_UNSUPPORTED, "num_q_heads must be 4 * num_kv_heads");
  int32_t ppp, parts, ppp_b, parts_b;
  bdfp4_status s = plan_bf16(batch, num_kv_heads, max_seq_len, pages_per_partition, &ppp_b, &parts_b);
  if (s != BDFP4_OK) return s;
  size_t need = workspace_bytes(batch, num_kv_heads, max_seq_len, ppp_b);
  if (pages_per_partition <= kMaxPpp) {
    // 0: both decodes' automatic plans; 1 .. 4: a plan either decode accepts
    s = plan(batch, num_kv_heads, max_seq_len, pages_per_partition, &ppp, &parts);
    if (s != BDFP4_OK) return s;
    const size_t fp4 = workspace_bytes(batch, num_kv_heads, max_seq_len, ppp);
    if (fp4 > need) need = fp4;
  }
  *bytes = need;
  return ok();
}

static bdfp4_status check_decode_common(const void* q, int32_t batch, int32_t hq, int32_t hkv,
                                        const int32_t* block_tables, int32_t max_pages_per_seq,
                                        const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                                        int32_t ppp_in, void* workspace, size_t workspace_bytes_in,
                                        float* out, int32_t* ppp, int32_t* parts, bool bf16 = false) {
  if (hq != bdfp4::kGroup * hkv)
    return fail(BDFP4_E_UNSUPPORTED, "num_q_heads must be 4 * num_kv_heads (got %d, %d)", hq, hkv);
  bdfp4_status s = bf16 ? plan_bf16(batch, hkv, max_seq_len, ppp_in, ppp, parts)
                        : plan(batch, hkv, max_seq_len, ppp_in, ppp, parts);
  if (s != BDFP4_OK) return s;
  if (!q || !block_tables || !seq_lens || !out) return fail(BDFP4_E_INVALID, "NULL input or output pointer");
  if (!aligned16(q) || !aligned16(out)) return fail(BDFP4_E_INVALID, "q and out must be 16-byte aligned");
  if (max_pages_per_seq < 1) return fail(BDFP4_E_INVALID, "max_pages_per_seq must be positive");
  if (!isfinite(softmax_scale)) return fail(BDFP4_E_INVALID, "softmax_scale must be finite");
  if (workspace != nullptr && !aligned16(workspace)) return fail(BDFP4_E_INVALID, "workspace must be 16-byte aligned");
  return BDFP4_OK;
}

// Checked last, after every input check: the workspace holds the tickets and
// the partials of the plan.
static bdfp4_status check_workspace(int32_t batch, int32_t hkv, int32_t max_seq_len, int32_t ppp,
                                    const void* workspace, size_t workspace_bytes_in) {
  const size_t need = workspace_bytes(batch, hkv, max_seq_len, ppp);
  if (workspace == nullptr || workspace_bytes_in < need)
    return fail(BDFP4_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes_in);
  return BDFP4_OK;
}

// The FP4 decode behind both entry points. With noalloc the workspace
// arguments are ignored and the library's own per-GPU scratch array is used
// instead, once the plan's workspace is known to fit in it.
static bdfp4_status decode_impl(const bdfp4_recipe* r, const bdfp4_cache* cache, const void* q_bf16,
                                int32_t batch, int32_t num_q_heads, const int32_t* block_tables,
                                int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                const void* sink_k, const void* sink_v, const void* tail_k, const void* tail_v,
                                const float* key_shift, float softmax_scale, int32_t pages_per_partition,
                                void* workspace, size_t workspace_bytes_in, float* out, void* stream,
                                bool noalloc, float* logits = nullptr) {
  if (r == nullptr) return fail(BDFP4_E_INVALID, "recipe is NULL");
  bdfp4_status s = check_recipe(r);
  if (s != BDFP4_OK) return s;
  if ((s = check_cache(cache)) != BDFP4_OK) return s;
  int32_t ppp, parts;
  s = check_decode_common(q_bf16, batch, num_q_heads, cache->num_kv_heads, block_tables, max_pages_per_seq,
                          seq_lens, max_seq_len, softmax_scale, pages_per_partition, workspace,
                          workspace_bytes_in, out, &ppp, &parts);
  if (s != BDFP4_OK) return s;
  if (r->sink_tokens > 0 && (!sink_k || !sink_v)) return fail(BDFP4_E_INVALID, "sink buffers are NULL");
  if (!tail_k || !tail_v) return fail(BDFP4_E_INVALID, "tail buffers are NULL");
  if ((sink_k && !aligned16(sink_k)) || (sink_v && !aligned16(sink_v)) || !aligned16(tail_k) ||
      !aligned16(tail_v))
    return fail(BDFP4_E_INVALID, "sink and tail buffers must be 16-byte aligned");
  if (r->key_smoothing && key_shift == nullptr)
    return fail(BDFP4_E_INVALID, "key_smoothing needs key_shift (the key-mean sidecar)");
  if (!r->key_smoothing && key_shift != nullptr)
    return fail(BDFP4_E_INVALID, "key_shift given but key_smoothing is off");
  if (key_shift && !aligned16(key_shift)) return fail(BDFP4_E_INVALID, "key_shift must be 16-byte aligned");
  if (max_seq_len / 128 > max_pages_per_seq)
    return fail(BDFP4_E_INVALID, "max_seq_len needs %d pages but block tables hold %d", max_seq_len / 128,
                max_pages_per_seq);
  if (noalloc) {
    const size_t need = workspace_bytes(batch, cache->num_kv_heads, max_seq_len, ppp);
    if (need > bdfp4::kNoAllocScratchBytes)
      return fail(BDFP4_E_WORKSPACE,
                  "this call needs %zu bytes of workspace; the allocation-free decode has %zu "
                  "(use bdfp4_decode_attention with a caller workspace)",
                  need, bdfp4::kNoAllocScratchBytes);
    const hipError_t e = bdfp4::noalloc_scratch(static_cast<hipStream_t>(stream), &workspace);
    if (e != hipSuccess) return hip_status(e, "scratch set-up");
    workspace_bytes_in = bdfp4::kNoAllocScratchBytes;
  } else if ((s = check_workspace(batch, cache->num_kv_heads, max_seq_len, ppp, workspace, workspace_bytes_in)) !=
             BDFP4_OK) {
    return s;
  }
  bdfp4::DecodeLaunch L;
  L.sink = r->sink_tokens;
  L.rotation = r->rotation;
  L.rotate_v = r->rotate_v;
  L.run_max = r->p_running_max;
  L.k_chan = r->key_scale_geometry == BDFP4_KEY_GEOMETRY_CHANNEL;
  L.key_smoothing = r->key_smoothing;
  L.mx = is_mx_kv(r) ? 1 : 0;
  L.k_four_six = r->scale_mode_k == BDFP4_SCALE_FOUR_SIX;
  L.p_mode = r->scale_mode_p;
  L.terms = r->query_terms;
  L.c = r->c;
  L.tau = r->scale_mode_p == BDFP4_SCALE_AMAX2_OR_AMAX6 ? r->tau : 0.0f;
  L.k_codes = static_cast<const uint8_t*>(cache->k_codes);
  L.k_scales = static_cast<const uint8_t*>(cache->k_scales);
  L.v_codes = static_cast<const uint8_t*>(cache->v_codes);
  L.v_scales = static_cast<const uint8_t*>(cache->v_scales);
  L.num_pages = cache->num_pages;
  L.hkv = cache->num_kv_heads;
  L.q = static_cast<const uint16_t*>(q_bf16);
  L.batch = batch;
  L.hq = num_q_heads;
  L.block_tables = block_tables;
  L.max_pages_per_seq = max_pages_per_seq;
  L.seq_lens = seq_lens;
  L.max_seq_len = max_seq_len;
  L.sink_k = static_cast<const uint16_t*>(sink_k);
  L.sink_v = static_cast<const uint16_t*>(sink_v);
  L.tail_k = static_cast<const uint16_t*>(tail_k);
  L.tail_v = static_cast<const uint16_t*>(tail_v);
  L.key_shift = key_shift;
  L.softmax_scale = softmax_scale;
  L.ppp = ppp;
  L.max_parts = parts;
  L.counters = static_cast<uint32_t*>(workspace);
  L.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + bdfp4::kTicketBytes);
  L.counter_stride = bdfp4::kTicketStride;
  L.slot_stride = bdfp4::workspace_slot_stride(workspace_parts(max_seq_len, ppp));
  L.out = out;
  L.dbg_logits = logits;
  L.dbg_stride = 128 * max_pages_per_seq;
  return hip_status(bdfp4::launch_decode(L, static_cast<hipStream_t>(stream)), "decode launch");
}

bdfp4_status bdfp4_decode_attention(const bdfp4_recipe* r, const bdfp4_cache* cache, const void* q_bf16,
                                    int32_t batch, int32_t num_q_heads, const int32_t* block_tables,
                                    int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                    const void* sink_k, const void* sink_v, const void* tail_k,
                                    const void* tail_v, const float* key_shift, float softmax_scale,
                                    int32_t pages_per_partition, void* workspace, size_t workspace_bytes_in,
                                    float* out, void* stream) {
  return decode_impl(r, cache, q_bf16, batch, num_q_heads, block_tables, max_pages_per_seq, seq_lens, max_seq_len,
                     sink_k, sink_v, tail_k, tail_v, key_shift, softmax_scale, pages_per_partition, workspace,
                     workspace_bytes_in, out, stream, false);
}

bdfp4_status bdfp4_decode_attention_noalloc(const bdfp4_recipe* r, const bdfp4_cache* cache, const void* q_bf16,
                                            int32_t batch, int32_t num_q_heads, const int32_t* block_tables,
                                            int32_t max_pages_per_seq, const int32_t* seq_lens,
                                            int32_t max_seq_len, const void* sink_k, const void* sink_v,
                                            const void* tail_k, const void* tail_v, const float* key_shift,
                                            float softmax_scale, int32_t pages_per_partition, float* out,
                                            void* stream) {
  return decode_impl(r, cache, q_bf16, batch, num_q_heads, block_tables, max_pages_per_seq, seq_lens, max_seq_len,
                     sink_k, sink_v, tail_k, tail_v, key_shift, softmax_scale, pages_per_partition, nullptr, 0, out,
                     stream, true);
}

size_t bdfp4_decode_noalloc_max_workspace(void) { return bdfp4::kNoAllocScratchBytes; }

bdfp4_status bdfp4_decode_attention_logits(const bdfp4_recipe* r, const bdfp4_cache* cache, const void* q_bf16,
                                           int32_t batch, int32_t num_q_heads, const int32_t* block_tables,
                                           int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                           const void* sink_k, const void* sink_v, const void* tail_k,
                                           const void* tail_v, const float* key_shift, float softmax_scale,
                                           int32_t pages_per_partition, void* workspace, size_t workspace_bytes_in,
                                           float* out, float* logits, void* stream) {
  if (logits == nullptr) return fail(BDFP4_E_INVALID, "logits is NULL");
  if (((uintptr_t)logits & 3) != 0) return fail(BDFP4_E_INVALID, "logits must be 4-byte aligned");
  return decode_impl(r, cache, q_bf16, batch, num_q_heads, block_tables, max_pages_per_seq, seq_lens, max_seq_len,
                     sink_k, sink_v, tail_k, tail_v, key_shift, softmax_scale, pages_per_partition, workspace,
                     workspace_bytes_in, out, stream, false, logits);
}

bdfp4_status bdfp4_bf16_decode_attention(const void* q_bf16, int32_t batch, int32_t num_q_heads,
                                         int32_t num_kv_heads, const void* k_pages, const void* v_pages,
                                         int32_t num_pages, const int32_t* block_tables,
                                         int32_t max_pages_per_seq, const int32_t* seq_lens,
                                         int32_t max_seq_len, float softmax_scale, int32_t pages_per_partition,
                                         void* workspace, size_t workspace_bytes_in, float* out, void* stream) {
  int32_t ppp, parts;
  bdfp4_status s = check_decode_common(q_bf16, batch, num_q_heads, num_kv_heads, block_tables,
                                       max_pages_per_seq, seq_lens, max_seq_len, softmax_scale,
                                       pages_per_partition, workspace, workspace_bytes_in, out, &ppp, &parts,
                                       true);
  if (s != BDFP4_OK) return s;
  if (!k_pages || !v_pages) return fail(BDFP4_E_INVALID, "NULL page pointer");
  if (!aligned16(k_pages) || !aligned16(v_pages)) return fail(BDFP4_E_INVALID, "pages must be 16-byte aligned");
  if (num_pages < 1) return fail(BDFP4_E_INVALID, "num_pages must be positive");
  if ((max_seq_len + 127) / 128 > max_pages_per_seq)
    return fail(BDFP4_E_INVALID, "max_seq_len needs %d pages but block tables hold %d",
                (max_seq_len + 127) / 128, max_pages_per_seq);
  if ((s = check_workspace(batch, num_kv_heads, max_seq_len, ppp, workspace, workspace_bytes_in)) != BDFP4_OK)
    return s;
  bdfp4::Bf16DecodeLaunch L;
  L.q = static_cast<const uint16_t*>(q_bf16);
  L.batch = batch;
  L.hq = num_q_heads;
  L.hkv = num_kv_heads;
  L.k_pages = static_cast<const uint16_t*>(k_pages);
  L.v_pages = static_cast<const uint16_t*>(v_pages);
  L.num_pages = num_pages;
  L.block_tables = block_tables;
  L.max_pages_per_seq = max_pages_per_seq;
  L.seq_lens = seq_lens;
  L.max_seq_len = max_seq_len;
  L.softmax_scale = softmax_scale;
  // every page of a BF16 cache is read, the partial last one included
  L.ppp = ppp;
  L.max_parts = workspace_parts(max_seq_len, ppp);
  L.counters = static_cast<uint32_t*>(workspace);
  L.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + bdfp4::kTicketBytes);
  L.counter_stride = bdfp4::kTicketStride;
  L.slot_stride = bdfp4::workspace_slot_stride(L.max_parts);
  L.out = out;
  return hip_status(bdfp4::launch_bf16_decode(L, static_cast<hipStream_t>(stream)), "bf16 decode launch");
}

bdfp4_status bdfp4_quantize_rows(const void* rows_bf16, int32_t n_rows, const float* shift, int32_t rotation,
                                 int32_t mode, int32_t terms, uint8_t* codes, uint8_t* scales, void* stream) {
  if (n_rows < 0) return fail(BDFP4_E_INVALID, "n_rows must be >= 0");
  if (mode != BDFP4_SCALE_AMAX6 && mode != BDFP4_SCALE_FOUR_SIX && mode != BDFP4_SCALE_MXFP4_SEARCH)
    return fail(BDFP4_E_INVALID, "mode must be amax6, four_six or mxfp4_search");
  if (terms != 1 && terms != 2) return fail(BDFP4_E_INVALID, "terms must be 1 or 2");
  if (rotation != 0 && rotation != 1) return fail(BDFP4_E_INVALID, "rotation must be 0 or 1");
  if (n_rows == 0) return ok();
  if (!rows_bf16 || !codes || !scales) return fail(BDFP4_E_INVALID, "NULL pointer");
  if (!aligned16(rows_bf16) || !aligned16(codes)) return fail(BDFP4_E_INVALID, "rows/codes must be 16-byte aligned");
  if (n_rows > (1 << 28)) return fail(BDFP4_E_INVALID, "too many rows");
  const int m = mode == BDFP4_SCALE_AMAX6 ? 1 : (mode == BDFP4_SCALE_FOUR_SIX ? 2 : 3);
  return hip_status(bdfp4::launch_rows(rows_bf16, n_rows, shift, rotation, m, terms, codes, scales,
                                       static_cast<hipStream_t>(stream)),
                    "row quantizer launch");
}

bdfp4_status bdfp4_decode_query_codes(const bdfp4_recipe* r, const void* q_bf16, int32_t batch, int32_t num_q_heads,
                                      int32_t num_kv_heads, uint8_t* codes, uint8_t* scales, void* stream) {
  if (r == nullptr) return fail(BDFP4_E_INVALID, "recipe is NULL");
  bdfp4_status s = check_recipe(r);
  if (s != BDFP4_OK) return s;
  if (batch < 1 || num_kv_heads < 1 || (int64_t)batch * num_kv_heads > 0x7FFFFFFF)
    return fail(BDFP4_E_INVALID, "batch and num_kv_heads must be positive");
  if (num_q_heads != bdfp4::kGroup * num_kv_heads)
    return fail(BDFP4_E_UNSUPPORTED, "num_q_heads must be 4 * num_kv_heads (got %d, %d)", num_q_heads, num_kv_heads);
  if (!q_bf16 || !codes || !scales) return fail(BDFP4_E_INVALID, "NULL pointer");
  if (!aligned16(q_bf16)) return fail(BDFP4_E_INVALID, "q must be 16-byte aligned");
  bdfp4::DecodeLaunch L;
  memset(&L, 0, sizeof L);
  L.rotation = r->rotation;
  L.mx = is_mx_kv(r) ? 1 : 0;
  L.terms = r->query_terms;
  L.q = static_cast<const uint16_t*>(q_bf16);
  L.batch = batch;
  L.hq = num_q_heads;
  L.hkv = num_kv_heads;
  return hip_status(bdfp4::launch_query_codes(L, codes, scales, static_cast<hipStream_t>(stream)),
                    "query codes launch");
}

bdfp4_status bdfp4_quantize_p_blocks(const float* pp, int32_t n_blocks, int32_t mode, float tau, uint8_t* codes,
                                     uint8_t* scales, void* stream) {
  if (n_blocks < 0) return fail(BDFP4_E_INVALID, "n_blocks must be >= 0");
  if (mode != BDFP4_SCALE_AMAX2_OR_AMAX6 && mode != BDFP4_SCALE_AMAX6)
    return fail(BDFP4_E_INVALID, "mode must be amax2_or_amax6 or amax6");
  if (mode == BDFP4_SCALE_AMAX2_OR_AMAX6) {
    const bdfp4_status s = check_tau(tau);
    if (s != BDFP4_OK) return s;
  }
  if (n_blocks == 0) return ok();
  if (!pp || !codes || !scales) return fail(BDFP4_E_INVALID, "NULL pointer");
  if (!aligned16(pp) || (reinterpret_cast<uintptr_t>(codes) & 7u))
    return fail(BDFP4_E_INVALID, "pp must be 16-byte and codes 8-byte aligned");
  if (n_blocks > (1 << 28)) return fail(BDFP4_E_INVALID, "too many blocks");
  return hip_status(bdfp4::launch_p_blocks(pp, n_blocks, mode, tau, codes, scales, static_cast<hipStream_t>(stream)),
                    "probability quantizer launch");
}

bdfp4_status bdfp4_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, int32_t workgroups,
                               void* stream) {
  if (workgroups < 1 || workgroups > 65536) return fail(BDFP4_E_INVALID, "workgroups must be in [1, 65536]");
  if (bytes % 16 != 0) return fail(BDFP4_E_INVALID, "bytes must be a multiple of 16");
  if (!src || !sink) return fail(BDFP4_E_INVALID, "NULL pointer");
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return fail(BDFP4_E_INVALID, "src must be 16-byte and sink 4-byte aligned");
  if (sink_bytes < (size_t)workgroups * 256 * 4) return fail(BDFP4_E_INVALID, "sink needs workgroups * 1024 bytes");
  return hip_status(bdfp4::launch_stream_read(src, bytes, static_cast<uint32_t*>(sink), workgroups,
                                              static_cast<hipStream_t>(stream)),
                    "stream read launch");
}

}  // extern "C"
