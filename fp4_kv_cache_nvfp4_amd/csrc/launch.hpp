// Internal launch interface between the host API (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdfp4 {

struct WriterLaunch {
  const void* k;
  const void* v;
  const int32_t* page_ids;
  const float* key_shift;
  void* k_codes;
  void* k_scales;
  void* v_codes;
  void* v_scales;
  int32_t num_pages, hkv, n_pages, rotation, rotate_v;
  int32_t k_mode, v_mode;  // 1 amax6, 2 four_six, 3 mxfp4_search
  int32_t k_chan;          // channel key scale geometry (NVFP4 keys only)
};

hipError_t launch_writer(const WriterLaunch& L, hipStream_t stream);

// Decode-time append: w carries the cache, key_shift, rotation and modes
// (its k, v, page_ids and n_pages are unused).
struct AppendLaunch {
  WriterLaunch w;
  const void* k_new;
  const void* v_new;
  const int32_t* positions;
  const int32_t* block_tables;
  void* sink_k;
  void* sink_v;
  void* tail_k;
  void* tail_v;
  int32_t batch, max_pages_per_seq, sink_tokens;
};

hipError_t launch_append(const AppendLaunch& L, hipStream_t stream);

// Quantization diagnostics over n_pages written pages (L as for the writer):
// out (device double[4]) = [sum (k_hat - y)^2, sum y^2, sum (v_hat - v)^2,
// sum v^2], through a float64 workspace of page_errors_workspace_bytes.
size_t page_errors_workspace_bytes(int n_pages, int hkv);
hipError_t launch_page_errors(const WriterLaunch& L, void* workspace, double* out, hipStream_t stream);

// Calibration: per-(KV head, channel) key means of tokens x hkv bf16 rows
// (two passes through a float64 workspace of key_means_workspace_bytes), and
// float64 error sums [sum (got - ref)^2, sum ref^2] over n floats.
size_t key_means_workspace_bytes(int tokens, int hkv);
hipError_t launch_key_means(const void* k, int tokens, int hkv, void* workspace, float* mu, hipStream_t stream);
hipError_t launch_error_sums(const float* got, const float* ref, int64_t n, double* out, hipStream_t stream);

hipError_t launch_rows(const void* rows, int n_rows, const float* shift, int rotation, int mode,
                       int terms, uint8_t* codes, uint8_t* scales, hipStream_t stream);

hipError_t launch_p_blocks(const float* pp, int n_blocks, int mode, float tau, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream);

struct DecodeLaunch {
  // recipe
  int32_t sink, rotation, key_smoothing, mx, k_four_six, p_mode, terms, c, rotate_v, run_max, k_chan;
  float tau;
  // cache
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  int32_t num_pages, hkv;
  // problem
  const uint16_t* q;
  int32_t batch, hq;
  const int32_t* block_tables;
  int32_t max_pages_per_seq;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  const uint16_t* sink_k;
  const uint16_t* sink_v;
  const uint16_t* tail_k;
  const uint16_t* tail_v;
  const float* key_shift;
  float softmax_scale;
  int32_t ppp, max_parts;
  uint32_t* counters;     // workspace tickets
  float* partials;        // workspace partials
  int32_t counter_stride, slot_stride;
  float* out;
  float* dbg_logits;      // debug: raw FP4-token logits [batch * hkv][4][dbg_stride], or null
  int32_t dbg_stride;
  int32_t split_bf16;     // the BF16 partitions of sequences with >= 2 FP4 workgroups get workgroups of their own
  int32_t compact;        // a grid larger than the chip holds: workgroups take the units with work first
  int32_t bf16_last;      // split_bf16 with more FP4 workgroups than compute units: the BF16 column is dispatched last
};

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream);

// The decode's query prologue alone (debug): codes [batch * hq][terms][64],
// scales [batch * hq][terms][nb] of each query row (L.q, L.batch, L.hq, L.hkv,
// L.mx, L.terms, L.rotation used).
hipError_t launch_query_codes(const DecodeLaunch& L, uint8_t* codes, uint8_t* scales, hipStream_t stream);

struct Bf16DecodeLaunch {
  const uint16_t* q;
  int32_t batch, hq, hkv;
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  int32_t num_pages;
  const int32_t* block_tables;
  int32_t max_pages_per_seq;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  float softmax_scale;
  int32_t ppp, max_parts;
  uint32_t* counters;
  float* partials;
  int32_t counter_stride, slot_stride;
  float* out;
};

hipError_t launch_bf16_decode(const Bf16DecodeLaunch& L, hipStream_t stream);

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream);

constexpr int kGroup = 4;                         // query heads per KV head
constexpr int kPartialFloats = kGroup * 130;      // o[4][128], m[4], l[4] (+pad)
constexpr int kMaxSeqHeads = 16384;               // (sequence, KV head) pairs per call
// One completion ticket per (sequence, KV head), each on a 128-byte line of
// its own: every workgroup of a launch takes a device-scope ticket, and with
// the tickets of all heads on one line those atomics queue on it (the 32K
// layer's 264 workgroups finish within about 1.5 us: 17.33 -> 16.98 us apart).
constexpr int kTicketStride = 32;

// FP4 workgroups of a sequence with `parts` FP4 partitions (four per
// workgroup, at least one).
__host__ __device__ inline int fp4_wgs(int parts) {
  const int g = (parts + 3) / 4;
  return g > 0 ? g : 1;
}

// Workspace shared by both decodes. A fixed ticket region,
// [kMaxSeqHeads][kTicketStride] uint32, 2 MiB (the same for every call, so one
// zero-filled workspace serves calls of any shape), then partials
// [batch * hkv][slot_stride][kPartialFloats] float32 (slots in pairs), slot_stride = parts + 2 rounded up to even
// for parts = partitions of the longest sequence counting its partial last
// page (ceil(ceil(max_seq_len / 128) / pages_per_partition)). An FP4 decode
// of a sequence with w FP4 workgroups uses slots 0 .. w-1, one per
// workgroup (the BF16 partition is folded into slot 0); the BF16 decode uses
// one slot per partition.
constexpr size_t kTicketBytes = (size_t)kMaxSeqHeads * kTicketStride * sizeof(uint32_t);

// parts + 2 slots, rounded up to even: the slots are stored in pairs
inline int32_t workspace_slot_stride(int32_t parts) { return (parts + 3) & ~1; }

// The allocation-free decode's workspace: a device array of this many bytes
// (tickets, then partials) that the library keeps per GPU. noalloc_scratch
// returns its address on the current device; the first call on a device also
// enqueues the zeroing of its ticket words on `stream`.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

inline size_t workspace_bytes_for(int32_t batch, int32_t hkv, int32_t parts) {
  return kTicketBytes + (size_t)batch * hkv * workspace_slot_stride(parts) * kPartialFloats * sizeof(float);
}

}  // namespace bdfp4
