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
  int32_t num_pages, hkv, n_pages, rotation;
  int32_t k_mode, v_mode;  // 1 amax6, 2 four_six, 3 mxfp4_search
};

hipError_t launch_writer(const WriterLaunch& L, hipStream_t stream);

hipError_t launch_rows(const void* rows, int n_rows, const float* shift, int rotation, int mode,
                       int terms, uint8_t* codes, uint8_t* scales, hipStream_t stream);

hipError_t launch_p_blocks(const float* pp, int n_blocks, int mode, float tau, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream);

struct DecodeLaunch {
  // recipe
  int32_t sink, rotation, key_smoothing, mx, k_four_six, p_mode, terms, c;
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
  void* workspace;
  float* out;
};

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream);

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
  void* workspace;
  float* out;
};

hipError_t launch_bf16_decode(const Bf16DecodeLaunch& L, hipStream_t stream);

// Workspace layout shared by both decodes: a fixed counter region followed
// by the per-partition partials.
constexpr size_t kCounterBytes = 65536;          // 16384 (sequence, KV head) tickets
constexpr int kMaxSeqHeads = 16384;
constexpr int kGroup = 4;                         // query heads per KV head
constexpr int kPartialFloats = kGroup * 130;      // o[4][128], m[4], l[4] (+pad)

}  // namespace bdfp4
