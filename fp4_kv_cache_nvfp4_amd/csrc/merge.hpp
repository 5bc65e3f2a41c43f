// Split-K partials and the last-arriver log-sum-exp merge shared by the FP4
// and BF16 decodes.
//
// Workspace: [kCounterBytes of uint32 tickets, one per (sequence, KV head)]
// then partials [sequence][KV head][partition][kPartialFloats] with
// o[4][128] at 0, m[4] at 512, l[4] at 516. Each partition workgroup writes
// its partial, releases it, and takes a ticket; the workgroup that draws the
// last ticket acquires all partials, merges them
//   M = max m_s, L = sum l_s e^(m_s - M), out = sum o_s e^(m_s - M) / L
// (partials with m_s = -inf are empty and skipped), writes the output and
// puts the ticket back to zero, so a workspace zeroed once stays reusable.
#pragma once

#include "codec.hpp"
#include "launch.hpp"

namespace bdfp4 {

struct MergeCtx {
  uint32_t* counters;
  float* partials;
  float* out;
  int32_t hq, hkv, max_parts;   // max_parts + 1 partial slots per (sequence, KV head)
};

__device__ __forceinline__ float* partial_slot(const MergeCtx& C, int bh, int s) {
  return C.partials + ((size_t)bh * (C.max_parts + 1) + s) * kPartialFloats;
}

// All 256 threads call this after the partial of slot s is stored.
// n_slots: number of partials of this (sequence, KV head).
__device__ __forceinline__ void publish_and_merge(const MergeCtx& C, int* s_ticket, int b, int h, int n_slots) {
  const int bh = b * C.hkv + h;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) *s_ticket = (int)atomicAdd(&C.counters[bh], 1u);
  __syncthreads();
  if (*s_ticket != n_slots - 1) return;
  __threadfence();
  const int tid = threadIdx.x;
  const int head = tid >> 6, d = (tid & 63) * 2;
  const float ninf = -__builtin_inff();
  float M = ninf;
  for (int s = 0; s < n_slots; ++s) M = fmaxf(M, partial_slot(C, bh, s)[512 + head]);
  float Lsum = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int s = 0; s < n_slots; ++s) {
    const float* P = partial_slot(C, bh, s);
    const float ms = P[512 + head];
    if (ms == ninf) continue;
    const float w = __expf(ms - M);
    Lsum = fmaf(w, P[516 + head], Lsum);
    const float2 o = *reinterpret_cast<const float2*>(P + head * kD + d);
    o0 = fmaf(w, o.x, o0);
    o1 = fmaf(w, o.y, o1);
  }
  float* out = C.out + ((size_t)b * C.hq + h * kGroup + head) * kD + d;
  *reinterpret_cast<float2*>(out) = make_float2(o0 / Lsum, o1 / Lsum);
  if (tid == 0) C.counters[bh] = 0u;
}

// NaN output rows for a sequence whose length or pages are invalid.
__device__ __forceinline__ void poison_rows(float* out, int hq, int b, int h) {
  float* o = out + ((size_t)b * hq + h * kGroup) * kD;
  o[threadIdx.x] = __builtin_nanf("");
  o[threadIdx.x + 256] = __builtin_nanf("");
}

}  // namespace bdfp4
