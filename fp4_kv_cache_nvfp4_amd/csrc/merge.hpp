// Split-K partials and the last-arriver log-sum-exp merge shared by the FP4
// and BF16 decodes.
//
// Workspace: [kCounterBytes of uint32 tickets, one per (sequence, KV head)]
// then partials [sequence][KV head][partition][kPartialFloats] with
// o[4][128] at 0, m[4] at 512, l[4] at 516. Each partition workgroup writes
// its partial, makes it visible device-wide, and takes a ticket; the
// workgroup that draws the last ticket reads all partials, merges them
//   M = max m_s, L = sum l_s e^(m_s - M), out = sum o_s e^(m_s - M) / L
// (partials with m_s = -inf are empty and skipped), writes the output and
// puts the ticket back to zero, so a workspace zeroed once stays reusable.
//
// Visibility without cache flushes: the partials are written with agent-scope
// relaxed atomic stores (written through to the device coherence point, not
// held in one XCD's L2), every thread waits for its stores to complete
// (s_waitcnt vmcnt(0)) before the workgroup barrier that precedes the ticket,
// and the merging workgroup reads them with agent-scope atomic loads (not
// served from a possibly stale L2 line). A generic agent-scope fence would
// instead write back the whole L2 of the XCD for every partition.
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

// Device-coherent partial stores and loads (see above).
__device__ __forceinline__ void pstore(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void pstore2(float* p, float a, float b) {
  pstore(p, a);
  pstore(p + 1, b);
}
__device__ __forceinline__ float pload(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All 256 threads call this after the workgroup's partials are stored.
// n_slots: number of partials of this (sequence, KV head); inc: how many of
// them this workgroup stored (the ticket advances by inc). s_red: LDS scratch
// of at least 16 floats; s_w: LDS scratch of w_cap floats; s_ticket: one LDS
// int.
// The merging workgroup reads the slots in parallel: the per-head maxima and
// normalisers are block reductions over slots (thread t takes slots t, t+256,
// ...), the weights e^(m_s - M) go to LDS, and the weighted sum of o is split
// over four groups of 64 threads (each a quarter of the slots, 8 channels
// per thread, all its loads issued together) and added up in LDS.
__device__ __forceinline__ void publish_and_merge(const MergeCtx& C, int* s_ticket, float* s_red, float* s_w,
                                                  int w_cap, int b, int h, int n_slots, int inc = 1) {
  const int bh = b * C.hkv + h;
  __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0): this thread's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0)
    *s_ticket = (int)__hip_atomic_fetch_add(&C.counters[bh], (uint32_t)inc, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*s_ticket + inc != n_slots) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float ninf = -__builtin_inff();
  const float* base = partial_slot(C, bh, 0);
  // per-head maximum
  float mx[4] = {ninf, ninf, ninf, ninf};
  for (int s = tid; s < n_slots; s += 256) {
    const float* P = base + (size_t)s * kPartialFloats + 512;
#pragma unroll
    for (int g = 0; g < 4; ++g) mx[g] = fmaxf(mx[g], pload(P + g));
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    for (int o = 32; o >= 1; o >>= 1) mx[g] = fmaxf(mx[g], __shfl_xor(mx[g], o, 64));
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) s_red[wave * 4 + g] = mx[g];
  }
  __syncthreads();
  float M[4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
    M[g] = fmaxf(fmaxf(s_red[g], s_red[4 + g]), fmaxf(s_red[8 + g], s_red[12 + g]));
  __syncthreads();
  // weights and per-head normaliser
  const bool w_in_lds = n_slots * 4 <= w_cap;
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = tid; s < n_slots; s += 256) {
    const float* P = base + (size_t)s * kPartialFloats + 512;
    const float mm[4] = {pload(P), pload(P + 1), pload(P + 2), pload(P + 3)};
    const float ll[4] = {pload(P + 4), pload(P + 5), pload(P + 6), pload(P + 7)};
    float w[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      w[g] = mm[g] == ninf ? 0.0f : __expf(mm[g] - M[g]);
      ls[g] = fmaf(w[g], ll[g], ls[g]);
    }
    if (w_in_lds) *reinterpret_cast<float4*>(s_w + 4 * s) = make_float4(w[0], w[1], w[2], w[3]);
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    for (int o = 32; o >= 1; o >>= 1) ls[g] += __shfl_xor(ls[g], o, 64);
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) s_red[wave * 4 + g] = ls[g];
  }
  __syncthreads();
  // o: group `wave` takes slots wave, wave + 4, ...; lane owns head lane >> 4,
  // channels 8 (lane & 15) .. +8
  const int head = lane >> 4, c0 = 8 * (lane & 15);
  const float Mh = M[0] * (head == 0) + M[1] * (head == 1) + M[2] * (head == 2) + M[3] * (head == 3);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int s = wave; s < n_slots; s += 4) {
    const float* P = base + (size_t)s * kPartialFloats;
    float w;
    if (w_in_lds) {
      w = s_w[4 * s + head];
    } else {
      const float ms = pload(P + 512 + head);
      w = ms == ninf ? 0.0f : __expf(ms - Mh);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = fmaf(w, pload(P + head * kD + c0 + k), acc[k]);
  }
  const float Lh = s_red[head] + s_red[4 + head] + s_red[8 + head] + s_red[12 + head];
  __syncthreads();                               // weights no longer needed: reuse s_w
  float* so = s_w;                               // [group][head][128]
  *reinterpret_cast<float4*>(so + (wave * 4 + head) * kD + c0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(so + (wave * 4 + head) * kD + c0 + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();
  const int oh = tid >> 6, od = 2 * (tid & 63);
  const float Lo = s_red[oh] + s_red[4 + oh] + s_red[8 + oh] + s_red[12 + oh];
  float r0 = 0.f, r1 = 0.f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    r0 += so[(g * 4 + oh) * kD + od];
    r1 += so[(g * 4 + oh) * kD + od + 1];
  }
  (void)Lh;
  float* out = C.out + ((size_t)b * C.hq + h * kGroup + oh) * kD + od;
  *reinterpret_cast<float2*>(out) = make_float2(r0 / Lo, r1 / Lo);
  if (tid == 0) __hip_atomic_store(&C.counters[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// NaN output rows for a sequence whose length or pages are invalid.
__device__ __forceinline__ void poison_rows(float* out, int hq, int b, int h) {
  float* o = out + ((size_t)b * hq + h * kGroup) * kD;
  o[threadIdx.x] = __builtin_nanf("");
  o[threadIdx.x + 256] = __builtin_nanf("");
}

}  // namespace bdfp4
