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
// Visibility without cache flushes: partials are written and read with
// 16-byte buffer accesses carrying the SC1 cache policy (coherent at device
// scope: the stores are written through to the device coherence point
// instead of being held in one XCD's L2, and the merging workgroup's loads
// are not served from a possibly stale L2 line). Every thread waits for its
// stores to complete (s_waitcnt vmcnt(0)) before the workgroup barrier that
// precedes the ticket. A generic agent-scope fence would instead write back
// the whole L2 of the XCD for every partition.
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

// Device-coherent partial stores and loads (see above): 16-byte buffer
// accesses with the SC1 cache policy (coherent at device scope, so neither
// side is served by a possibly stale line of one XCD's L2). The resource
// covers the partials of one (sequence, KV head); offsets are in bytes.
constexpr int kCachePolicySc1 = 16;
constexpr int kRawBufferWord3 = 0x00020000;   // 32-bit data format, untyped access

// Resource over the max_parts + 1 slots of one (sequence, KV head): an
// offset past them reads 0 / writes nothing instead of leaving the workspace.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const MergeCtx& C, int bh) {
  return __builtin_amdgcn_make_buffer_rsrc(partial_slot(C, bh, 0), (short)0,
                                           (C.max_parts + 1) * kPartialFloats * 4, kRawBufferWord3);
}
__device__ __forceinline__ float4 cload4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 v = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCachePolicySc1));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void cstore4(__amdgpu_buffer_rsrc_t r, int byte_off, float4 v) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, byte_off, 0, kCachePolicySc1);
}

// Writes one partial: o[4][128] (thread t of 256 stores o[t >> 6][2 (t & 63)
// .. +2] as part of a 16-byte row written by every other thread), then m[4]
// and l[4] (thread 0).
struct PartialWriter {
  __amdgpu_buffer_rsrc_t r;
  int slot_off;   // byte offset of the slot
};

__device__ __forceinline__ PartialWriter partial_writer(const MergeCtx& C, int bh, int s) {
  PartialWriter w;
  w.r = partial_rsrc(C, bh);
  w.slot_off = s * kPartialFloats * 4;
  return w;
}

// o of 2 consecutive channels per thread: pairs are combined across lanes
// (t, t ^ 1) so even lanes store 16 bytes.
__device__ __forceinline__ void write_partial(const PartialWriter& W, float o0, float o1, const float* m4,
                                              const float* l4) {
  const int t = threadIdx.x;
  const float p0 = __shfl_xor(o0, 1, 64), p1 = __shfl_xor(o1, 1, 64);
  if ((t & 1) == 0) {
    const int head = t >> 6, d = 2 * (t & 63);
    cstore4(W.r, W.slot_off + (head * kD + d) * 4, make_float4(o0, o1, p0, p1));
  }
  if (t == 0) {
    cstore4(W.r, W.slot_off + 512 * 4, make_float4(m4[0], m4[1], m4[2], m4[3]));
    cstore4(W.r, W.slot_off + 516 * 4, make_float4(l4[0], l4[1], l4[2], l4[3]));
  }
}

// All 256 threads call this after the workgroup's partials are stored.
// n_slots: number of partials of this (sequence, KV head); inc: how many of
// them this workgroup stored (the ticket advances by inc). s_red: LDS scratch
// of at least 16 floats; s_w: LDS scratch of w_cap floats (w_cap >= 4096);
// s_ticket: one LDS int.
// The merging workgroup issues its loads in batches before using them:
// (m, l) of every slot (one slot per thread), then the weighted o sum with
// thread t owning 4 channels (16 bytes) of o for the slots of parity t >> 7.
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
  const __amdgpu_buffer_rsrc_t R = partial_rsrc(C, bh);
  constexpr int kSlotBytes = kPartialFloats * 4;
  // (m, l) per slot; maximum per head
  const bool w_in_lds = n_slots * 4 <= w_cap - 2048;     // the o reduction below uses s_w[0, 2048)
  float* s_wt = s_w + 2048;
  float mx[4] = {ninf, ninf, ninf, ninf};
  for (int s = tid; s < n_slots; s += 256) {
    const float4 m = cload4(R, s * kSlotBytes + 512 * 4);
    mx[0] = fmaxf(mx[0], m.x); mx[1] = fmaxf(mx[1], m.y); mx[2] = fmaxf(mx[2], m.z); mx[3] = fmaxf(mx[3], m.w);
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
  // weights e^(m_s - M) and the per-head normaliser
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = tid; s < n_slots; s += 256) {
    const float4 m = cload4(R, s * kSlotBytes + 512 * 4);
    const float4 l = cload4(R, s * kSlotBytes + 516 * 4);
    const float mm[4] = {m.x, m.y, m.z, m.w}, ll[4] = {l.x, l.y, l.z, l.w};
    float w[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      w[g] = mm[g] == ninf ? 0.0f : __expf(mm[g] - M[g]);
      ls[g] = fmaf(w[g], ll[g], ls[g]);
    }
    if (w_in_lds) *reinterpret_cast<float4*>(s_wt + 4 * s) = make_float4(w[0], w[1], w[2], w[3]);
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
  // o: thread t owns float4 q = t & 127 of o (head q >> 5, channels
  // 4 (q & 31) .. +4) for the slots s = (t >> 7) + 2k, 16 slots per batch
  const int q = tid & 127, par = tid >> 7, head = q >> 5;
  const float Mh = head == 0 ? M[0] : (head == 1 ? M[1] : (head == 2 ? M[2] : M[3]));
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int kBatch = 16;
  for (int s0 = par; s0 < n_slots; s0 += 2 * kBatch) {
    float4 ov[kBatch];
    float wv[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int s = s0 + 2 * k;
      ov[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      wv[k] = 0.0f;
      if (s < n_slots) {
        ov[k] = cload4(R, s * kSlotBytes + q * 16);
        if (w_in_lds) {
          wv[k] = s_wt[4 * s + head];
        } else {
          const float4 m = cload4(R, s * kSlotBytes + 512 * 4);
          const float ms = head == 0 ? m.x : (head == 1 ? m.y : (head == 2 ? m.z : m.w));
          wv[k] = ms == ninf ? 0.0f : __expf(ms - Mh);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      acc.x = fmaf(wv[k], ov[k].x, acc.x);
      acc.y = fmaf(wv[k], ov[k].y, acc.y);
      acc.z = fmaf(wv[k], ov[k].z, acc.z);
      acc.w = fmaf(wv[k], ov[k].w, acc.w);
    }
  }
  __syncthreads();                               // weights no longer needed: reuse s_w
  reinterpret_cast<float4*>(s_w)[tid] = acc;     // [parity][q]
  __syncthreads();
  const int oh = tid >> 6, od = 2 * (tid & 63);
  const float Lo = s_red[oh] + s_red[4 + oh] + s_red[8 + oh] + s_red[12 + oh];
  const float* lo_par = s_w + oh * kD + od;      // parity 0: float4 index q = oh * 32 + od / 4
  const float r0 = lo_par[0] + lo_par[512], r1 = lo_par[1] + lo_par[513];
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
