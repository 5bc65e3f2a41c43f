// Split-K partials and their log-sum-exp merge, shared by the FP4 and BF16
// decodes.
//
// A partial (kPartialFloats floats) holds, for the 4 query heads of a KV
// head, o[4][128] (unnormalized: sum over its tokens of p v) at 0, m[4] (the
// maximum logit, sigma included) at 512 and l[4] = sum p at 516. Merging
// partials s gives
//   M = max m_s, L = sum l_s e^(m_s - M), o = sum o_s e^(m_s - M)
// (partials with m_s = -inf are empty and weigh 0), and the output is o / L.
// The workspace layout (tickets, slots) is described with workspace_layout.
//
// Completion is counted with tickets: a workgroup stores its partial, then
// takes a ticket; the one that draws the last ticket of its set does the
// merge of that set and puts the ticket back to zero, so a workspace zeroed
// once stays reusable. The FP4 decode merges in two levels (groups of
// fp4_group_size workgroups, then the group results and the BF16 partition), so
// most of the merging overlaps the workgroups still streaming and the last
// one to finish reads only a few partials.
//
// Visibility without cache flushes: partials are written and read with
// 16-byte buffer accesses carrying the SC1 cache policy (coherent at device
// scope: the stores are written through to the device coherence point
// instead of being held in one XCD's L2, and the merging workgroup's loads
// are not served from a possibly stale L2 line). Every thread waits for its
// stores to complete (s_waitcnt vmcnt(0)) before the workgroup barrier that
// precedes a ticket. A generic agent-scope fence would instead write back
// the whole L2 of the XCD for every partition.
#pragma once

#include "codec.hpp"
#include "launch.hpp"

namespace bdfp4 {

struct MergeCtx {
  uint32_t* counters;   // [sequence * hkv][counter_stride] tickets
  float* partials;      // [sequence * hkv][slot_stride][kPartialFloats]
  float* out;
  int32_t hq, hkv, counter_stride, slot_stride;
};

__device__ __forceinline__ float* partial_slot(const MergeCtx& C, int bh, int s) {
  return C.partials + ((size_t)bh * C.slot_stride + s) * kPartialFloats;
}

constexpr int kCachePolicySc1 = 16;
constexpr int kRawBufferWord3 = 0x00020000;   // 32-bit data format, untyped access

// Resource over the slots of one (sequence, KV head): an offset past them
// reads 0 / writes nothing instead of leaving the workspace.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const MergeCtx& C, int bh) {
  return __builtin_amdgcn_make_buffer_rsrc(partial_slot(C, bh, 0), (short)0, C.slot_stride * kPartialFloats * 4,
                                           kRawBufferWord3);
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

// Stores one partial. Thread t (of 256) holds o[t >> 6][2 (t & 63) .. +2];
// pairs of lanes combine into 16-byte stores; thread 0 stores m[4] and l[4].
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

// All 256 threads: wait until this thread's stores are complete, then add
// inc to the ticket; every thread gets the ticket's previous value.
__device__ __forceinline__ int take_ticket(uint32_t* ticket, int inc, int* s_ticket) {
  __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0): this thread's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0)
    *s_ticket = (int)__hip_atomic_fetch_add(ticket, (uint32_t)inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *s_ticket;
}

__device__ __forceinline__ void reset_ticket(uint32_t* ticket) {
  if (threadIdx.x == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merges slots [first, first + n) of (sequence b, KV head h); all 256
// threads. With to_slot >= 0 the result is stored as a partial in that slot,
// otherwise out = o / L is written. s_red: LDS scratch of at least 16
// floats; s_w: LDS scratch of w_cap floats (w_cap >= 1024).
// One memory round trip for up to 32 slots: each thread issues the loads of
// its share of o (float4 t & 127 of o for the slots of parity t >> 7)
// together with the (m, l) of slot t, then M, the weights e^(m_s - M) (in
// LDS) and L are formed while the o loads land.
constexpr int kMergeBatch = 16;                  // slots per parity per round trip

__device__ __forceinline__ void merge_slots(const MergeCtx& C, float* s_red, float* s_w, int w_cap, int b, int h,
                                            int first, int n, int to_slot) {
  const int bh = b * C.hkv + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float ninf = -__builtin_inff();
  const __amdgpu_buffer_rsrc_t R = partial_rsrc(C, bh);
  constexpr int kSlotBytes = kPartialFloats * 4;
  const int base = first * kSlotBytes;
  const int q = tid & 127, par = tid >> 7, head = q >> 5;
  // the weights of slots [0, n_w) live in LDS past the o reduction area
  const int n_w = min(n, (w_cap - 1024) / 4);
  float* s_wt = s_w + 1024;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float M[4] = {ninf, ninf, ninf, ninf};
  for (int s0 = 0; s0 < n; s0 += 2 * kMergeBatch) {
    float4 ov[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int s = s0 + par + 2 * k;
      ov[k] = s < n ? cload4(R, base + s * kSlotBytes + q * 16) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (s0 == 0) {
      // M and L over all slots (thread t takes slots t, t + 256, ...)
      float4 mv[4], lv[4];
      float mx[4] = {ninf, ninf, ninf, ninf};
      for (int sb = 0; sb < n; sb += 1024) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int s = sb + tid + 256 * k;
          mv[k] = s < n ? cload4(R, base + s * kSlotBytes + 512 * 4) : make_float4(ninf, ninf, ninf, ninf);
          lv[k] = s < n ? cload4(R, base + s * kSlotBytes + 516 * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          mx[0] = fmaxf(mx[0], mv[k].x); mx[1] = fmaxf(mx[1], mv[k].y);
          mx[2] = fmaxf(mx[2], mv[k].z); mx[3] = fmaxf(mx[3], mv[k].w);
        }
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
#pragma unroll
      for (int g = 0; g < 4; ++g)
        M[g] = fmaxf(fmaxf(s_red[g], s_red[4 + g]), fmaxf(s_red[8 + g], s_red[12 + g]));
      __syncthreads();
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
      for (int sb = 0; sb < n; sb += 1024) {
        if (sb > 0) {                            // more than 1024 slots: reload (m, l)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int s = sb + tid + 256 * k;
            mv[k] = s < n ? cload4(R, base + s * kSlotBytes + 512 * 4) : make_float4(ninf, ninf, ninf, ninf);
            lv[k] = s < n ? cload4(R, base + s * kSlotBytes + 516 * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int s = sb + tid + 256 * k;
          const float mm[4] = {mv[k].x, mv[k].y, mv[k].z, mv[k].w}, ll[4] = {lv[k].x, lv[k].y, lv[k].z, lv[k].w};
          float w[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            w[g] = mm[g] == ninf ? 0.0f : __expf(mm[g] - M[g]);
            ls[g] = fmaf(w[g], ll[g], ls[g]);
          }
          if (s < n_w) *reinterpret_cast<float4*>(s_wt + 4 * s) = make_float4(w[0], w[1], w[2], w[3]);
        }
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
    }
    const float Mh = head == 0 ? M[0] : (head == 1 ? M[1] : (head == 2 ? M[2] : M[3]));
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int s = s0 + par + 2 * k;
      float w = 0.0f;
      if (s < n_w) {
        w = s_wt[4 * s + head];
      } else if (s < n) {
        const float4 m = cload4(R, base + s * kSlotBytes + 512 * 4);
        const float ms = head == 0 ? m.x : (head == 1 ? m.y : (head == 2 ? m.z : m.w));
        w = ms == ninf ? 0.0f : __expf(ms - Mh);
      }
      acc.x = fmaf(w, ov[k].x, acc.x);
      acc.y = fmaf(w, ov[k].y, acc.y);
      acc.z = fmaf(w, ov[k].z, acc.z);
      acc.w = fmaf(w, ov[k].w, acc.w);
    }
  }
  __syncthreads();
  reinterpret_cast<float4*>(s_w)[tid] = acc;     // [parity][q]: o reduction area s_w[0, 1024)
  __syncthreads();
  const int oh = tid >> 6, od = 2 * (tid & 63);
  float L4[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) L4[g] = (s_red[g] + s_red[4 + g]) + (s_red[8 + g] + s_red[12 + g]);
  const float* lo_par = s_w + oh * kD + od;      // parity 0: float4 index q = oh * 32 + od / 4
  const float r0 = lo_par[0] + lo_par[512], r1 = lo_par[1] + lo_par[513];
  if (to_slot >= 0) {
    write_partial(partial_writer(C, bh, to_slot), r0, r1, M, L4);
  } else {
    const float Lo = oh == 0 ? L4[0] : (oh == 1 ? L4[1] : (oh == 2 ? L4[2] : L4[3]));
    float* out = C.out + ((size_t)b * C.hq + h * kGroup + oh) * kD + od;
    *reinterpret_cast<float2*>(out) = make_float2(r0 / Lo, r1 / Lo);
  }
}

// NaN output rows for a sequence whose length or pages are invalid.
__device__ __forceinline__ void poison_rows(float* out, int hq, int b, int h) {
  float* o = out + ((size_t)b * hq + h * kGroup) * kD;
  o[threadIdx.x] = __builtin_nanf("");
  o[threadIdx.x + 256] = __builtin_nanf("");
}

}  // namespace bdfp4
