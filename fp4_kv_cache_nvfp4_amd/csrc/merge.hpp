// Split-K partials and their log-sum-exp merge, shared by the FP4 and BF16
// decodes.
//
// A partial holds, for the 4 query heads of a KV head, o[4][128]
// (unnormalized: sum over its tokens of p v), m[4] (the maximum logit, sigma
// included) and l[4] = sum p: kPartialFloats floats, stored in pairs of
// slots (o_byte, ml_byte). Merging
// partials s gives
//   M = max m_s, L = sum l_s e^(m_s - M), o = sum o_s e^(m_s - M)
// (partials with m_s = -inf are empty and weigh 0), and the output is o / L.
// The workspace layout (tickets, slots) is described beside kTicketBytes.
//
// Completion is counted with tickets: a workgroup stores its partial, then
// takes the ticket of its (sequence, KV head); the one that draws the last
// ticket merges all partials in one level (their loads in one or two memory
// round trips) and puts the ticket back to zero, so a workspace zeroed once
// stays reusable. One level keeps the chain after the last partition short:
// store, ticket, loads, output.
//
// Visibility without cache flushes: partials are written and read with
// buffer accesses carrying the SC1 cache policy (coherent at device
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

// Slots are stored in pairs (2p, 2p + 1), a block of 2 kPartialFloats floats
// (slot_stride is even): o of both slots interleaved first, the 16 bytes at
// float (head * 64 + c) * 4 holding channels 2c, 2c + 1 of slot 2p, then of
// slot 2p + 1; then m[4], l[4] of slot 2p at float 1024 and of slot 2p + 1 at
// 1032. One 16-byte load thus gives a lane its two channels of two slots.
constexpr int kPairBytes = 2 * kPartialFloats * 4;
__device__ __forceinline__ int o_byte(int s, int head, int c) {
  return (s >> 1) * kPairBytes + ((head * 64 + c) * 4 + (s & 1) * 2) * 4;
}
__device__ __forceinline__ int ml_byte(int s) {      // m[4] here, l[4] 16 bytes on
  return (s >> 1) * kPairBytes + (1024 + (s & 1) * 8) * 4;
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
__device__ __forceinline__ void cstore2(__amdgpu_buffer_rsrc_t r, int byte_off, float2 v) {
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  const u2 w = {__float_as_uint(v.x), __float_as_uint(v.y)};
  __builtin_amdgcn_raw_buffer_store_b64(w, r, byte_off, 0, kCachePolicySc1);
}
__device__ __forceinline__ void cstore4(__amdgpu_buffer_rsrc_t r, int byte_off, float4 v) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, byte_off, 0, kCachePolicySc1);
}

struct PartialWriter {
  __amdgpu_buffer_rsrc_t r;
  int slot;
};

__device__ __forceinline__ PartialWriter partial_writer(const MergeCtx& C, int bh, int s) {
  PartialWriter w;
  w.r = partial_rsrc(C, bh);
  w.slot = s;
  return w;
}

// Stores one partial. Thread t (of 256) holds o[t >> 6][2 (t & 63) .. +2] and
// stores it as 8 bytes into the slot pair's interleaved o; thread 0 stores
// m[4] and l[4].
__device__ __forceinline__ void write_partial(const PartialWriter& W, float o0, float o1, const float* m4,
                                              const float* l4) {
  const int t = threadIdx.x;
  cstore2(W.r, o_byte(W.slot, t >> 6, t & 63), make_float2(o0, o1));
  if (t == 0) {
    cstore4(W.r, ml_byte(W.slot), make_float4(m4[0], m4[1], m4[2], m4[3]));
    cstore4(W.r, ml_byte(W.slot) + 16, make_float4(l4[0], l4[1], l4[2], l4[3]));
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

// One partition's result as its threads hold it: thread t has
// o[t >> 6][2 (t & 63) .. +2]; m and l are the same in every thread.
struct Partial {
  float o0, o1;
  float m[4], l[4];
};

__device__ __forceinline__ void write_partial(const PartialWriter& W, const Partial& p) {
  write_partial(W, p.o0, p.o1, p.m, p.l);
}

__device__ __forceinline__ float cload1(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kCachePolicySc1));
}
__device__ __forceinline__ float2 cload2(__amdgpu_buffer_rsrc_t r, int byte_off) {
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kCachePolicySc1));
  return make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
}

__device__ __forceinline__ float lane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
// Maximum and sum over the 64 lanes of a wave (uniform result; the sum in a
// fixed order).
__device__ __forceinline__ float wave_max(float v) {
  v = max16(v);
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}

// v[g] of a 4-array held in registers, by value selects (an indexed or
// pointer-selected access would put the array in scratch memory).
__device__ __forceinline__ float of_head(float v0, float v1, float v2, float v3, int g) {
  const float lo = g == 0 ? v0 : v1, hi = g == 2 ? v2 : v3;
  return g < 2 ? lo : hi;
}

// The normalised 128-point Hadamard rotation (H / sqrt(128), its own
// inverse) of one head's row held by a wave, lane l holding channels 2l and
// 2l + 1: stages h = 1, 2, ..., 64 of (a, b) -> (a + b, a - b) in float32,
// then the factor 1/sqrt(128), as the key rotation. All 64 lanes take part.
__device__ __forceinline__ void wave_rotate2(float& x0, float& x1) {
  const int lane = threadIdx.x & 63;
  {
    const float a = x0, b = x1;
    x0 = __fadd_rn(a, b);
    x1 = __fsub_rn(a, b);
  }
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {                 // stage h = 2 s: partner lane l ^ s
    const float p0 = __shfl_xor(x0, s, 64), p1 = __shfl_xor(x1, s, 64);
    const bool upper = (lane & s) != 0;
    x0 = upper ? __fsub_rn(p0, x0) : __fadd_rn(x0, p0);
    x1 = upper ? __fsub_rn(p1, x1) : __fadd_rn(x1, p1);
  }
  x0 = __fmul_rn(x0, inv_sqrt_d());
  x1 = __fmul_rn(x1, inv_sqrt_d());
}

// Merges the n partials of (sequence b, KV head h) and writes out = o / L.
// Each wave merges its own query head (wave g, head g) with no workgroup
// barrier: per batch of 64 (or 32) partials, lane i loads (m, l) of partial i
// and every lane loads its two channels of o of every slot of the batch, two
// slots per 16-byte load (one memory round trip, the (m, l) loads first so
// the maximum and the weights are formed while o lands); a batch after the
// first rescales what came before. The merging
// workgroup reads its own partial back like the others (its stores completed
// before it took the ticket). The resource covers the pairs of the n slots,
// so a pair past them reads 0 and needs no address select; a slot n in the
// last pair (odd n) is zeroed; either weighs 0. The
// partials are always combined in slot order (lane order for l, a fixed
// tree over slot-ordered chains for o), so the result does not depend on
// which workgroup merges: the
// output is deterministic. With extra >= 0 the partial in slot `extra` (past
// the n, the FP4 decode's BF16 partition) is merged too: its loads are
// issued ahead of the first batch's, so they share that round trip, and it
// is combined after the last batch. With rotate_back (values stored
// rotated), the merged o is rotated back before the division.
// Partials are taken in batches of kB = 32 or 64 slots: lane i loads (m, l) of
// slot i0 + i (lanes past a batch of 32 weigh 0 there; they belong to the
// next) and every lane loads its two channels of o of each slot, a slot pair
// per 16-byte load. A batch of 64 covers the 64 partials of a 128K head in
// one round trip; with at most 32 partials a batch of 32 halves the loads
// (measured with one slot per 8-byte load: 34 per wave instead of 66, under
// the 63 loads a wave's counter tracks: the 32K layer 16.9-17.1 -> 16.0-16.2
// us, the tiny case 11.2 -> 10.2 us, bit-identical: the slots past n weigh 0
// either way).
template <int kB>
__device__ __forceinline__ void merge_batches(__amdgpu_buffer_rsrc_t R, int ns, int g, int lane, float& M,
                                              float& Ls, float& o0, float& o1) {
  const float ninf = -__builtin_inff();
  for (int i0 = 0; i0 < ns; i0 += kB) {
    const int i = i0 + lane;
    const float mr = cload1(R, ml_byte(i) + g * 4);
    float lr = cload1(R, ml_byte(i) + 16 + g * 4);
    float2 ov[kB];
#pragma unroll
    for (int k = 0; k < kB; k += 2) {
      const float4 v = cload4(R, o_byte(i0 + k, g, lane));
      ov[k] = make_float2(v.x, v.y);
      ov[k + 1] = make_float2(v.z, v.w);
    }
    // with an odd n, slot n shares the last pair and lies inside the
    // resource: whatever it holds (another call's partial, or a NaN one)
    // weighs 0 and is zeroed (0 x NaN would not vanish)
    if ((ns & 1) && ns >= i0 && ns < i0 + kB) {
#pragma unroll
      for (int k = 0; k < kB; ++k)
        if (i0 + k == ns) ov[k] = make_float2(0.0f, 0.0f);
    }
    lr = i < ns ? lr : 0.0f;
    const float ms = (i < ns && lane < kB) ? mr : ninf;
    const float Mn = fmaxf(M, wave_max(ms));
    const float f = M == ninf ? 0.0f : __expf(M - Mn);     // rescale of the partials before
    const float w = ms == ninf ? 0.0f : __expf(ms - Mn);
    Ls = fmaf(Ls, f, wave_sum(w * lr));
    // the batch's weighted sum in four independent FMA chains (slots k with
    // k mod 4 = c), added in a fixed tree: a quarter of the dependent latency
    float c0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, c1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const float wk = lane_f32(w, k);
      c0[k & 3] = fmaf(wk, ov[k].x, c0[k & 3]);
      c1[k & 3] = fmaf(wk, ov[k].y, c1[k & 3]);
    }
    o0 = fmaf(o0, f, (c0[0] + c0[1]) + (c0[2] + c0[3]));
    o1 = fmaf(o1, f, (c1[0] + c1[1]) + (c1[2] + c1[3]));
    M = Mn;
  }
}

__device__ __forceinline__ void merge_out(const MergeCtx& C, int b, int h, int n, bool rotate_back,
                                          int extra = -1) {
  // (sequence, KV head) and n as scalars: the buffer resource below must
  // live in scalar registers, or every load becomes a loop over distinct values
  const int bh = __builtin_amdgcn_readfirstlane(b * C.hkv + h);
  const int ns = __builtin_amdgcn_readfirstlane(n);
  const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const float ninf = -__builtin_inff();
  // the pair blocks that hold slots 0 .. n-1 (a pair past them reads 0)
  const __amdgpu_buffer_rsrc_t R = __builtin_amdgcn_make_buffer_rsrc(partial_slot(C, bh, 0), (short)0,
                                                                     ((ns + 1) >> 1) * kPairBytes, kRawBufferWord3);
  // the extra partial, through a resource that covers its pair as well
  const int xs = __builtin_amdgcn_readfirstlane(extra);
  float mx = ninf, lx = 0.0f;
  float2 ox = make_float2(0.0f, 0.0f);
  if (xs >= 0) {
    const __amdgpu_buffer_rsrc_t RX = __builtin_amdgcn_make_buffer_rsrc(partial_slot(C, bh, 0), (short)0,
                                                                        ((xs >> 1) + 1) * kPairBytes, kRawBufferWord3);
    mx = cload1(RX, ml_byte(xs) + g * 4);
    lx = cload1(RX, ml_byte(xs) + 16 + g * 4);
    ox = cload2(RX, o_byte(xs, g, lane));
  }
  float M = ninf, Ls = 0.0f, o0 = 0.0f, o1 = 0.0f;
  // up to 64 partials in one round trip; up to 32 with half the loads
  if (ns <= 32) merge_batches<32>(R, ns, g, lane, M, Ls, o0, o1);
  else merge_batches<64>(R, ns, g, lane, M, Ls, o0, o1);
  if (xs >= 0) {
    const float Mn = fmaxf(M, mx);
    const float f = M == ninf ? 0.0f : __expf(M - Mn);
    const float w = mx == ninf ? 0.0f : __expf(mx - Mn);
    Ls = fmaf(Ls, f, w * lx);
    o0 = fmaf(w, ox.x, o0 * f);
    o1 = fmaf(w, ox.y, o1 * f);
  }
  if (rotate_back) wave_rotate2(o0, o1);                // uniform per workgroup
  float* out = C.out + ((size_t)b * C.hq + h * kGroup + g) * kD + 2 * lane;
  *reinterpret_cast<float2*>(out) = make_float2(o0 / Ls, o1 / Ls);
}

// NaN output rows for a sequence whose length or pages are invalid.
__device__ __forceinline__ void poison_rows(float* out, int hq, int b, int h) {
  float* o = out + ((size_t)b * hq + h * kGroup) * kD;
  o[threadIdx.x] = __builtin_nanf("");
  o[threadIdx.x + 256] = __builtin_nanf("");
}

}  // namespace bdfp4
