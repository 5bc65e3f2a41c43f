// BF16-KV paged decode attention for gfx950: the unquantized baseline arm
// (kv_cache_dtype "auto" in the KV_MODES of "BitDecoding-FP4
// evaluation/config.py"), with the same split-K partials and merge as the FP4
// decode and a plan of its own (up to 16 pages per partition, about 512
// workgroups: a BF16 page is 4.5 times the bytes of an NVFP4 one).
//
// Pages are bf16 [page][KV head][128 tokens][128 channels]. One workgroup (4
// waves) per (sequence, KV head, partition of pages_per_partition pages):
//  * pass 1: QK^T with v_mfma_f32_16x16x32_bf16; A = the 4 bf16 query rows
//    (exact operands), B = 16 tokens per tile, a lane holding 32 consecutive
//    channels of one token (one 64-byte run; the wave reads 4 KiB contiguous
//    per tile), the page's 8 tiles requested together. Logits to LDS, tokens
//    at or past L masked.
//  * partition max; p = exp(t - m) in float32 (not rounded to bf16).
//  * pass 2: PV on the vector ALU in float32: each wave takes a quarter of the
//    partition's tokens, each lane two channels for all 4 heads; one 256-byte
//    coalesced V row per token per wave, a page's 32 rows requested together.
#include "codec.hpp"
#include "launch.hpp"
#include "merge.hpp"

namespace bdfp4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxTokB = 16 * kPage;
constexpr float kNegInfB = -__builtin_inff();

struct SmemB {
  float logit[kMaxTokB * 4];   // [token][head]; p after the max
  float o[4][4][kD];           // [wave][head][channel]
  float red[4][4];
  float lsum[4][4];
  int flag;
  int ticket;
};

struct Bf16Args {
  Bf16DecodeLaunch L;
};

__global__ void __launch_bounds__(256) bf16_decode_kernel(Bf16Args A) {
  __shared__ __align__(16) SmemB sm;
  const Bf16DecodeLaunch& P = A.L;
  const int nps = P.max_parts;                  // workgroups per (sequence, KV head)
  const int s = blockIdx.x % nps;
  const int bh = blockIdx.x / nps;
  const int b = bh / P.hkv, h = bh - b * P.hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  MergeCtx C;
  C.counters = P.counters;
  C.partials = P.partials;
  C.out = P.out;
  C.hq = P.hq;
  C.hkv = P.hkv;
  C.counter_stride = P.counter_stride;
  C.slot_stride = P.slot_stride;

  const int L = P.seq_lens[b];
  const int npages = L > 0 ? (L + kPage - 1) / kPage : 0;
  if (L < 1 || L > P.max_seq_len || npages > P.max_pages_per_seq) {
    if (s == 0) poison_rows(P.out, P.hq, b, h);
    return;
  }
  const int nparts = (npages + P.ppp - 1) / P.ppp;
  if (s >= nparts) return;
  const int p0 = s * P.ppp;
  const int npg = min(npages, p0 + P.ppp) - p0;
  const int32_t* bt = P.block_tables + (size_t)b * P.max_pages_per_seq + p0;
  if (tid == 0) sm.flag = 0;

  // A operands: row = lane & 15 (heads 0..3), k-group kg = lane >> 4, MFMA c
  // covers channels 32 kg + 8 c + [0, 8)
  const int row = lane & 15, kg = lane >> 4;
  bf16x8_t aq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (row < 4) {
      const uint4 t = *reinterpret_cast<const uint4*>(P.q + ((size_t)b * P.hq + h * kGroup + row) * kD + 32 * kg + 8 * c);
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
    aq[c] = __builtin_bit_cast(bf16x8_t, v);
  }
  __syncthreads();
  const float sigma = P.softmax_scale;
  float mrun[4] = {kNegInfB, kNegInfB, kNegInfB, kNegInfB};
  bool bad = false;
  for (int pi = wave; pi < npg; pi += 4) {
    int phys = bt[pi];
    if (phys < 0 || phys >= P.num_pages) { bad = true; phys = 0; }
    const uint16_t* kp = P.k_pages + ((size_t)phys * P.hkv + h) * (kPage * kD);
    // the page's 8 tiles requested together (one memory round trip per page)
    uint4 kw[8][4];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint4* src = reinterpret_cast<const uint4*>(kp + (size_t)(16 * t + row) * kD + 32 * kg);
#pragma unroll
      for (int c = 0; c < 4; ++c) kw[t][c] = src[c];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 w = kw[t][c];
        const u32x4_t v = {w.x, w.y, w.z, w.w};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[c], __builtin_bit_cast(bf16x8_t, v), acc, 0, 0, 0);
      }
      if (lane < 16) {
        const int local = pi * kPage + 16 * t + lane;
        const bool live = p0 * kPage + local < L;
        float4 lg;
        lg.x = live ? sigma * acc[0] : kNegInfB;
        lg.y = live ? sigma * acc[1] : kNegInfB;
        lg.z = live ? sigma * acc[2] : kNegInfB;
        lg.w = live ? sigma * acc[3] : kNegInfB;
        *reinterpret_cast<float4*>(&sm.logit[local * 4]) = lg;
        mrun[0] = fmaxf(mrun[0], lg.x);
        mrun[1] = fmaxf(mrun[1], lg.y);
        mrun[2] = fmaxf(mrun[2], lg.z);
        mrun[3] = fmaxf(mrun[3], lg.w);
      }
    }
  }
  if (bad) sm.flag = 1;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float v = mrun[g];
    for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    mrun[g] = v;
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) sm.red[wave][g] = mrun[g];
  }
  __syncthreads();
  float m[4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
    m[g] = fmaxf(fmaxf(sm.red[0][g], sm.red[1][g]), fmaxf(sm.red[2][g], sm.red[3][g]));
  // p = exp(t - m) in place, l per head
  const int ntok = npg * kPage;
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = tid; i < ntok; i += 256) {
    float4 t = *reinterpret_cast<float4*>(&sm.logit[i * 4]);
    t.x = m[0] == kNegInfB ? 0.f : __expf(t.x - m[0]);
    t.y = m[1] == kNegInfB ? 0.f : __expf(t.y - m[1]);
    t.z = m[2] == kNegInfB ? 0.f : __expf(t.z - m[2]);
    t.w = m[3] == kNegInfB ? 0.f : __expf(t.w - m[3]);
    *reinterpret_cast<float4*>(&sm.logit[i * 4]) = t;
    ls[0] += t.x; ls[1] += t.y; ls[2] += t.z; ls[3] += t.w;
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float v = ls[g];
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    ls[g] = v;
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) sm.lsum[wave][g] = ls[g];
  }
  __syncthreads();
  // PV: wave takes tokens local = wave, wave+4, ...; lane owns channels 2 lane, 2 lane + 1
  float o[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
  for (int pi = 0; pi < npg; ++pi) {
    int phys = bt[pi];
    if (phys < 0 || phys >= P.num_pages) phys = 0;
    const uint16_t* vp = P.v_pages + ((size_t)phys * P.hkv + h) * (kPage * kD);
    const int tmax = min(kPage, L - (p0 + pi) * kPage);
    // the wave's 32 rows of the page (tokens wave + 4 i) requested together;
    // a row at or past tmax reads row tmax - 1 (in the page) and is skipped
    uint32_t vw[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int t = min(wave + 4 * i, tmax - 1);
      vw[i] = *reinterpret_cast<const uint32_t*>(vp + (size_t)t * kD + 2 * lane);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int t = wave + 4 * i;
      if (t < tmax) {
        const float4 p = *reinterpret_cast<const float4*>(&sm.logit[(pi * kPage + t) * 4]);
        const float v0 = bf16_lo(vw[i]), v1 = bf16_hi(vw[i]);
        o[0][0] = fmaf(p.x, v0, o[0][0]); o[0][1] = fmaf(p.x, v1, o[0][1]);
        o[1][0] = fmaf(p.y, v0, o[1][0]); o[1][1] = fmaf(p.y, v1, o[1][1]);
        o[2][0] = fmaf(p.z, v0, o[2][0]); o[2][1] = fmaf(p.z, v1, o[2][1]);
        o[3][0] = fmaf(p.w, v0, o[3][0]); o[3][1] = fmaf(p.w, v1, o[3][1]);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<float2*>(&sm.o[wave][g][2 * lane]) = make_float2(o[g][0], o[g][1]);
  __syncthreads();
  const int head = tid >> 6, d = (tid & 63) * 2;
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    o0 += sm.o[w][head][d];
    o1 += sm.o[w][head][d + 1];
  }
  const bool poisoned = sm.flag != 0;
  const float nan = __builtin_nanf("");
  float mm[4], ll[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    mm[g] = poisoned ? 0.0f : m[g];
    ll[g] = poisoned ? 1.0f : (sm.lsum[0][g] + sm.lsum[1][g]) + (sm.lsum[2][g] + sm.lsum[3][g]);
  }
  Partial mine;
  mine.o0 = poisoned ? nan : o0;
  mine.o1 = poisoned ? nan : o1;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    mine.m[g] = mm[g];
    mine.l[g] = ll[g];
  }
  write_partial(partial_writer(C, bh, s), mine);
  uint32_t* ticket = C.counters + (size_t)bh * C.counter_stride;
  if (take_ticket(ticket, 1, &sm.ticket) + 1 == nparts) {
    merge_out(C, b, h, nparts, false);
    reset_ticket(ticket);
  }
}

}  // namespace

hipError_t launch_bf16_decode(const Bf16DecodeLaunch& L, hipStream_t stream) {
  Bf16Args A;
  A.L = L;
  // partition slots 0 .. max_parts-1 (there is no separate BF16 partition)
  const dim3 grid((unsigned)(L.batch * L.hkv * L.max_parts)), block(256u);
  hipLaunchKernelGGL(bf16_decode_kernel, grid, block, 0, stream, A);
  return hipGetLastError();
}

}  // namespace bdfp4
