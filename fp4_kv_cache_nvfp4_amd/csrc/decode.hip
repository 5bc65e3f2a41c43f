// Paged FP4 decode attention for gfx950 over the NVFP4 / MXFP4 page cache,
// with the BF16 sink and tail handled exactly and a split-K log-sum-exp merge.
//
// Method names and constants: "BitDecoding-FP4 evaluation/config.py" (RECIPE
// dual_residual_query_quantization and underflow_aware_probability_scaling
// {c, tau}; recipe_additional_config query amax6 and query_terms;
// probability_environment amax2_or_amax6 / amax6; KV_MODES bitdecoding-nvfp4
// sink_tokens 16 and rotation; PARITY_ENGINE_KWARGS block_size 128). The
// gitdiagram "How openbitsys/bitdecoding-fp4 works": the decode interface
// dispatches to the paged attention kernel, which uses block scaling and scale
// modes; the tail control plane keeps the partial page in BF16.
//
// Grid: one workgroup (256 threads, 4 waves) per (sequence, KV head,
// partition). Partition 0 is the BF16 partition (sink + tail tokens, exact
// float32 attention of the raw query). Partitions 1..S each own
// pages_per_partition FP4 pages. A partition computes, for the 4 query heads
// of its KV head, m = max logit, l = sum exp(t - m) and o = sum P_hat v_hat,
// writes them to the workspace and takes a ticket; the last workgroup of the
// (sequence, KV head) merges all partials and resets the ticket.
//
// FP4 partition, per workgroup:
//  * prologue: the 4 query rows are rotated (128-point Hadamard, float32) and
//    quantized as Q1 + Q2 (amax6 per 16 or mxfp4_search per 32); the
//    dequantized terms are exact in 16 bits and become the A operands of
//    v_mfma_f32_16x16x32_{f16,bf16} (rows 0..3 = heads, 12 zero rows); q . mu
//    is formed from the raw float32 query.
//  * pass 1 (QK^T): each wave streams whole pages: per 16-token tile one
//    coalesced 1 KiB run of K codes (16 B per lane) plus one 16 B load of the
//    page's scales per lane; codes are converted with their block scale
//    (exactly, see deq_pair) and fed to 4 MFMAs per query term.
//    Logits sigma * (q_hat . k_hat + q . mu) go to LDS; masked (sink) slots
//    get -inf.
//  * partition max over the 4 waves.
//  * pass 2 (softmax, P quantization, PV): per 32-token chunk the 4 x 32
//    probabilities p = exp(t - m) are formed two per lane, l accumulates the
//    unquantized p, p' = c p is quantized per aligned 16-token block
//    (amax2_or_amax6 with tau, or amax6), and s * e2m1 (exact in 16 bits) is
//    staged in LDS as the A operand; V codes, stored so that a lane's 32 bytes
//    hold 8 tokens of one 8-channel group, are converted and permuted
//    into the B operand of 8 MFMAs (one per output column slab).
//  * the 4 waves' o and l are summed in LDS; o is divided by c.
#include "codec.hpp"
#include "launch.hpp"
#include "merge.hpp"

namespace bdfp4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxPpp = 16;
constexpr int kMaxTok = kMaxPpp * kPage;   // tokens of one partition
constexpr float kNegInf = -__builtin_inff();

struct DecArgs {
  DecodeLaunch L;
  uint32_t* counters;
  float* partials;
};

// ------------------------------------------------------------ small helpers

// The scaled FP4 converts of gfx950 apply only the exponent of their float32
// scale (an E8M0 scale). MXFP4 scales are powers of two and convert exactly
// to bf16. An E4M3 scale s = mant * 2^e is split: the codes are converted to
// f16 with 2^e, then multiplied by mant (at most 4 significant bits) in
// packed f16; the product has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in f16. NVFP4 operands are therefore f16,
// MXFP4 operands bf16.

__device__ __forceinline__ uint32_t cvt_bf16_pair(uint32_t w, float s, int byte) {
  bf16x2_t r;
  switch (byte) {
    case 0: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0); break;
    case 1: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1); break;
    case 2: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2); break;
    default: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3); break;
  }
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ f16x2_t cvt_f16_pair(uint32_t w, float s, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 3);
  }
}

// An element scale as (power of two for the convert, multiplier pair).
struct ElemScale {
  float p2;
  f16x2_t mant;
};

__device__ __forceinline__ ElemScale elem_scale(uint32_t code, bool mx) {
  ElemScale r;
  if (mx) {
    r.p2 = pow2_f32((int)code - 127);
    r.mant = (f16x2_t){(_Float16)1.0f, (_Float16)1.0f};
    return r;
  }
  const uint32_t e = (code >> 3) & 0xFu, m = code & 7u;
  const float mf = e == 0u ? (float)m * 0.125f : 1.0f + (float)m * 0.125f;   // exact
  r.p2 = e == 0u ? 0.015625f : __uint_as_float((e + 120u) << 23);           // 2^-6 or 2^(e-7)
  const _Float16 mh = (_Float16)mf;                                          // exact
  r.mant = (f16x2_t){mh, mh};
  return r;
}

// Dequantized pair (elements 2 byte, 2 byte + 1 of word w) as two 16-bit values.
template <bool kMx>
__device__ __forceinline__ uint32_t deq_pair(uint32_t w, const ElemScale& sc, int byte) {
  if (kMx) return cvt_bf16_pair(w, sc.p2, byte);
  const f16x2_t v = cvt_f16_pair(w, sc.p2, byte) * sc.mant;
  return __builtin_bit_cast(uint32_t, v);
}

// 8 codes of one word (element 2i in the low nibble of byte i), dequantized.
template <bool kMx>
__device__ __forceinline__ u32x4_t deq_word(uint32_t w, const ElemScale& sc) {
  u32x4_t r;
  r[0] = deq_pair<kMx>(w, sc, 0);
  r[1] = deq_pair<kMx>(w, sc, 1);
  r[2] = deq_pair<kMx>(w, sc, 2);
  r[3] = deq_pair<kMx>(w, sc, 3);
  return r;
}

// D += A B on 16x16x32 tiles: bf16 operands for MXFP4, f16 for NVFP4.
template <bool kMx>
__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  if (kMx)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                               __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// 16-bit operand bits of an exactly representable float32 value.
template <bool kMx>
__device__ __forceinline__ uint32_t op16(float v) {
  if (kMx) return __float_as_uint(v) >> 16;                 // bf16: exact values truncate exactly
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) {
  return __shfl_xor(v, m, 64);
}

__device__ __forceinline__ uint8_t byte_of(const uint4& v, int i) {
  const uint32_t w = i < 4 ? v.x : (i < 8 ? v.y : (i < 12 ? v.z : v.w));
  return (uint8_t)(w >> (8 * (i & 3)));
}

// ------------------------------------------------------------ shared memory

struct Smem {
  float logit[kMaxTok * 4];                 // [token][head], reused for o reduction
  uint16_t qhat[2][4][kD];                  // bf16 bits of the dequantized terms
  float q[4][kD];                           // raw float32 query
  float qmu[4];
  uint16_t p[4][4][32];                     // per wave: bf16 P_hat staging [head][token]
  float red[4][4];                          // per wave, per head
  float m[4];
  float lsum[4][4];
  int flag;                                 // invalid page seen
  int ticket;
};

// ------------------------------------------------------------ partials

__device__ __forceinline__ MergeCtx merge_ctx(const DecArgs& A) {
  MergeCtx C;
  C.counters = A.counters;
  C.partials = A.partials;
  C.out = A.L.out;
  C.hq = A.L.hq;
  C.hkv = A.L.hkv;
  C.max_parts = A.L.max_parts;
  return C;
}

__device__ __forceinline__ float* partial_ptr(const DecArgs& A, int bh, int s) {
  return partial_slot(merge_ctx(A), bh, s);
}

// ------------------------------------------------------------ BF16 partition

__device__ void bf16_partition(const DecArgs& A, Smem& sm, int b, int h, int L, int n_full) {
  const DecodeLaunch& P = A.L;
  const int tid = threadIdx.x;
  const int S = P.sink;
  const int nsink = L < S ? L : S;
  const int tail_lo = S > kPage * n_full ? S : kPage * n_full;
  const int ntail = L > tail_lo ? L - tail_lo : 0;
  const int nb = nsink + ntail;                      // <= 112 + 127 < 256
  // raw query
  for (int i = tid; i < 4 * kD; i += 256) {
    const int g = i >> 7, d = i & 127;
    sm.q[g][d] = bf16_lo(P.q[((size_t)b * P.hq + h * kGroup + g) * kD + d]);
  }
  __syncthreads();
  float t[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  const int tok = tid;
  if (tok < nb) {
    const uint16_t* krow;
    if (tok < nsink)
      krow = P.sink_k + (((size_t)b * P.hkv + h) * S + tok) * kD;
    else
      krow = P.tail_k + (((size_t)b * P.hkv + h) * kPage + (tail_lo - kPage * n_full) + (tok - nsink)) * kD;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const uint4* k4 = reinterpret_cast<const uint4*>(krow);
    for (int c = 0; c < 16; ++c) {
      const uint4 w = k4[c];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 8 * c + 2 * i;
        const float k0 = bf16_lo(ww[i]), k1 = bf16_hi(ww[i]);
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[g] = fmaf(sm.q[g][d + 1], k1, fmaf(sm.q[g][d], k0, acc[g]));
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) t[g] = P.softmax_scale * acc[g];
  }
  // max per head
  float mx[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float v = t[g];
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, shfl_xor(v, o));
    mx[g] = v;
  }
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) sm.red[wave][g] = mx[g];
  }
  __syncthreads();
  float m[4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
    m[g] = fmaxf(fmaxf(sm.red[0][g], sm.red[1][g]), fmaxf(sm.red[2][g], sm.red[3][g]));
  // probabilities into LDS [token][head]
  float ls[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float p = (tok < nb && m[g] != kNegInf) ? __expf(t[g] - m[g]) : 0.0f;
    sm.logit[tok * 4 + g] = p;
    float v = p;
    for (int o = 32; o >= 1; o >>= 1) v += shfl_xor(v, o);
    ls[g] = v;
  }
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) sm.lsum[wave][g] = ls[g];
  }
  // o[head][d] = sum_tok p v ; thread = (head, channel pair)
  const int head = tid >> 6, d = (tid & 63) * 2;
  float o0 = 0.f, o1 = 0.f;
  for (int j = 0; j < nb; ++j) {
    const uint16_t* vrow;
    if (j < nsink)
      vrow = P.sink_v + (((size_t)b * P.hkv + h) * S + j) * kD;
    else
      vrow = P.tail_v + (((size_t)b * P.hkv + h) * kPage + (tail_lo - kPage * n_full) + (j - nsink)) * kD;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(vrow + d);
    const float p = sm.logit[j * 4 + head];
    o0 = fmaf(p, bf16_lo(w), o0);
    o1 = fmaf(p, bf16_hi(w), o1);
  }
  __syncthreads();
  float* part = partial_ptr(A, b * P.hkv + h, 0);
  *reinterpret_cast<float2*>(part + head * kD + d) = make_float2(o0, o1);
  if (tid < 4) {
    part[512 + tid] = nb > 0 ? m[tid] : kNegInf;
    part[516 + tid] = sm.lsum[0][tid] + sm.lsum[1][tid] + sm.lsum[2][tid] + sm.lsum[3][tid];
  }
}

// ------------------------------------------------------------ FP4 partition

// Query prologue, run by lanes 0..15 of wave 0 (row g = tid >> 2, quarter q =
// tid & 3): q . mu from the raw query, then the rotated row quantized as Q1
// and the residual as Q2; the dequantized terms (exact in bf16) go to LDS.
template <bool kMx, int kTerms>
__device__ __forceinline__ void query_prologue(const DecodeLaunch& P, Smem& sm, int b, int h, int tid) {
  const int g = tid >> 2, q = tid & 3;
  const uint16_t* qrow = P.q + ((size_t)b * P.hq + h * kGroup + g) * kD;
  const uint4* q4 = reinterpret_cast<const uint4*>(qrow + 32 * q);
  uint4 w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = q4[k];
  float x[32];
  widen32(w, x);
  float dot = 0.0f;
  if (P.key_smoothing) {
    const float* mu = P.key_shift + h * kD + 32 * q;
#pragma unroll
    for (int i = 0; i < 32; ++i) dot = fmaf(x[i], mu[i], dot);
  }
  dot += dpp_f32<kDppQuadXor1>(dot);
  dot += dpp_f32<kDppQuadXor2>(dot);
  if (q == 0) sm.qmu[g] = P.key_smoothing ? dot : 0.0f;
  if (P.rotation) rotate_row_quad(x, q);
#pragma unroll
  for (int term = 0; term < 2; ++term) {
    uint32_t pk[4];
    float deq[32];
    if (term < kTerms) {
      if (kMx) {
        const uint32_t sc = mx_block(x, pk);
        const float sv = pow2_f32((int)sc - 127);
#pragma unroll
        for (int k = 0; k < 4; ++k) deq8(pk[k], sv, deq + 8 * k);
      } else {
        const uint32_t s0 = nv_block<false>(x, pk);
        const uint32_t s1 = nv_block<false>(x + 16, pk + 2);
        deq8(pk[0], e4m3_value(s0), deq);
        deq8(pk[1], e4m3_value(s0), deq + 8);
        deq8(pk[2], e4m3_value(s1), deq + 16);
        deq8(pk[3], e4m3_value(s1), deq + 24);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) deq[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      sm.qhat[term][g][32 * q + i] = (uint16_t)op16<kMx>(deq[i]);   // exact
      x[i] = __fsub_rn(x[i], deq[i]);
    }
  }
}

template <bool kMx, int kTerms, bool kUnder>
__device__ void fp4_partition(const DecArgs& A, Smem& sm, int b, int h, int s, int L, int n_full) {
  const DecodeLaunch& P = A.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p0 = (s - 1) * P.ppp;
  const int p1 = min(n_full, s * P.ppp);
  const int npg = p1 - p0;
  const int lo = max(P.sink, kPage * p0);
  const int sbytes = kMx ? 512 : 1024;
  const size_t hkv = P.hkv;
  const int32_t* bt = P.block_tables + (size_t)b * P.max_pages_per_seq + p0;

  if (tid == 0) sm.flag = 0;

  // ---- prologue: query rows -> rotated, two-term quantized, bf16 staging
  if (tid < 16) query_prologue<kMx, kTerms>(P, sm, b, h, tid);
  __syncthreads();

  // ---- A operands: lane (row = lane & 15, k-group kg = lane >> 4); MFMA c
  // covers d = 32 kg + 8 c + [0, 8)
  const int row = lane & 15, kg = lane >> 4;
  u32x4_t aq[2][4];
#pragma unroll
  for (int term = 0; term < 2; ++term) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row < 4 && term < kTerms) {
        const uint4 t = *reinterpret_cast<const uint4*>(&sm.qhat[term][row][32 * kg + 8 * c]);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
      }
      aq[term][c] = v;
    }
  }
  float qmu[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) qmu[g] = sm.qmu[g];
  const float sigma = P.softmax_scale;

  // ---- pass 1: logits
  float mrun[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  bool bad = false;
  for (int pi = wave; pi < npg; pi += 4) {
    int phys = bt[pi];
    if (phys < 0 || phys >= P.num_pages) { bad = true; phys = 0; }
    const size_t blk = (size_t)phys * hkv + h;
    const uint4* kc = reinterpret_cast<const uint4*>(P.k_codes + blk * 8192) + lane;
    uint4 code[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) code[t] = kc[t * 64];
    uint4 sc4;
    if (kMx) {
      const uint2 t2 = *reinterpret_cast<const uint2*>(P.k_scales + blk * sbytes + lane * 8);
      sc4 = make_uint4(t2.x, t2.y, 0u, 0u);
    } else {
      sc4 = *reinterpret_cast<const uint4*>(P.k_scales + blk * sbytes + lane * 16);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      ElemScale s_lo, s_hi;
      if (kMx) {
        s_lo = s_hi = elem_scale(byte_of(sc4, t), true);
      } else {
        s_lo = elem_scale(byte_of(sc4, 2 * t), false);
        s_hi = elem_scale(byte_of(sc4, 2 * t + 1), false);
      }
      const uint32_t cw[4] = {code[t].x, code[t].y, code[t].z, code[t].w};
      u32x4_t bk[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) bk[c] = deq_word<kMx>(cw[c], c < 2 ? s_lo : s_hi);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int term = 0; term < kTerms; ++term) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = mfma<kMx>(aq[term][c], bk[c], acc);
      }
      if (lane < 16) {
        const int local = pi * kPage + t * 16 + lane;        // token - 128 p0
        const bool live = kPage * p0 + local >= lo;
        float4 lg;
        lg.x = live ? sigma * (acc[0] + qmu[0]) : kNegInf;
        lg.y = live ? sigma * (acc[1] + qmu[1]) : kNegInf;
        lg.z = live ? sigma * (acc[2] + qmu[2]) : kNegInf;
        lg.w = live ? sigma * (acc[3] + qmu[3]) : kNegInf;
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
    for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, shfl_xor(v, o));
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

  // ---- pass 2: P, PV
  const int ph = lane >> 4;          // head of this lane in the P step
  const int pj = lane & 15;          // token pair within the 32-token chunk
  const float mh = m[ph];
  const float cf = (float)P.c;
  const float tau = P.tau;
  float lacc = 0.0f;
  f32x4_t acco[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acco[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15;           // V: 8-channel group (d = 8n .. 8n+7)
  for (int pi = wave; pi < npg; pi += 4) {
    int phys = bt[pi];
    if (phys < 0 || phys >= P.num_pages) phys = 0;
    const size_t blk = (size_t)phys * hkv + h;
    const uint8_t* vcb = P.v_codes + blk * 8192;
    const uint8_t* vsb = P.v_scales + blk * sbytes;
#pragma unroll 1
    for (int ch = 0; ch < 4; ++ch) {
      // V loads for this chunk (issued first)
      const uint4* vc = reinterpret_cast<const uint4*>(vcb + ch * 2048 + lane * 32);
      const uint4 v0 = vc[0], v1 = vc[1];
      const int sidx = kMx ? ((ch * 4 + kg) * 4 + (n >> 2)) * 8 : ((ch * 4 + kg) * 8 + (n >> 1)) * 8;
      const uint2 vs = *reinterpret_cast<const uint2*>(vsb + sidx);
      // probabilities of tokens (2 pj, 2 pj + 1), head ph
      const int local = pi * kPage + ch * 32 + 2 * pj;
      const float t0 = sm.logit[local * 4 + ph];
      const float t1 = sm.logit[(local + 1) * 4 + ph];
      const float e0 = (mh == kNegInf) ? 0.0f : __expf(t0 - mh);
      const float e1 = (mh == kNegInf) ? 0.0f : __expf(t1 - mh);
      lacc += e0 + e1;
      const float q0 = cf * e0, q1 = cf * e1;
      float a = fmaxf(q0, q1);
      a = fmaxf(a, shfl_xor(a, 1));
      a = fmaxf(a, shfl_xor(a, 2));
      a = fmaxf(a, shfl_xor(a, 4));
      const uint32_t scode = e4m3_encode((kUnder && a < tau) ? a * 0.5f : a / 6.0f);
      const float sv = e4m3_value(scode);
      const E2m1Thr T = e2m1_thresholds(sv);
      const float g0 = T.zero ? 0.0f : __fmul_rn(e2m1_grid(e2m1_mag(q0, T)), sv);
      const float g1 = T.zero ? 0.0f : __fmul_rn(e2m1_grid(e2m1_mag(q1, T)), sv);
      const uint32_t pair = op16<kMx>(g0) | (op16<kMx>(g1) << 16);
      *reinterpret_cast<uint32_t*>(&sm.p[wave][ph][2 * pj]) = pair;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): staging visible to the wave
      __builtin_amdgcn_wave_barrier();
      u32x4_t av = {0u, 0u, 0u, 0u};
      if (row < 4) {
        const uint4 t = *reinterpret_cast<const uint4*>(&sm.p[wave][row][8 * kg]);
        av[0] = t.x; av[1] = t.y; av[2] = t.z; av[3] = t.w;
      }
      const u32x4_t ap = av;
      // V operand: token i = 8 kg + ii of the chunk, channels 8n .. 8n+7
      const uint32_t vw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      uint32_t x[8][4];   // x[ii][b] = bf16 pair (channels 8n+2b, 8n+2b+1) of token ii
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        const uint32_t sb = (ii < 4 ? (vs.x >> (8 * ii)) : (vs.y >> (8 * (ii - 4)))) & 0xFFu;
        const ElemScale svv = elem_scale(sb, kMx);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) x[ii][bb] = deq_pair<kMx>(vw[ii], svv, bb);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int bb = j >> 1;
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        u32x4_t bv;
#pragma unroll
        for (int r = 0; r < 4; ++r) bv[r] = __builtin_amdgcn_perm(x[2 * r + 1][bb], x[2 * r][bb], sel);
        acco[j] = mfma<kMx>(ap, bv, acco[j]);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  // l per head: lanes of one head are a 16-lane row
  for (int o = 8; o >= 1; o >>= 1) lacc += shfl_xor(lacc, o);
  if (pj == 0) sm.lsum[wave][ph] = lacc;
  __syncthreads();   // all waves done with logits: reuse it for o
  float* so = sm.logit;   // [wave][head][128]
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4* dst = reinterpret_cast<float4*>(so + (wave * 4 + r) * kD + 8 * lane);
      dst[0] = make_float4(acco[0][r], acco[1][r], acco[2][r], acco[3][r]);
      dst[1] = make_float4(acco[4][r], acco[5][r], acco[6][r], acco[7][r]);
    }
  }
  __syncthreads();
  const int head = tid >> 6, d = (tid & 63) * 2;
  const float invc = 1.0f / cf;    // exact (c is a power of two)
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    o0 += so[(w * 4 + head) * kD + d];
    o1 += so[(w * 4 + head) * kD + d + 1];
  }
  float* part = partial_ptr(A, b * P.hkv + h, s);
  const bool poisoned = sm.flag != 0;
  const float nan = __builtin_nanf("");
  *reinterpret_cast<float2*>(part + head * kD + d) =
      poisoned ? make_float2(nan, nan) : make_float2(o0 * invc, o1 * invc);
  if (tid < 4) {
    part[512 + tid] = poisoned ? 0.0f : m[tid];
    part[516 + tid] = poisoned ? 1.0f : sm.lsum[0][tid] + sm.lsum[1][tid] + sm.lsum[2][tid] + sm.lsum[3][tid];
  }
}

template <bool kMx, int kTerms, bool kUnder>
__global__ void __launch_bounds__(256) decode_kernel(DecArgs A) {
  __shared__ __align__(16) Smem sm;
  const DecodeLaunch& P = A.L;
  const int nps = P.max_parts + 1;
  const int s = blockIdx.x % nps;
  const int bh = blockIdx.x / nps;
  const int b = bh / P.hkv, h = bh - b * P.hkv;
  const int L = P.seq_lens[b];
  const int n_full = L > 0 ? L / kPage : 0;
  if (L < 1 || L > P.max_seq_len || n_full > P.max_pages_per_seq) {
    if (s == 0) poison_rows(P.out, P.hq, b, h);
    return;
  }
  const int nparts = n_full > 0 ? (n_full + P.ppp - 1) / P.ppp : 0;
  if (s > nparts) return;
  if (s == 0)
    bf16_partition(A, sm, b, h, L, n_full);
  else
    fp4_partition<kMx, kTerms, kUnder>(A, sm, b, h, s, L, n_full);
  publish_and_merge(merge_ctx(A), &sm.ticket, b, h, nparts + 1);
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  DecArgs A;
  A.L = L;
  A.counters = static_cast<uint32_t*>(L.workspace);
  A.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(L.workspace) + kCounterBytes);
  const dim3 grid((unsigned)(L.batch * L.hkv * (L.max_parts + 1))), block(256u);
  const bool under = L.p_mode == 4;
#define BDFP4_LAUNCH(MX, T, U) hipLaunchKernelGGL((decode_kernel<MX, T, U>), grid, block, 0, stream, A)
  if (L.mx) {
    if (L.terms == 2) { if (under) BDFP4_LAUNCH(true, 2, true); else BDFP4_LAUNCH(true, 2, false); }
    else { if (under) BDFP4_LAUNCH(true, 1, true); else BDFP4_LAUNCH(true, 1, false); }
  } else {
    if (L.terms == 2) { if (under) BDFP4_LAUNCH(false, 2, true); else BDFP4_LAUNCH(false, 2, false); }
    else { if (under) BDFP4_LAUNCH(false, 1, true); else BDFP4_LAUNCH(false, 1, false); }
  }
#undef BDFP4_LAUNCH
  return hipGetLastError();
}

}  // namespace bdfp4
