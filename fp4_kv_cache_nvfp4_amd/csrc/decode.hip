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
// Grid: one workgroup (256 threads, 4 waves) per 4 FP4 partitions of a
// (sequence, KV head); each wave owns one partition of pages_per_partition
// (1..4) consecutive full pages. The BF16 partition (sink + tail tokens,
// exact float32 attention of the raw query) of (sequence, KV head) j is
// computed by workgroup j, among the first dispatched, while its own first
// K page loads. Every partition computes, for the 4 query heads of its KV
// head, m = max logit, l = sum exp(t - m) and o = sum P_hat v_hat; a
// workgroup merges its four waves in LDS, stores one partial and takes a
// ticket; the last of a (sequence, KV head) merges all of them (merge.hpp).
//
// FP4 partition, per wave:
//  * page ids: lane i reads page i of the partition's block-table run; the
//    wave then issues its first two K page loads;
//  * prologue: wave g rotates (128-point Hadamard, float32) and quantizes
//    query row g as Q1 + Q2 (amax6 per 16 or mxfp4_search per 32), two
//    elements per lane; the dequantized terms are exact in 16 bits and become
//    the A operands of v_mfma_f32_16x16x32_{f16,bf16}: row 2g + t holds term
//    t of head g and rows 8..15 repeat rows 0..7. q . mu (raw float32 query,
//    key means) seeds the term-1 rows of the accumulator.
//  * pass 1 (QK^T): the wave streams its K pages with two pages in flight;
//    per 16-token tile a lane holds 16 code bytes (one coalesced 1 KiB run
//    per wave) and the page's scales come in one 16-byte load per lane. Four
//    MFMAs give both terms of all four heads; their sum, the raw logit
//    q . mu + q_hat . k_hat, goes to the wave's LDS rows [head][token]. Sink
//    tokens fill whole tiles of the first page and get -inf.
//  * the partition maximum of each head (DPP within 16 lanes, then lanes).
//  * pass 2 (softmax, P quantization, PV): per 32-token chunk the 4 x 32
//    values p' = c exp(sigma (t - m)) are formed two per lane; l accumulates
//    them; p' is quantized per aligned 16-token block (amax2_or_amax6 with
//    tau, or amax6) and s * e2m1 (exact in 16 bits) is staged in LDS as the A
//    operand. V codes come as B operands of 8 MFMAs (one per output channel
//    slab).
//  * the 4 waves' (m, l, o) are merged by log-sum-exp in LDS; o and l are
//    divided by c.
//
// E2M1 codes of p' are found without comparing against the grid midpoints:
// with the block scale s = 2^E m (E4M3), the exact float32 quotient p' / m
// (one multiply and two FMA corrections) goes through the hardware
// down-convert, which divides by 2^E and rounds to nearest even; the result
// is the code of the exact ratio p' / s (see quot and e2m1_pair).
//
// Operand construction. The scaled FP4 converts of gfx950 apply only the
// exponent of their float32 scale. MXFP4 scales are powers of two and convert
// exactly to bf16 in one step. For NVFP4 the codes are converted with scale 1
// to f16 and multiplied, two at a time, by their E4M3 scales converted to f16
// by the hardware E4M3 convert; the product has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in f16. The NVFP4 V page stores tokens
// t, t+1 of one channel in a byte, so a converted pair is directly one 32-bit
// word of the PV B operand.
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

constexpr int kMaxPpw = 4;                 // pages per partition = per wave
constexpr int kWaveTok = kMaxPpw * kPage;  // tokens of one partition

constexpr float kNegInf = -__builtin_inff();

struct DecArgs {
  DecodeLaunch L;
};

// ------------------------------------------------------------ converts

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

// E2M1 codes of byte `byte` of w as an f16 pair (grid values, exact).
__device__ __forceinline__ f16x2_t grid_f16_pair(uint32_t w, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  }
}

// Two E4M3 codes (bytes 0,1 or 2,3 of w) as an exact f16 pair.
__device__ __forceinline__ f16x2_t e4m3_pair_f16(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

__device__ __forceinline__ uint32_t u32_of(f16x2_t v) { return __builtin_bit_cast(uint32_t, v); }

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

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) {
  return __shfl_xor(v, m, 64);
}

// ------------------------------------------------------------ shared memory

struct Smem {
  float logit[4][4 * kWaveTok];             // per wave: [head][token] raw logits; then its o [head][128]
  uint16_t qhat[2][4][kD];                  // 16-bit dequantized query terms [term][head][channel]
  float q[4][kD];                           // raw float32 query (BF16 partition)
  uint32_t pst[4][16][16];                  // per wave: P_hat staging [row][token pair]; rows 4..15 stay 0
  float qmu[4];
  float red[4][4];                          // per wave, per head: partition maximum (raw logit)
  float lsum[4][4];                         // per wave, per head: sum of c p
  float rcp[8];                             // RN(1 / (1 + k/8)), k = 0..7
  int bad[4];                               // per wave: its block table names an invalid page
  int tick;
};

// ------------------------------------------------------------ partials

__device__ __forceinline__ MergeCtx merge_ctx(const DecArgs& A) {
  MergeCtx C;
  C.counters = A.L.counters;
  C.partials = A.L.partials;
  C.out = A.L.out;
  C.hq = A.L.hq;
  C.hkv = A.L.hkv;
  C.counter_stride = A.L.counter_stride;
  C.slot_stride = A.L.slot_stride;
  return C;
}


// ------------------------------------------------------------ BF16 partition

// Tokens [0, min(S, L)) from the sink buffer and [max(S, 128 n), L) from the
// tail page: exact float32 attention of the raw query. All of the
// workgroup's loads (K row of token t for thread t, the query, and the V rows
// of its token group for thread (token group, channel quad)) are issued
// before the first barrier, so the partition costs one memory round trip.
__device__ Partial bf16_partition(const DecArgs& A, Smem& sm, int b, int h, int L, int n_full) {
  const DecodeLaunch& P = A.L;
  const int tid = threadIdx.x;
  const int S = P.sink;
  const int nsink = L < S ? L : S;
  const int tail_lo = S > kPage * n_full ? S : kPage * n_full;
  const int ntail = L > tail_lo ? L - tail_lo : 0;
  const int nb = nsink + ntail;                      // <= 112 + 127 < 256
  const size_t bhk = (size_t)b * P.hkv + h;
  const int tail0 = tail_lo - kPage * n_full;
  auto row_of = [&](const uint16_t* sink, const uint16_t* tail, int j) -> const uint16_t* {
    return j < nsink ? sink + (bhk * S + j) * kD : tail + (bhk * kPage + tail0 + (j - nsink)) * kD;
  };
  uint4 kw[16];
  if (tid < nb) {
    const uint4* k4 = reinterpret_cast<const uint4*>(row_of(P.sink_k, P.tail_k, tid));
#pragma unroll
    for (int c = 0; c < 16; ++c) kw[c] = k4[c];
  }
  constexpr int kVPer = 30;                          // ceil(240 / 8) tokens per token group
  const int tg = tid >> 5, cq = tid & 31;            // token group, channel quad
  uint2 vv[kVPer];
#pragma unroll
  for (int k = 0; k < kVPer; ++k) {
    const int j = tg + 8 * k;
    vv[k] = j < nb ? *reinterpret_cast<const uint2*>(row_of(P.sink_v, P.tail_v, j) + 4 * cq) : make_uint2(0u, 0u);
  }
  for (int i = tid; i < 4 * kD; i += 256) {
    const int g = i >> 7, d = i & 127;
    sm.q[g][d] = bf16_lo(P.q[((size_t)b * P.hq + h * kGroup + g) * kD + d]);
  }
  __syncthreads();
  float t[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  if (tid < nb) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint32_t ww[4] = {kw[c].x, kw[c].y, kw[c].z, kw[c].w};
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
  float ls[4];
  float4 pr;
  {
    float pv[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float p = (tid < nb && m[g] != kNegInf) ? __expf(t[g] - m[g]) : 0.0f;
      pv[g] = p;
      float v = p;
      for (int o = 32; o >= 1; o >>= 1) v += shfl_xor(v, o);
      ls[g] = v;
    }
    pr = make_float4(pv[0], pv[1], pv[2], pv[3]);
  }
  float* flat = &sm.logit[0][0];
  reinterpret_cast<float4*>(flat)[tid] = pr;         // p of token tid, [token][head]
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) sm.lsum[wave][g] = ls[g];
  }
  __syncthreads();
  // o[head][4 cq .. +4] over the tokens tg, tg + 8, ... of this thread
  float o[4][4] = {};
#pragma unroll
  for (int k = 0; k < kVPer; ++k) {
    const int j = tg + 8 * k;
    if (j < nb) {
      const float4 p = reinterpret_cast<const float4*>(flat)[j];
      const float v[4] = {bf16_lo(vv[k].x), bf16_hi(vv[k].x), bf16_lo(vv[k].y), bf16_hi(vv[k].y)};
      const float pg[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int c = 0; c < 4; ++c) o[g][c] = fmaf(pg[g], v[c], o[g][c]);
      }
    }
  }
  float* so = flat + 1024;                           // [token group][head][128], past the p values
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<float4*>(so + (tg * 4 + g) * kD + 4 * cq) = make_float4(o[g][0], o[g][1], o[g][2], o[g][3]);
  __syncthreads();
  const int head = tid >> 6, d = (tid & 63) * 2;
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int g8 = 0; g8 < 8; ++g8) {
    o0 += so[(g8 * 4 + head) * kD + d];
    o1 += so[(g8 * 4 + head) * kD + d + 1];
  }
  Partial r;
  r.o0 = o0;
  r.o1 = o1;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    r.m[g] = nb > 0 ? m[g] : kNegInf;
    r.l[g] = (sm.lsum[0][g] + sm.lsum[1][g]) + (sm.lsum[2][g] + sm.lsum[3][g]);
  }
  __syncthreads();                                   // LDS is reused by the caller
  return r;
}

// ------------------------------------------------------------ query prologue

// Butterfly stage across lanes for the two elements a lane holds: the lane
// whose selector bit is clear keeps own + partner, the other partner - own.
__device__ __forceinline__ void xstage(float& x0, float& x1, float p0, float p1, bool upper) {
  x0 = upper ? __fsub_rn(p0, x0) : __fadd_rn(x0, p0);
  x1 = upper ? __fsub_rn(p1, x1) : __fadd_rn(x1, p1);
}

template <int kPattern>
__device__ __forceinline__ float swizzle_f32(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kPattern));
}

// ds_swizzle bit-mode patterns: lane ^ 4, ^ 8, ^ 16 inside 32-lane halves.
constexpr int kSwzXor4 = 0x101F;
constexpr int kSwzXor8 = 0x201F;
constexpr int kSwzXor16 = 0x401F;

// Query row g of the group on a whole wave: lane i holds elements 2i, 2i+1.
// q . mu (raw float32 query, key means), the Hadamard rotation (stage 1
// in-lane, stages 2 .. 64 across lanes), then Q1 and the residual Q2,
// dequantized into LDS as 16-bit MFMA operands. The quantizer is the one of
// the page writer and the row quantizer (quant_block), so the codes are the
// same functions of the rotated values.
template <bool kMx, int kTerms>
__device__ __forceinline__ void query_prologue(const DecodeLaunch& P, uint32_t qw, float2 mu, Smem& sm, int g,
                                               int i) {
  float x0 = bf16_lo(qw), x1 = bf16_hi(qw);
  float dot = __builtin_fmaf(x1, mu.y, __fmul_rn(x0, mu.x));
  dot = sum16(dot);
  dot += shfl_xor(dot, 16);
  dot += shfl_xor(dot, 32);
  if (i == 0) sm.qmu[g] = dot;
  if (P.rotation) {
    const float a = x0, c = x1;
    x0 = __fadd_rn(a, c);
    x1 = __fsub_rn(a, c);
    xstage(x0, x1, dpp_f32<kDppQuadXor1>(x0), dpp_f32<kDppQuadXor1>(x1), (i & 1) != 0);
    xstage(x0, x1, dpp_f32<kDppQuadXor2>(x0), dpp_f32<kDppQuadXor2>(x1), (i & 2) != 0);
    xstage(x0, x1, swizzle_f32<kSwzXor4>(x0), swizzle_f32<kSwzXor4>(x1), (i & 4) != 0);
    xstage(x0, x1, swizzle_f32<kSwzXor8>(x0), swizzle_f32<kSwzXor8>(x1), (i & 8) != 0);
    xstage(x0, x1, swizzle_f32<kSwzXor16>(x0), swizzle_f32<kSwzXor16>(x1), (i & 16) != 0);
    xstage(x0, x1, shfl_xor(x0, 32), shfl_xor(x1, 32), (i & 32) != 0);
    const float cs = inv_sqrt_d();
    x0 = __fmul_rn(x0, cs);
    x1 = __fmul_rn(x1, cs);
  }
#pragma unroll
  for (int term = 0; term < kTerms; ++term) {
    const float xx[2] = {x0, x1};
    float a = __builtin_fmaxf(__builtin_fabsf(x0), __builtin_fabsf(x1));
    float s;
    uint32_t pk;
    if (kMx) {
      // 32-element block = 16 lanes; candidates E_hi, E_hi - 1 by squared error
      a = max16(a);
      int ehi = a > 0.0f ? mx_exponent_hi(a) : -127;
      ehi = ehi < -127 ? -127 : (ehi > 127 ? 127 : ehi);
      const int elo = ehi - 1 < -127 ? -127 : ehi - 1;
      uint32_t phi, plo;
      float ehi_err = quant_block<2, true>(xx, pow2_f32(ehi), &phi);
      float elo_err = quant_block<2, true>(xx, pow2_f32(elo), &plo);
      // levels 2 .. 5 of the 32-element tree: partners lane ^ 1, ^ 2, then
      // the mirrors inside 8 and 16 lanes (the values are uniform per quad /
      // per 8 lanes by then)
      ehi_err = __fadd_rn(ehi_err, dpp_f32<kDppQuadXor1>(ehi_err));
      elo_err = __fadd_rn(elo_err, dpp_f32<kDppQuadXor1>(elo_err));
      ehi_err = __fadd_rn(ehi_err, dpp_f32<kDppQuadXor2>(ehi_err));
      elo_err = __fadd_rn(elo_err, dpp_f32<kDppQuadXor2>(elo_err));
      ehi_err = __fadd_rn(ehi_err, dpp_f32<kDppRowHalfMirror>(ehi_err));
      elo_err = __fadd_rn(elo_err, dpp_f32<kDppRowHalfMirror>(elo_err));
      ehi_err = __fadd_rn(ehi_err, dpp_f32<kDppRowMirror>(ehi_err));
      elo_err = __fadd_rn(elo_err, dpp_f32<kDppRowMirror>(elo_err));
      const bool take_lo = (elo_err < ehi_err) && (elo < ehi) && a > 0.0f;
      s = a > 0.0f ? pow2_f32(take_lo ? elo : ehi) : 0.0f;
      pk = a > 0.0f ? (take_lo ? plo : phi) : 0u;
    } else {
      // 16-element block = 8 lanes
      a = max8(a);
      s = e4m3_value(e4m3_encode(div6(a)));
      quant_block<2, false>(xx, s, &pk);
    }
    float deq[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t nib = (pk >> (4 * k)) & 0xFu;
      const float gv = __fmul_rn(e2m1_grid(nib & 7u), s);
      deq[k] = (nib & 8u) ? -gv : gv;
    }
    reinterpret_cast<uint32_t*>(&sm.qhat[term][g][0])[i] = op16<kMx>(deq[0]) | (op16<kMx>(deq[1]) << 16);
    x0 = __fsub_rn(x0, deq[0]);
    x1 = __fsub_rn(x1, deq[1]);
  }
}

// ------------------------------------------------------------ page loads

// One page of K for one wave: lane l holds the 16 code bytes of tile t at
// t * 1024 + 16 l (token l & 15, channels 32 (l >> 4) .. +32) and the scales
// of its (token, channel group) for all 8 tiles (16 B NVFP4 / 8 B MXFP4).
struct KPage {
  uint4 code[8];
  uint4 sc;
};

// One page of V for one wave: chunk c (32 tokens) of lane l is the 32 bytes at
// c * 2048 + 32 l (tokens 8 (l >> 4) .. +8 of the chunk, channels 8 (l & 15)
// .. +8) and its 8 token scales.
struct VPage {
  uint4 code[8];
  uint2 sc[4];
};

template <bool kMx>
__device__ __forceinline__ void load_k(KPage& k, const DecodeLaunch& P, size_t blk, int lane) {
  const uint4* kc = reinterpret_cast<const uint4*>(P.k_codes + blk * 8192) + lane;
#pragma unroll
  for (int t = 0; t < 8; ++t) k.code[t] = kc[t * 64];
  if (kMx) {
    const uint2 t2 = *reinterpret_cast<const uint2*>(P.k_scales + blk * 512 + lane * 8);
    k.sc = make_uint4(t2.x, t2.y, 0u, 0u);
  } else {
    k.sc = *reinterpret_cast<const uint4*>(P.k_scales + blk * 1024 + lane * 16);
  }
}

template <bool kMx>
__device__ __forceinline__ void load_v(VPage& v, const DecodeLaunch& P, size_t blk, int lane) {
  const uint4* vc = reinterpret_cast<const uint4*>(P.v_codes + blk * 8192 + lane * 32);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v.code[2 * c] = vc[c * 128];
    v.code[2 * c + 1] = vc[c * 128 + 1];
  }
  const int kg = lane >> 4, n = lane & 15;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int sidx = kMx ? ((c * 4 + kg) * 4 + (n >> 2)) * 8 : ((c * 4 + kg) * 8 + (n >> 1)) * 8;
    v.sc[c] = *reinterpret_cast<const uint2*>(P.v_scales + blk * (kMx ? 512 : 1024) + sidx);
  }
}

// ------------------------------------------------------------ FP4 partitions

__device__ __forceinline__ uint32_t umax_dpp8(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor2, 0xF, 0xF, false));
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowHalfMirror, 0xF, 0xF, false));
}

__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// The four FP4 partitions 4 sp + w (w = wave) of one (sequence, KV head):
// each wave streams its own pages_per_partition consecutive pages through
// pass 1, its own maximum and pass 2 with no workgroup barrier in between;
// the four (m, l, o) are then merged by log-sum-exp in LDS and stored as the
// workgroup's partial (returned; the caller stores it).
template <bool kMx, int kTerms, bool kUnder>
__device__ Partial fp4_wg(const DecArgs& A, Smem& sm, int b, int h, int sp, int n_full) {
  const DecodeLaunch& P = A.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p0 = (4 * sp + wave) * P.ppp;                       // first page of this wave's partition
  const int npg = max(0, min(n_full, p0 + P.ppp) - p0);         // its pages, 0 .. pages_per_partition
  const size_t hkv = P.hkv;

  // physical pages of the partition: lane i < npg holds page p0 + i
  int pid = 0;
  if (lane < npg) pid = P.block_tables[(size_t)b * P.max_pages_per_seq + p0 + lane];
  const bool bad_lane = lane < npg && (pid < 0 || pid >= P.num_pages);
  const bool bad = __ballot(bad_lane) != 0;
  if (bad_lane) pid = 0;                                        // keep addresses inside the cache
  auto blk_of = [&](int pi) -> size_t { return (size_t)__builtin_amdgcn_readlane(pid, pi) * hkv + h; };

  // the query row of this wave and the key means
  const uint32_t qw =
      reinterpret_cast<const uint32_t*>(P.q + ((size_t)b * P.hq + h * kGroup + wave) * kD)[lane];
  const float2 mu = P.key_smoothing ? reinterpret_cast<const float2*>(P.key_shift + h * kD)[lane]
                                    : make_float2(0.0f, 0.0f);
  if (tid < 8) sm.rcp[tid] = rcp_significand((uint32_t)tid);
  {
    uint32_t* pz = &sm.pst[0][0][0];       // rows 4 .. 15 of every wave's staging tile
    for (int i = tid; i < 4 * 192; i += 256) pz[(i / 192) * 256 + 64 + (i % 192)] = 0u;
  }
  // The wave reads a stream of eight slots, K pages 0..3 then V pages 0..3
  // (slots of pages >= npg are empty), keeping the next two slots in flight
  // while one is used. K page i lands in kb[i % 3], V page j in vb[j % 3];
  // every load has a fixed destination, so at most four buffers are live.
  // The loads are unconditional (a slot past npg reads physical page 0,
  // which always exists, and is never used) so the compiler can count the
  // loads in flight exactly and wait only for the slot about to be used.
  KPage kb0, kb1, kb2;
  VPage vb0, vb1, vb2;
  load_k<kMx>(kb0, P, blk_of(0), lane);
  load_k<kMx>(kb1, P, blk_of(1), lane);
  query_prologue<kMx, kTerms>(P, qw, mu, sm, wave, lane);
  __syncthreads();

  // A operands: lane (row = lane & 15, k-group kg = lane >> 4); row 2 g + t
  // holds query term t of head g, and rows 8 .. 15 repeat rows 0 .. 7, so
  // lanes 32 .. 63 of the result hold exactly what lanes 0 .. 31 hold and
  // every lane can store its logits without a branch; MFMA c covers channels
  // 32 kg + 8 c + [0, 8)
  const int row = lane & 15, kg = lane >> 4;
  const int qr = row & 7;
  u32x4_t aq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if ((qr & 1) < kTerms) {
      const uint4 t = *reinterpret_cast<const uint4*>(&sm.qhat[qr & 1][qr >> 1][32 * kg + 8 * c]);
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
    aq[c] = v;
  }
  // D lane l holds rows 4 (l >> 4) + i: lanes 0..15 (and 32..47) heads 0, 1,
  // lanes 16..31 (and 48..63) heads 2, 3; term 1 in i = 0, 2, term 2 in
  // i = 1, 3. q . mu enters through the term-1 rows.
  const int hp = kg & 1;                                        // head pair of this lane's result
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f};
  acc0[0] = sm.qmu[2 * hp];
  acc0[2] = sm.qmu[2 * hp + 1];
  float* lgw = &sm.logit[wave][0];                              // this wave's [head][token]
  float* lg_a = lgw + (2 * hp) * kWaveTok + row;                // head 2 hp
  float* lg_b = lg_a + kWaveTok;                                // head 2 hp + 1

  // ---- pass 1: raw logits q . mu + q_hat . k_hat
  // Sink tokens (global tokens below the sink size, a multiple of 16) fill
  // whole 16-token tiles of the sequence's first page; those tiles get -inf.
  const int sink_tiles = p0 == 0 ? P.sink / 16 : 0;
  float ma = kNegInf, mb = kNegInf;
  auto k_page = [&](const KPage& cur, int pi) {
    const int skip = pi == 0 ? sink_tiles : 0;                  // uniform
    float pa = kNegInf, pb = kNegInf;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int local = pi * kPage + t * 16;                    // first token of the tile - 128 p0
      u32x4_t bk[4];
      if (kMx) {
        const uint32_t sb = (word_of(cur.sc, t >> 2) >> (8 * (t & 3))) & 0xFFu;
        const float sv = __uint_as_float(sb << 23);             // E8M0: only the exponent field is used
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t cw = word_of(cur.code[t], c);
          bk[c] = (u32x4_t){cvt_bf16_pair(cw, sv, 0), cvt_bf16_pair(cw, sv, 1), cvt_bf16_pair(cw, sv, 2),
                            cvt_bf16_pair(cw, sv, 3)};
        }
      } else {
        const f16x2_t sp2 = e4m3_pair_f16(word_of(cur.sc, t >> 1), (t & 1) != 0);   // (s_lo, s_hi)
        const f16x2_t slo = {sp2[0], sp2[0]}, shi = {sp2[1], sp2[1]};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t cw = word_of(cur.code[t], c);
          const f16x2_t sc = c < 2 ? slo : shi;
          bk[c] = (u32x4_t){u32_of(grid_f16_pair(cw, 0) * sc), u32_of(grid_f16_pair(cw, 1) * sc),
                            u32_of(grid_f16_pair(cw, 2) * sc), u32_of(grid_f16_pair(cw, 3) * sc)};
        }
      }
      f32x4_t acc = acc0;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma<kMx>(aq[c], bk[c], acc);
      const bool sink = t < skip;                               // uniform: a sink tile of page 0
      const float ta = sink ? kNegInf : __fadd_rn(acc[0], acc[1]);
      const float tb = sink ? kNegInf : __fadd_rn(acc[2], acc[3]);
      lg_a[local] = ta;
      lg_b[local] = tb;
      pa = __builtin_fmaxf(pa, ta);
      pb = __builtin_fmaxf(pb, tb);
    }
    ma = __builtin_fmaxf(ma, pa);
    mb = __builtin_fmaxf(mb, pb);
  };
  static_assert(kMaxPpw == 4, "the stream below is unrolled for up to 4 pages");
  load_k<kMx>(kb2, P, blk_of(2), lane);
  if (npg > 0) k_page(kb0, 0);
  load_k<kMx>(kb0, P, blk_of(3), lane);
  if (npg > 1) k_page(kb1, 1);
  load_v<kMx>(vb0, P, blk_of(0), lane);
  if (npg > 2) k_page(kb2, 2);
  load_v<kMx>(vb1, P, blk_of(1), lane);
  if (npg > 3) k_page(kb0, 3);
  // the partition maximum of each head (rows of 16 lanes hold heads 2 hp, 2 hp + 1)
  ma = max16(ma);
  mb = max16(mb);
  const float m4[4] = {readlane_f32(ma, 0), readlane_f32(mb, 0), readlane_f32(ma, 16), readlane_f32(mb, 16)};

  // ---- pass 2: P, PV
  const int ph = lane >> 4;          // head of this lane in the P step
  const int pj = lane & 15;          // token pair within the 32-token chunk
  const float mh = ph == 0 ? m4[0] : (ph == 1 ? m4[1] : (ph == 2 ? m4[2] : m4[3]));
  const float ks = __fmul_rn(P.softmax_scale, 1.44269504088896341f);   // sigma log2(e)
  const float cf = (float)P.c;
  const float tau = P.tau;
  const float* lrow = lgw + ph * kWaveTok + 2 * pj;
  uint32_t* pst_w = &sm.pst[wave][ph][pj];
  const u32x4_t* pst_r = reinterpret_cast<const u32x4_t*>(&sm.pst[wave][row][4 * kg]);
  float lacc = 0.0f;                 // sum of c p over this lane's tokens
  f32x4_t acco[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acco[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  auto v_page = [&](const VPage& vcur, int pi) {
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      // p' = c exp(sigma (t - m)) of tokens 2 pj, 2 pj + 1 of the chunk, head ph
      const float2 tt = *reinterpret_cast<const float2*>(lrow + pi * kPage + ch * 32);
      const float x0 = __fmul_rn(cf, __builtin_amdgcn_exp2f(__fmul_rn(__fsub_rn(tt.x, mh), ks)));
      const float x1 = __fmul_rn(cf, __builtin_amdgcn_exp2f(__fmul_rn(__fsub_rn(tt.y, mh), ks)));
      lacc = __fadd_rn(lacc, __fadd_rn(x0, x1));
      // block maximum over the aligned 16 tokens (8 lanes); p' >= 0, so the
      // unsigned order of the bit patterns is the float order
      const float a = __uint_as_float(umax_dpp8(max(__float_as_uint(x0), __float_as_uint(x1))));
      const uint32_t sc = p_scale_code<kUnder>(a, tau);
      const float sv = e4m3_value(sc);
      const uint32_t byte =
          sv > 0.0f ? e2m1_pair(x0, x1, sv, significand(sv), sm.rcp[sig_index(sv)]) : 0u;
      uint32_t word;
      if (kMx) {
        const auto g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, 1.0f, 0);
        word = __builtin_amdgcn_perm(__float_as_uint(__fmul_rn(g[1], sv)), __float_as_uint(__fmul_rn(g[0], sv)),
                                     0x07060302u);
      } else {
        const f16x2_t s16 = e4m3_pair_f16(sc * 0x0101u, false);
        word = u32_of(grid_f16_pair(byte, 0) * s16);
      }
      *pst_w = word;
      const u32x4_t ap = *pst_r;     // LDS instructions of one wave complete in order
      const uint4 v0 = vcur.code[2 * ch], v1 = vcur.code[2 * ch + 1];
      const uint2 vs = vcur.sc[ch];
      const uint32_t vw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      if (kMx) {
        // element pairs per byte: vw[ii] = token 8 kg + ii, channels 8n .. 8n+7;
        // byte bb of every token gives channels 8n + 2bb, +1 (MFMAs j = 2bb, 2bb+1)
        float svv[8];
#pragma unroll
        for (int ii = 0; ii < 8; ++ii)
          svv[ii] = __uint_as_float(((ii < 4 ? (vs.x >> (8 * ii)) : (vs.y >> (8 * (ii - 4)))) & 0xFFu) << 23);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          uint32_t x[8];
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) x[ii] = cvt_bf16_pair(vw[ii], svv[ii], bb);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const uint32_t sel = jj ? 0x07060302u : 0x05040100u;
            u32x4_t bv;
#pragma unroll
            for (int r = 0; r < 4; ++r) bv[r] = __builtin_amdgcn_perm(x[2 * r + 1], x[2 * r], sel);
            acco[2 * bb + jj] = mfma<kMx>(ap, bv, acco[2 * bb + jj]);
          }
        }
      } else {
        // token pairs per byte: byte r of vw[j] = tokens 8 kg + 2r, +1 at channel 8n + j
        const f16x2_t spv[4] = {e4m3_pair_f16(vs.x, false), e4m3_pair_f16(vs.x, true),
                                e4m3_pair_f16(vs.y, false), e4m3_pair_f16(vs.y, true)};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          u32x4_t bv;
#pragma unroll
          for (int r = 0; r < 4; ++r) bv[r] = u32_of(grid_f16_pair(vw[j], r) * spv[r]);
          acco[j] = mfma<kMx>(ap, bv, acco[j]);
        }
      }
    }
  };
  load_v<kMx>(vb2, P, blk_of(2), lane);
  if (npg > 0) v_page(vb0, 0);
  load_v<kMx>(vb0, P, blk_of(3), lane);
  if (npg > 1) v_page(vb1, 1);
  if (npg > 2) v_page(vb2, 2);
  if (npg > 3) v_page(vb0, 3);
  // ---- this wave's (m, l, o) to LDS: o over its own logit rows (read above
  // by this wave only; its LDS instructions complete in order)
  lacc = sum16(lacc);                // rows of 16 lanes = heads
  float* so = lgw;                   // [head][128]
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4* dst = reinterpret_cast<float4*>(so + r * kD + 8 * lane);
      dst[0] = make_float4(acco[0][r], acco[1][r], acco[2][r], acco[3][r]);
      dst[1] = make_float4(acco[4][r], acco[5][r], acco[6][r], acco[7][r]);
    }
  }
  // cross-lane reads in uniform control flow: a lane's value is only
  // guaranteed to live on while that lane itself still uses it
  const float l4[4] = {readlane_f32(lacc, 0), readlane_f32(lacc, 16), readlane_f32(lacc, 32),
                       readlane_f32(lacc, 48)};
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      sm.red[wave][g] = m4[g];
      sm.lsum[wave][g] = l4[g];
    }
    sm.bad[wave] = bad ? 1 : 0;
  }
  __syncthreads();
  // ---- log-sum-exp merge of the four partitions: thread (head, channel pair)
  const float sigma = P.softmax_scale;
  const float invc = 1.0f / cf;      // exact (c is a power of two)
  float mm[4], ll[4], wgt[4][4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float M = fmaxf(fmaxf(sm.red[0][g], sm.red[1][g]), fmaxf(sm.red[2][g], sm.red[3][g]));
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm.red[w][g];
      wgt[g][w] = mw == kNegInf ? 0.0f : __expf(sigma * (mw - M));
      l = fmaf(wgt[g][w], sm.lsum[w][g], l);
    }
    mm[g] = sigma * M;
    ll[g] = l * invc;
  }
  const int head = tid >> 6, d = (tid & 63) * 2;
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float wh = head == 0 ? wgt[0][w] : (head == 1 ? wgt[1][w] : (head == 2 ? wgt[2][w] : wgt[3][w]));
    const float* ow = &sm.logit[w][head * kD + d];
    o0 = fmaf(wh, ow[0], o0);
    o1 = fmaf(wh, ow[1], o1);
  }
  const bool poisoned = (sm.bad[0] | sm.bad[1] | sm.bad[2] | sm.bad[3]) != 0;
  const float nan = __builtin_nanf("");
  Partial r;
  r.o0 = poisoned ? nan : o0 * invc;
  r.o1 = poisoned ? nan : o1 * invc;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    r.m[g] = poisoned ? 0.0f : mm[g];
    r.l[g] = poisoned ? 1.0f : ll[g];
  }
  return r;
}

// Workgroup j is FP4 workgroup j % G of (sequence, KV head) j / G, G per
// (sequence, KV head). The BF16 partition of (sequence, KV head) j is
// computed by workgroup j of the grid after its FP4 partition: the first
// workgroups are dispatched first and, being the oldest on their CUs, finish
// first, so the extra work lands where there is slack. Slots: FP4 workgroup
// sp -> sp, the BF16 partition -> the FP4 workgroup count of its sequence.
// Each partition takes its (sequence, KV head)'s ticket once its partial is
// stored; the last one merges all nwg + 1 partials.
template <bool kMx, int kTerms, bool kUnder>
__global__ void __launch_bounds__(256) decode_kernel(DecArgs A) {
  __shared__ __align__(16) Smem sm;
  const DecodeLaunch& P = A.L;
  const MergeCtx C = merge_ctx(A);
  auto fp4_count = [&](int L) {
    const int n_full = L / kPage;
    return n_full > 0 ? fp4_wgs((n_full + P.ppp - 1) / P.ppp) : 0;
  };
  auto valid = [&](int L) { return L >= 1 && L <= P.max_seq_len && L / kPage <= P.max_pages_per_seq; };
  // FP4 role
  const int G = fp4_wgs(P.max_parts);
  const int bh = (int)blockIdx.x / G, sp = (int)blockIdx.x - bh * G;
  const int b = bh / P.hkv, h = bh - b * P.hkv;
  const int L = P.seq_lens[b];
  const int nwg = valid(L) ? fp4_count(L) : 0;
  if (sp < nwg) {
    const Partial mine = fp4_wg<kMx, kTerms, kUnder>(A, sm, b, h, sp, L / kPage);
    write_partial(partial_writer(C, bh, sp), mine);
    uint32_t* ticket = C.counters + (size_t)bh * C.counter_stride;
    if (take_ticket(ticket, 1, &sm.tick) == nwg) {
      merge_out(C, b, h, nwg + 1, sp, true, mine);
      reset_ticket(ticket);
    }
  }
  // BF16 role
  const int bh2 = (int)blockIdx.x;
  if (bh2 < P.batch * P.hkv) {
    const int b2 = bh2 / P.hkv, h2 = bh2 - b2 * P.hkv;
    const int L2 = P.seq_lens[b2];
    if (!valid(L2)) {
      poison_rows(P.out, P.hq, b2, h2);
      return;
    }
    const int nwg2 = fp4_count(L2);
    const Partial r = bf16_partition(A, sm, b2, h2, L2, L2 / kPage);
    write_partial(partial_writer(C, bh2, nwg2), r);
    uint32_t* ticket = C.counters + (size_t)bh2 * C.counter_stride;
    if (take_ticket(ticket, 1, &sm.tick) == nwg2) {
      merge_out(C, b2, h2, nwg2 + 1, nwg2, true, r);
      reset_ticket(ticket);
    }
  }
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  DecArgs A;
  A.L = L;
  const dim3 grid((unsigned)(L.batch * L.hkv * fp4_wgs(L.max_parts))), block(256u);
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
