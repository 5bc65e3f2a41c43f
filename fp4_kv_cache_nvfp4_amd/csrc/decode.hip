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
// Grid: one workgroup (256 threads, 4 waves) per (sequence, KV head, FP4
// partition); each FP4 partition owns pages_per_partition pages. The BF16
// partition (sink + tail tokens, exact float32 attention of the raw query)
// is computed by the first workgroup of each (sequence, KV head) after its
// FP4 pages, so the grid has no extra short workgroups that would spill
// the 2-per-CU residency into a second round. A partition computes, for the
// 4 query heads of its KV head, m = max logit, l = sum exp(t - m) and
// o = sum P_hat v_hat, writes them to the workspace and takes a ticket; the
// last workgroup of the (sequence, KV head) merges all partials and resets
// the ticket.
//
// FP4 partition, per workgroup:
//  * the page ids are staged in LDS and each wave starts loading its first K
//    page before the query prologue;
//  * prologue: wave g rotates (128-point Hadamard, float32) and quantizes
//    query row g as Q1 + Q2 (amax6 per 16 or mxfp4_search per 32), two
//    elements per lane; the dequantized terms are exact in 16 bits and become
//    the A operands of v_mfma_f32_16x16x32_{f16,bf16}: row 2g + t holds term
//    t of head g, rows 8..15 are zero. q . mu (raw float32 query, key means)
//    seeds the term-1 rows of the accumulator.
//  * pass 1 (QK^T): each wave streams whole pages, the next page in flight
//    while the current one is used; per 16-token tile a lane holds 16 code
//    bytes (one coalesced 1 KiB run per wave) and the page's scales come in
//    one 16-byte load per lane. Four MFMAs give both terms of all four heads;
//    their sum, the raw logit q . mu + q_hat . k_hat, goes to LDS
//    [head][token]. Sink tokens fill whole tiles of the first page and get
//    -inf.
//  * partition max over the 4 waves.
//  * pass 2 (softmax, P quantization, PV): per 32-token chunk the 4 x 32
//    values p' = c exp(sigma (t - m)) are formed two per lane; l accumulates
//    them; p' is quantized per aligned 16-token block (amax2_or_amax6 with
//    tau, or amax6) and s * e2m1 (exact in 16 bits) is staged in LDS as the A
//    operand. V codes come as B operands of 8 MFMAs (one per output channel
//    slab).
//  * the 4 waves' o and l are summed in LDS; both are divided by c.
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

constexpr int kMaxPpp = 16;
constexpr int kMaxTok = kMaxPpp * kPage;   // tokens of one partition
constexpr float kNegInf = -__builtin_inff();

struct DecArgs {
  DecodeLaunch L;
  uint32_t* counters;
  float* partials;
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
  float logit[4 * kMaxTok];                 // [head][token] raw logits; reused for the o reduction
  uint16_t qhat[2][4][kD];                  // 16-bit dequantized query terms [term][head][channel]
  float q[4][kD];                           // raw float32 query (BF16 partition)
  uint32_t pst[4][16][16];                  // per wave: P_hat staging [row][token pair]; rows 4..15 stay 0
  float qmu[4];
  float red[4][4];                          // per wave, per head
  float lsum[4][4];
  float rcp[8];                             // RN(1 / (1 + k/8)), k = 0..7
  int page[kMaxPpp];                        // physical pages of the partition (-1: invalid)
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

// Tokens [0, min(S, L)) from the sink buffer and [max(S, 128 n), L) from the
// tail page: exact float32 attention of the raw query, thread = token for the
// logits, thread = (head, channel pair) for o.
__device__ void bf16_partition(const DecArgs& A, Smem& sm, int b, int h, int L, int n_full) {
  const DecodeLaunch& P = A.L;
  const int tid = threadIdx.x;
  const int S = P.sink;
  const int nsink = L < S ? L : S;
  const int tail_lo = S > kPage * n_full ? S : kPage * n_full;
  const int ntail = L > tail_lo ? L - tail_lo : 0;
  const int nb = nsink + ntail;                      // <= 112 + 127 < 256
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
    uint4 kw[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) kw[c] = k4[c];      // the whole row in flight at once
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint4 w = kw[c];
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
  const int head = tid >> 6, d = (tid & 63) * 2;
  float o0 = 0.f, o1 = 0.f;
#pragma unroll 16
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
  pstore2(part + head * kD + d, o0, o1);
  if (tid < 4) {
    pstore(part + 512 + tid, nb > 0 ? m[tid] : kNegInf);
    pstore(part + 516 + tid, sm.lsum[0][tid] + sm.lsum[1][tid] + sm.lsum[2][tid] + sm.lsum[3][tid]);
  }
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

// ------------------------------------------------------------ FP4 partition

__device__ __forceinline__ uint32_t umax_dpp8(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor2, 0xF, 0xF, false));
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowHalfMirror, 0xF, 0xF, false));
}

template <bool kMx, int kTerms, bool kUnder>
__device__ void fp4_partition(const DecArgs& A, Smem& sm, int b, int h, int s, int L, int n_full) {
  const DecodeLaunch& P = A.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p0 = (s - 1) * P.ppp;
  const int p1 = min(n_full, s * P.ppp);
  const int npg = p1 - p0;
  const size_t hkv = P.hkv;

  // the query row of this wave and the key means, first so their latency
  // overlaps the page-id staging and the first page loads
  const uint32_t qw =
      reinterpret_cast<const uint32_t*>(P.q + ((size_t)b * P.hq + h * kGroup + wave) * kD)[lane];
  const float2 mu = P.key_smoothing ? reinterpret_cast<const float2*>(P.key_shift + h * kD)[lane]
                                    : make_float2(0.0f, 0.0f);
  if (tid < npg) {
    const int ph = P.block_tables[(size_t)b * P.max_pages_per_seq + p0 + tid];
    sm.page[tid] = (ph < 0 || ph >= P.num_pages) ? -1 : ph;
  }
  if (tid < 8) sm.rcp[tid] = rcp_significand((uint32_t)tid);
  {
    uint32_t* pz = &sm.pst[0][0][0];       // rows 4 .. 15 of every wave's staging tile
    for (int i = tid; i < 4 * 192; i += 256) pz[(i / 192) * 256 + 64 + (i % 192)] = 0u;
  }
  __syncthreads();
  auto blk_of = [&](int pi) -> size_t {
    const int ph = sm.page[pi];
    return (size_t)(ph < 0 ? 0 : ph) * hkv + h;
  };

  KPage kcur;
  if (wave < npg) load_k<kMx>(kcur, P, blk_of(wave), lane);
  query_prologue<kMx, kTerms>(P, qw, mu, sm, wave, lane);
  __syncthreads();

  // A operands: lane (row = lane & 15, k-group kg = lane >> 4); row 2 g + t
  // holds query term t of head g (rows 8 .. 15 zero); MFMA c covers channels
  // 32 kg + 8 c + [0, 8)
  const int row = lane & 15, kg = lane >> 4;
  u32x4_t aq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (row < 2 * kGroup && ((row & 1) < kTerms)) {
      const uint4 t = *reinterpret_cast<const uint4*>(&sm.qhat[row & 1][row >> 1][32 * kg + 8 * c]);
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
    aq[c] = v;
  }
  // D lane l holds rows 4 (l >> 4) + i: lanes 0..15 heads 0, 1 and lanes
  // 16..31 heads 2, 3 (term 1 in i = 0, 2; term 2 in i = 1, 3); q . mu
  // enters through the term-1 rows
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f};
  if (kg < 2) {
    acc0[0] = sm.qmu[2 * kg];
    acc0[2] = sm.qmu[2 * kg + 1];
  }
  float* lg_a = sm.logit + (2 * (kg & 1)) * kMaxTok + row;   // head 2 kg (lanes < 32)
  float* lg_b = lg_a + kMaxTok;                                // head 2 kg + 1

  // ---- pass 1: raw logits q . mu + q_hat . k_hat
  // Sink tokens (global tokens below the sink size, a multiple of 16) fill
  // whole 16-token tiles of the sequence's first page; those tiles get -inf.
  const int sink_tiles = p0 == 0 ? P.sink / 16 : 0;
  float ma = kNegInf, mb = kNegInf;
  auto k_page = [&](const KPage& cur, KPage& nxt, int pi) {
    if (pi + 4 < npg) load_k<kMx>(nxt, P, blk_of(pi + 4), lane);
    const int skip = pi == 0 ? sink_tiles : 0;             // uniform
    float pa = kNegInf, pb = kNegInf;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int local = pi * kPage + t * 16;               // token - 128 p0 of the tile's first token
      if (t < skip) {
        if (lane < 32) {
          lg_a[local] = kNegInf;
          lg_b[local] = kNegInf;
        }
        continue;
      }
      u32x4_t bk[4];
      if (kMx) {
        const uint32_t sb = (word_of(cur.sc, t >> 2) >> (8 * (t & 3))) & 0xFFu;
        const float sv = pow2_f32((int)sb - 127);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t cw = word_of(cur.code[t], c);
          bk[c] = (u32x4_t){cvt_bf16_pair(cw, sv, 0), cvt_bf16_pair(cw, sv, 1), cvt_bf16_pair(cw, sv, 2),
                            cvt_bf16_pair(cw, sv, 3)};
        }
      } else {
        const f16x2_t sp = e4m3_pair_f16(word_of(cur.sc, t >> 1), (t & 1) != 0);   // (s_lo, s_hi)
        const f16x2_t slo = {sp[0], sp[0]}, shi = {sp[1], sp[1]};
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
      const float ta = __fadd_rn(acc[0], acc[1]);
      const float tb = __fadd_rn(acc[2], acc[3]);
      if (lane < 32) {
        lg_a[local] = ta;
        lg_b[local] = tb;
      }
      pa = __builtin_fmaxf(pa, ta);
      pb = __builtin_fmaxf(pb, tb);
    }
    ma = __builtin_fmaxf(ma, pa);
    mb = __builtin_fmaxf(mb, pb);
  };
  {
    KPage kb;
    for (int pi = wave; pi < npg; pi += 8) {
      k_page(kcur, kb, pi);
      if (pi + 4 >= npg) break;
      k_page(kb, kcur, pi + 4);
    }
  }
  VPage vcur;
  if (wave < npg) load_v<kMx>(vcur, P, blk_of(wave), lane);
  ma = max16(ma);
  mb = max16(mb);
  if (lane == 0 || lane == 16) {
    sm.red[wave][2 * kg] = ma;
    sm.red[wave][2 * kg + 1] = mb;
  }
  __syncthreads();
  float m[4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
    m[g] = fmaxf(fmaxf(sm.red[0][g], sm.red[1][g]), fmaxf(sm.red[2][g], sm.red[3][g]));

  // ---- pass 2: P, PV
  const int ph = lane >> 4;          // head of this lane in the P step
  const int pj = lane & 15;          // token pair within the 32-token chunk
  const float mh = ph == 0 ? m[0] : (ph == 1 ? m[1] : (ph == 2 ? m[2] : m[3]));
  const float ks = __fmul_rn(P.softmax_scale, 1.44269504088896341f);   // sigma log2(e)
  const float cf = (float)P.c;
  const float tau = P.tau;
  const float* lrow = sm.logit + ph * kMaxTok + 2 * pj;
  uint32_t* pst_w = &sm.pst[wave][ph][pj];
  const u32x4_t* pst_r = reinterpret_cast<const u32x4_t*>(&sm.pst[wave][row][4 * kg]);
  float lacc = 0.0f;                 // sum of c p over this lane's tokens
  f32x4_t acco[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acco[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  auto v_page = [&](const VPage& vcur, VPage& vnxt, int pi) {
    if (pi + 4 < npg) load_v<kMx>(vnxt, P, blk_of(pi + 4), lane);
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
        // element pairs per byte: vw[ii] = token 8 kg + ii, channels 8n .. 8n+7
        uint32_t x[8][4];
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const uint32_t sb = (ii < 4 ? (vs.x >> (8 * ii)) : (vs.y >> (8 * (ii - 4)))) & 0xFFu;
          const float svv = pow2_f32((int)sb - 127);
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) x[ii][bb] = cvt_bf16_pair(vw[ii], svv, bb);
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
      } else {
        // token pairs per byte: byte r of vw[j] = tokens 8 kg + 2r, +1 at channel 8n + j
        const f16x2_t sp[4] = {e4m3_pair_f16(vs.x, false), e4m3_pair_f16(vs.x, true),
                               e4m3_pair_f16(vs.y, false), e4m3_pair_f16(vs.y, true)};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          u32x4_t bv;
#pragma unroll
          for (int r = 0; r < 4; ++r) bv[r] = u32_of(grid_f16_pair(vw[j], r) * sp[r]);
          acco[j] = mfma<kMx>(ap, bv, acco[j]);
        }
      }
    }
  };
  {
    VPage vb;
    for (int pi = wave; pi < npg; pi += 8) {
      v_page(vcur, vb, pi);
      if (pi + 4 >= npg) break;
      v_page(vb, vcur, pi + 4);
    }
  }
  lacc = sum16(lacc);                // lanes of one head are a 16-lane row
  if (pj == 0) sm.lsum[wave][ph] = lacc;
  __syncthreads();                   // all waves done with the logits: reuse for o
  float* so = sm.logit;              // [wave][head][128]
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
  const float invc = 1.0f / cf;      // exact (c is a power of two)
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    o0 += so[(w * 4 + head) * kD + d];
    o1 += so[(w * 4 + head) * kD + d + 1];
  }
  bool poisoned = false;
  for (int i = 0; i < npg; ++i) poisoned |= sm.page[i] < 0;
  float* part = partial_ptr(A, b * P.hkv + h, s);
  const float nan = __builtin_nanf("");
  pstore2(part + head * kD + d, poisoned ? nan : o0 * invc, poisoned ? nan : o1 * invc);
  if (tid < 4) {
    const float l = (sm.lsum[0][tid] + sm.lsum[1][tid]) + (sm.lsum[2][tid] + sm.lsum[3][tid]);
    pstore(part + 512 + tid, poisoned ? 0.0f : m[tid] * P.softmax_scale);
    pstore(part + 516 + tid, poisoned ? 1.0f : l * invc);
  }
}

template <bool kMx, int kTerms, bool kUnder>
__global__ void __launch_bounds__(256) decode_kernel(DecArgs A) {
  __shared__ __align__(16) Smem sm;
  const DecodeLaunch& P = A.L;
  const int G = P.max_parts > 0 ? P.max_parts : 1;     // workgroups per (sequence, KV head)
  const int sp = blockIdx.x % G;
  const int bh = blockIdx.x / G;
  const int b = bh / P.hkv, h = bh - b * P.hkv;
  const int L = P.seq_lens[b];
  const int n_full = L > 0 ? L / kPage : 0;
  if (L < 1 || L > P.max_seq_len || n_full > P.max_pages_per_seq) {
    if (sp == 0) poison_rows(P.out, P.hq, b, h);
    return;
  }
  const int nparts = n_full > 0 ? (n_full + P.ppp - 1) / P.ppp : 0;
  const int s = sp + 1;                                 // FP4 partition of this workgroup
  if (s > nparts && sp != 0) return;
  int inc = 0;
  if (s <= nparts) {
    fp4_partition<kMx, kTerms, kUnder>(A, sm, b, h, s, L, n_full);
    ++inc;
  }
  if (sp == 0) {
    // the BF16 partition (slot 0) rides on the first workgroup, after its
    // FP4 pages, so the grid is exactly one workgroup per FP4 partition
    if (inc) __syncthreads();
    bf16_partition(A, sm, b, h, L, n_full);
    ++inc;
  }
  publish_and_merge(merge_ctx(A), &sm.ticket, &sm.red[0][0], sm.logit, 4 * kMaxTok, b, h, nparts + 1, inc);
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  DecArgs A;
  A.L = L;
  A.counters = static_cast<uint32_t*>(L.workspace);
  A.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(L.workspace) + kCounterBytes);
  const dim3 grid((unsigned)(L.batch * L.hkv * (L.max_parts > 0 ? L.max_parts : 1))), block(256u);
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
