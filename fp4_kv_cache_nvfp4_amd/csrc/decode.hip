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
//  * the page ids are staged in LDS and each wave starts loading its first K
//    page before the query prologue;
//  * prologue: wave g rotates (128-point Hadamard, float32) and quantizes
//    query row g as Q1 + Q2 (amax6 per 16 or mxfp4_search per 32), 16 lanes
//    of 8 elements; the dequantized terms are exact in 16 bits and become the
//    A operands of v_mfma_f32_16x16x32_{f16,bf16} (rows 0..3 = heads, 12 zero
//    rows). q . mu (raw float32 query, key means) seeds the accumulator.
//  * pass 1 (QK^T): each wave streams whole pages, the next page in flight
//    while the current one is used; per 16-token tile a lane holds 16 code
//    bytes (one coalesced 1 KiB run per wave) and the page's scales come in
//    one 16-byte load per lane. Logits sigma (q . mu + q_hat . k_hat) go to
//    LDS [head][token]; sink slots of the first page get -inf.
//  * partition max over the 4 waves.
//  * pass 2 (softmax, P quantization, PV): per 32-token chunk the 4 x 32
//    probabilities p = exp(t - m) are formed two per lane; l accumulates the
//    unquantized p; p' = c p is quantized per aligned 16-token block
//    (amax2_or_amax6 with tau, or amax6) and s * e2m1 (exact in 16 bits) is
//    staged in LDS as the A operand. V codes come as B operands of 8 MFMAs
//    (one per output channel slab).
//  * the 4 waves' o and l are summed in LDS; o is divided by c.
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
  float logit[4 * kMaxTok];                 // [head][token]; reused for the o reduction
  uint16_t qhat[2][4][kD];                  // 16-bit dequantized query terms
  float q[4][kD];                           // raw float32 query (BF16 partition)
  float qmu[4];
  uint16_t p[4][4][32];                     // per wave: P_hat staging [head][token]
  float red[4][4];                          // per wave, per head
  float lsum[4][4];
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

// DPP row controls (16-lane rows): shift left / right by 4, rotate by 8.
constexpr int kDppRowShl4 = 0x104;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowRor8 = 0x128;

// Butterfly stages with partner lane ^ 4 and lane ^ 8 inside a 16-lane row.
__device__ __forceinline__ void fwht_xlane_4_8(float* x, int i) {
  const bool up4 = (i & 4) != 0, up8 = (i & 8) != 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float p = shfl_xor(x[k], 4);
    x[k] = up4 ? __fsub_rn(p, x[k]) : __fadd_rn(x[k], p);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float p = shfl_xor(x[k], 8);
    x[k] = up8 ? __fsub_rn(p, x[k]) : __fadd_rn(x[k], p);
  }
}

// The raw query elements and key means of lane i of row g (loaded first, so
// their latency overlaps the page-id staging and the first page loads).
struct QueryIn {
  uint4 q;
  float4 mu0, mu1;
};

__device__ __forceinline__ QueryIn query_load(const DecodeLaunch& P, int b, int h, int g, int i) {
  QueryIn in;
  in.q = *reinterpret_cast<const uint4*>(P.q + ((size_t)b * P.hq + h * kGroup + g) * kD + 8 * i);
  if (P.key_smoothing) {
    const float4* mu4 = reinterpret_cast<const float4*>(P.key_shift + h * kD + 8 * i);
    in.mu0 = mu4[0];
    in.mu1 = mu4[1];
  } else {
    in.mu0 = in.mu1 = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  return in;
}

// Query row g of the group on 16 lanes (lane i holds elements [8i, 8i+8)):
// q . mu, the Hadamard rotation (stages 1, 2, 4 in-lane, 8 .. 64 across
// lanes by DPP), then Q1 and the residual Q2, dequantized into LDS. The same
// float32 operations in the same order as the page writer's key path and the
// row quantizer, so the codes are identical.
template <bool kMx, int kTerms>
__device__ __forceinline__ void query_row(const DecodeLaunch& P, const QueryIn& in, Smem& sm, int g, int i) {
  float x[8];
  const uint32_t ww[4] = {in.q.x, in.q.y, in.q.z, in.q.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = bf16_lo(ww[k]);
    x[2 * k + 1] = bf16_hi(ww[k]);
  }
  const float mu[8] = {in.mu0.x, in.mu0.y, in.mu0.z, in.mu0.w, in.mu1.x, in.mu1.y, in.mu1.z, in.mu1.w};
  float dot = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) dot = fmaf(x[k], mu[k], dot);
  dot = sum16(dot);
  if (i == 0) sm.qmu[g] = dot;
  if (P.rotation) {
    fwht_inlane<8>(x);
    fwht_xlane<8, kDppQuadXor1>(x, (i & 1) != 0);
    fwht_xlane<8, kDppQuadXor2>(x, (i & 2) != 0);
    fwht_xlane_4_8(x, i);
    const float c = inv_sqrt_d();
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __fmul_rn(x[k], c);
  }
#pragma unroll
  for (int term = 0; term < kTerms; ++term) {
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a = __builtin_fmaxf(a, __builtin_fabsf(x[k]));
    float s;
    uint32_t pk;
    if (kMx) {
      // 32-element block = this quad of lanes; candidates E_hi, E_hi - 1
      a = __builtin_fmaxf(a, dpp_f32<kDppQuadXor1>(a));
      a = __builtin_fmaxf(a, dpp_f32<kDppQuadXor2>(a));
      int ehi = a > 0.0f ? mx_exponent_hi(a) : -127;
      ehi = ehi < -127 ? -127 : (ehi > 127 ? 127 : ehi);
      const int elo = ehi - 1 < -127 ? -127 : ehi - 1;
      uint32_t phi, plo;
      float ehi_err = quant_block<8, true>(x, pow2_f32(ehi), &phi);
      float elo_err = quant_block<8, true>(x, pow2_f32(elo), &plo);
      // the 32-element tree: ((t0 + t1) + (t2 + t3)) over the quad's subtrees
      ehi_err = __fadd_rn(ehi_err, dpp_f32<kDppQuadXor1>(ehi_err));
      ehi_err = __fadd_rn(ehi_err, dpp_f32<kDppQuadXor2>(ehi_err));
      elo_err = __fadd_rn(elo_err, dpp_f32<kDppQuadXor1>(elo_err));
      elo_err = __fadd_rn(elo_err, dpp_f32<kDppQuadXor2>(elo_err));
      const bool take_lo = (elo_err < ehi_err) && (elo < ehi) && a > 0.0f;
      s = a > 0.0f ? pow2_f32(take_lo ? elo : ehi) : 0.0f;
      pk = a > 0.0f ? (take_lo ? plo : phi) : 0u;
    } else {
      // 16-element block = this pair of lanes
      a = __builtin_fmaxf(a, dpp_f32<kDppQuadXor1>(a));
      s = e4m3_value(e4m3_encode(a / 6.0f));
      quant_block<8, false>(x, s, &pk);
    }
    float deq[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t nib = (pk >> (4 * k)) & 0xFu;
      const float gv = __fmul_rn(e2m1_grid(nib & 7u), s);
      deq[k] = (nib & 8u) ? -gv : gv;
    }
    uint4 o;
    o.x = op16<kMx>(deq[0]) | (op16<kMx>(deq[1]) << 16);
    o.y = op16<kMx>(deq[2]) | (op16<kMx>(deq[3]) << 16);
    o.z = op16<kMx>(deq[4]) | (op16<kMx>(deq[5]) << 16);
    o.w = op16<kMx>(deq[6]) | (op16<kMx>(deq[7]) << 16);
    *reinterpret_cast<uint4*>(&sm.qhat[term][g][8 * i]) = o;
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __fsub_rn(x[k], deq[k]);
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

template <bool kMx, int kTerms, bool kUnder>
__device__ void fp4_partition(const DecArgs& A, Smem& sm, int b, int h, int s, int L, int n_full) {
  const DecodeLaunch& P = A.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p0 = (s - 1) * P.ppp;
  const int p1 = min(n_full, s * P.ppp);
  const int npg = p1 - p0;
  const int lo = max(P.sink, kPage * p0);
  const size_t hkv = P.hkv;
  QueryIn qin;
  if (lane < 16) qin = query_load(P, b, h, wave, lane);

  if (tid < npg) {
    const int ph = P.block_tables[(size_t)b * P.max_pages_per_seq + p0 + tid];
    sm.page[tid] = (ph < 0 || ph >= P.num_pages) ? -1 : ph;
  }
  __syncthreads();
  auto blk_of = [&](int pi) -> size_t {
    const int ph = sm.page[pi];
    return (size_t)(ph < 0 ? 0 : ph) * hkv + h;
  };

  KPage kcur, knxt;
  if (wave < npg) load_k<kMx>(kcur, P, blk_of(wave), lane);
  if (lane < 16) query_row<kMx, kTerms>(P, qin, sm, wave, lane);
  __syncthreads();

  // A operands: lane (row = lane & 15, k-group kg = lane >> 4); MFMA c covers
  // channels 32 kg + 8 c + [0, 8)
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
  const f32x4_t acc0 = {sm.qmu[0], sm.qmu[1], sm.qmu[2], sm.qmu[3]};
  const float sigma = P.softmax_scale;
  float* logit = sm.logit;

  // ---- pass 1: logits
  float mrun[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  for (int pi = wave; pi < npg; pi += 4) {
    if (pi + 4 < npg) load_k<kMx>(knxt, P, blk_of(pi + 4), lane);
    const bool has_sink = kPage * (p0 + pi) < lo;          // uniform per page
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      u32x4_t bk[4];
      if (kMx) {
        const uint32_t sb = (word_of(kcur.sc, t >> 2) >> (8 * (t & 3))) & 0xFFu;
        const float sv = pow2_f32((int)sb - 127);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t cw = word_of(kcur.code[t], c);
          bk[c] = (u32x4_t){cvt_bf16_pair(cw, sv, 0), cvt_bf16_pair(cw, sv, 1), cvt_bf16_pair(cw, sv, 2),
                            cvt_bf16_pair(cw, sv, 3)};
        }
      } else {
        const f16x2_t sp = e4m3_pair_f16(word_of(kcur.sc, t >> 1), (t & 1) != 0);   // (s_lo, s_hi)
        const f16x2_t slo = {sp[0], sp[0]}, shi = {sp[1], sp[1]};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t cw = word_of(kcur.code[t], c);
          const f16x2_t sc = c < 2 ? slo : shi;
          bk[c] = (u32x4_t){u32_of(grid_f16_pair(cw, 0) * sc), u32_of(grid_f16_pair(cw, 1) * sc),
                            u32_of(grid_f16_pair(cw, 2) * sc), u32_of(grid_f16_pair(cw, 3) * sc)};
        }
      }
      f32x4_t acc = acc0;
#pragma unroll
      for (int term = 0; term < kTerms; ++term) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = mfma<kMx>(aq[term][c], bk[c], acc);
      }
      if (lane < 16) {
        const int local = pi * kPage + t * 16 + lane;        // token - 128 p0
        float lg[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) lg[g] = sigma * acc[g];
        if (has_sink && kPage * p0 + local < lo) {
#pragma unroll
          for (int g = 0; g < 4; ++g) lg[g] = kNegInf;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          logit[g * kMaxTok + local] = lg[g];
          mrun[g] = fmaxf(mrun[g], lg[g]);
        }
      }
    }
    kcur = knxt;
  }
  VPage vcur, vnxt;
  if (wave < npg) load_v<kMx>(vcur, P, blk_of(wave), lane);
#pragma unroll
  for (int g = 0; g < 4; ++g) mrun[g] = max16(mrun[g]);
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
  const float mh = ph == 0 ? m[0] : (ph == 1 ? m[1] : (ph == 2 ? m[2] : m[3]));
  const float cf = (float)P.c;
  const float tau = P.tau;
  const float* lrow = logit + ph * kMaxTok;
  float lacc = 0.0f;
  f32x4_t acco[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acco[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  for (int pi = wave; pi < npg; pi += 4) {
    if (pi + 4 < npg) load_v<kMx>(vnxt, P, blk_of(pi + 4), lane);
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      // probabilities of tokens (2 pj, 2 pj + 1), head ph
      const int local = pi * kPage + ch * 32 + 2 * pj;
      const float2 tt = *reinterpret_cast<const float2*>(lrow + local);
      const float e0 = (mh == kNegInf) ? 0.0f : __expf(tt.x - mh);
      const float e1 = (mh == kNegInf) ? 0.0f : __expf(tt.y - mh);
      lacc += e0 + e1;
      const float q0 = cf * e0, q1 = cf * e1;
      const float a = max8(fmaxf(q0, q1));     // the aligned 16-token block is 8 lanes
      const uint32_t scode = e4m3_encode((kUnder && a < tau) ? a * 0.5f : a / 6.0f);
      const float sv = e4m3_value(scode);
      const E2m1Thr T = e2m1_thresholds(sv);
      const float g0 = T.zero ? 0.0f : __fmul_rn(e2m1_grid(e2m1_mag(q0, T)), sv);
      const float g1 = T.zero ? 0.0f : __fmul_rn(e2m1_grid(e2m1_mag(q1, T)), sv);
      *reinterpret_cast<uint32_t*>(&sm.p[wave][ph][2 * pj]) = op16<kMx>(g0) | (op16<kMx>(g1) << 16);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): staging visible to the wave
      __builtin_amdgcn_wave_barrier();
      u32x4_t ap = {0u, 0u, 0u, 0u};
      if (row < 4) {
        const uint4 t = *reinterpret_cast<const uint4*>(&sm.p[wave][row][8 * kg]);
        ap[0] = t.x; ap[1] = t.y; ap[2] = t.z; ap[3] = t.w;
      }
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
      __builtin_amdgcn_wave_barrier();
    }
    vcur = vnxt;
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
    pstore(part + 512 + tid, poisoned ? 0.0f : m[tid]);
    pstore(part + 516 + tid, poisoned ? 1.0f : sm.lsum[0][tid] + sm.lsum[1][tid] + sm.lsum[2][tid] + sm.lsum[3][tid]);
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
  publish_and_merge(merge_ctx(A), &sm.ticket, &sm.red[0][0], sm.logit, 4 * kMaxTok, b, h, nparts + 1);
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
