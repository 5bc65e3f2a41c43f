// Device codecs for the bdfp4 kernels (gfx950): bf16 widening, E4M3 and E8M0
// scales, E2M1 element codes, the 128-point Hadamard butterflies and the
// float32 error tree of the adaptive scale searches.
//
// Format definitions: OCP 8-bit Floating Point (E4M3, max 448, no infinities)
// and OCP Microscaling v1.0 (E2M1 elements, E8M0 scales). Scale-mode names
// from "BitDecoding-FP4 evaluation/config.py" (recipe_additional_config,
// probability_environment, KV_MODES). Every value produced here must be a
// bit-exact function of its inputs: float32 operations are written out one
// by one and the library is compiled with -ffp-contract=off.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdfp4 {

constexpr int kD = 128;     // head_dim
constexpr int kPage = 128;  // tokens per page (block_size)

// float32 nearest to 1/sqrt(128) (0x3DB504F3)
__device__ __forceinline__ float inv_sqrt_d() { return __uint_as_float(0x3DB504F3u); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- E4M3

// Code of the E4M3 value nearest to v >= 0 (ties to even), saturating at 448.
// The gfx950 down-convert rounds to nearest even but turns values from 464
// up into NaN, so the input is clamped to 448 first (448 itself and every
// value in [448, 464) encode as 0x7E either way; a NaN clamps to 448).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const float c = __builtin_fminf(v, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// Value of an E4M3 code (the hardware up-convert is exact for every code).
__device__ __forceinline__ float e4m3_value(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }

// ---------------------------------------------------------------- exact quotients

// RN(x / m) for a divisor m with r = RN(1/m): q0 = RN(x r), then one FMA
// correction. Bit-identical to the IEEE quotient (signed zeros included) for
// the eight E4M3 significands m = 1 + k/8 and for m = 6 whenever
// |x| >= 2^-122 (exhaustive check over every float32 significand); for
// smaller |x| every caller's code is zero regardless.
__device__ __forceinline__ float quot(float x, float m, float r) {
  const float q0 = __fmul_rn(x, r);
  const float e = __builtin_fmaf(m, q0, -x);
  return __builtin_fmaf(e, -r, q0);
}

// RN(a / 6).
__device__ __forceinline__ float div6(float a) { return quot(a, 6.0f, __uint_as_float(0x3E2AAAABu)); }

// Significand m in [1, 2) of a positive normal float32 s = 2^E m, and the
// index k of m = 1 + k/8 when s is an E4M3 value.
__device__ __forceinline__ float significand(float s) {
  return __uint_as_float((__float_as_uint(s) & 0x007FFFFFu) | 0x3F800000u);
}
__device__ __forceinline__ uint32_t sig_index(float s) { return (__float_as_uint(s) >> 20) & 7u; }

// RN(1 / (1 + k/8)), k = 0..7.
__device__ __forceinline__ float rcp_significand(uint32_t k) {
  const uint32_t a0 = (k & 1u) ? 0x3F638E39u : 0x3F800000u;
  const uint32_t a1 = (k & 1u) ? 0x3F3A2E8Cu : 0x3F4CCCCDu;
  const uint32_t a2 = (k & 1u) ? 0x3F1D89D9u : 0x3F2AAAABu;
  const uint32_t a3 = (k & 1u) ? 0x3F088889u : 0x3F124925u;
  const uint32_t b0 = (k & 2u) ? a1 : a0;
  const uint32_t b1 = (k & 2u) ? a3 : a2;
  return __uint_as_float((k & 4u) ? b1 : b0);
}

// ---------------------------------------------------------------- E8M0

// 2^E as float32 for E in [-127, 127] (E = -127 is the float32 subnormal 2^-127).
__device__ __forceinline__ float pow2_f32(int e) {
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// Least integer E with a <= 6 * 2^E, for a > 0 (6 * 2^E = 1.5 * 2^(E+2)).
__device__ __forceinline__ int mx_exponent_hi(float a) {
  int bias = 0;
  uint32_t u = __float_as_uint(a);
  if (u < 0x00800000u) {                  // float32 subnormal: scale up exactly
    a = a * 18446744073709551616.0f;      // 2^64
    u = __float_as_uint(a);
    bias = 64;
  }
  const int e = (int)(u >> 23) - 127;
  return e - 2 + ((u & 0x7FFFFFu) > 0x400000u ? 1 : 0) - bias;
}

// ---------------------------------------------------------------- E2M1

// Thresholds between consecutive grid points times s: the midpoints 0.25,
// 0.75, 1.25, 1.75, 2.5, 3.5, 5 (exact products: s has at most 4 significant
// bits or is a power of two).
struct E2m1Thr {
  float t0, t1, t2, t3, t4, t5, t6;
  bool zero;
};

__device__ __forceinline__ E2m1Thr e2m1_thresholds(float s) {
  E2m1Thr T;
  T.t0 = 0.25f * s; T.t1 = 0.75f * s; T.t2 = 1.25f * s; T.t3 = 1.75f * s;
  T.t4 = 2.5f * s;  T.t5 = 3.5f * s;  T.t6 = 5.0f * s;
  T.zero = !(s > 0.0f);
  return T;
}

// Magnitude code (0..7) of |x| relative to s: nearest grid point of the exact
// ratio, ties to the even code. The code counts the thresholds passed; at a
// tie the step to an even code is taken, i.e. thresholds 1, 3, 5 are passed
// on >= and thresholds 0, 2, 4, 6 on >. The passed set is a prefix, so a
// three-level binary search finds its length.
__device__ __forceinline__ uint32_t e2m1_mag(float ax, const E2m1Thr& T) {
  uint32_t c = (ax >= T.t3) ? 4u : 0u;
  const float tb = c ? T.t5 : T.t1;
  c += (ax >= tb) ? 2u : 0u;
  const float tc = (c & 4u) ? ((c & 2u) ? T.t6 : T.t4) : ((c & 2u) ? T.t2 : T.t0);
  c += (ax > tc) ? 1u : 0u;
  return c;
}

// Grid magnitude of a code 0..7: 0, .5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_grid(uint32_t c) {
  return c < 4u ? 0.5f * (float)c : (c == 7u ? 6.0f : (float)(c - 2u));
}

// 4-bit code: sign bit of x in bit 3, magnitude in bits 2..0; 0 if s == 0.
__device__ __forceinline__ uint32_t e2m1_nibble(float x, const E2m1Thr& T) {
  const uint32_t mag = e2m1_mag(__builtin_fabsf(x), T);
  const uint32_t sgn = (__float_as_uint(x) >> 31) << 3;
  return T.zero ? 0u : (sgn | mag);
}

// E2M1 codes of x0 (bits 3..0) and x1 (bits 7..4) against a positive normal
// scale s = 2^E m whose significand m has reciprocal r = RN(1/m): the exact
// quotients x / m, then the gfx950 down-convert, which divides by 2^E (the
// exponent of its scale operand), rounds to nearest even with saturation at
// 6 and keeps the sign. A float32 quotient never lands on an E2M1 midpoint
// unless it is exactly that midpoint, so each code is the one of the exact
// ratio x / s.
__device__ __forceinline__ uint32_t e2m1_pair(float x0, float x1, float s, float m, float r) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, quot(x0, m, r), quot(x1, m, r), s, 0) & 0xFFu;
}

// The same two codes written into byte `byte` of old (the other bytes of
// old are kept; the select must be a constant).
__device__ __forceinline__ uint32_t e2m1_pair_into(uint32_t old, float q0, float q1, float s, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, q0, q1, s, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, q0, q1, s, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, q0, q1, s, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, q0, q1, s, 3);
  }
}

typedef float e2m1_f32x2_t __attribute__((ext_vector_type(2)));

// Signed grid values (exact float32) of the two E2M1 codes in byte `byte`
// of w: the hardware convert with scale 1 (the select must be a constant).
__device__ __forceinline__ e2m1_f32x2_t e2m1_grid_pair(uint32_t w, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

// ---------------------------------------------------------------- blocks

// Quantize N in-register values (N even) with scale value s (float32):
// codes packed 8 per uint32 (element 2i in the low nibble of byte i) and,
// when requested, the float32 squared error summed as a balanced pairwise
// tree ((e0+e1)+(e2+e3))+... . Normal scales take the exact-quotient route
// of e2m1_pair; the float32 subnormal 2^-127 (the lowest E8M0 scale) takes
// the threshold search; a zero scale gives all-zero codes. The error tree is
// built incrementally: lvl[k] holds the pending left sum of 2^k elements;
// element i is merged with the levels of its trailing one bits (left operand
// the older sum), so the additions and their order are exactly those of the
// level-by-level tree.
template <int N, bool kSse>
__device__ __forceinline__ float quant_block(const float* x, float s, uint32_t* packed) {
  static_assert(N % 2 == 0, "pairs of elements");
  constexpr int kLv = N == 32 ? 6 : (N == 16 ? 5 : (N == 8 ? 4 : (N == 4 ? 3 : 2)));
  constexpr int kW = (N + 7) / 8;
#pragma unroll
  for (int w = 0; w < kW; ++w) packed[w] = 0u;
  if (s >= 1.17549435e-38f) {
    const float m = significand(s);
    const float r = rcp_significand(sig_index(s));
#pragma unroll
    for (int i = 0; i < N; i += 2) packed[i >> 3] |= e2m1_pair(x[i], x[i + 1], s, m, r) << (4 * (i & 7));
  } else if (s > 0.0f) {
    const E2m1Thr T = e2m1_thresholds(s);
#pragma unroll
    for (int i = 0; i < N; ++i) packed[i >> 3] |= e2m1_nibble(x[i], T) << (4 * (i & 7));
  }
  if (!kSse) return 0.0f;
  float lvl[kLv];
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    // grid values of the two codes (hardware E2M1 -> float32 convert with
    // scale 1: exact), then |x| - s |grid| (the product is exact)
    const e2m1_f32x2_t gp = e2m1_grid_pair(packed[i >> 3], (i & 7) >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int ie = i + e;
      const float q = __fmul_rn(__builtin_fabsf(gp[e]), s);
      const float d = __fsub_rn(__builtin_fabsf(x[ie]), q);
      float v = __fmul_rn(d, d);
      int k = 0;
#pragma unroll
      for (int bit = 1; bit < N; bit <<= 1, ++k) {
        if ((ie & bit) == 0) break;
        v = __fadd_rn(lvl[k], v);
      }
      lvl[k] = v;
    }
  }
  return lvl[kLv - 1];
}

// The same for a scale value s that is either 0 or a normal float32, as every
// E4M3 value is (the least nonzero one is 2^-9): every pair takes the exact-quotient
// route, written by the down-convert straight into its byte of the packed
// word (the convert leaves the other three bytes as they were); a zero scale
// selects all-zero codes afterwards. The error term |x| - s |g| is one FMA,
// since s |g| is exact (at most 6 significant bits), so it rounds exactly as
// the subtraction of the rounded product does.
// kPow2: s is a power of two 2^E with E >= -126 (a normal E8M0 scale), so the
// quotient by the significand is x itself and the convert alone is exact.
template <int N, bool kSse, bool kPow2 = false>
__device__ __forceinline__ float quant_block_normal(const float* x, float s, uint32_t* packed) {
  static_assert(N % 8 == 0, "whole packed words");
  constexpr int kLv = N == 32 ? 6 : (N == 16 ? 5 : 4);
  constexpr int kW = N / 8;
  const float m = significand(s);               // 1 for s = 0
  const float r = rcp_significand(sig_index(s));
  const bool live = s > 0.0f;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    uint32_t word = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float x0 = x[8 * w + 2 * b], x1 = x[8 * w + 2 * b + 1];
      word = kPow2 ? e2m1_pair_into(word, x0, x1, s, b) : e2m1_pair_into(word, quot(x0, m, r), quot(x1, m, r), s, b);
    }
    packed[w] = (kPow2 || live) ? word : 0u;
  }
  if (!kSse) return 0.0f;
  float lvl[kLv];
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    const e2m1_f32x2_t gp = e2m1_grid_pair(packed[i >> 3], (i & 7) >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int ie = i + e;
      const float d = __builtin_fmaf(-__builtin_fabsf(gp[e]), s, __builtin_fabsf(x[ie]));
      float v = __fmul_rn(d, d);
      int k = 0;
#pragma unroll
      for (int bit = 1; bit < N; bit <<= 1, ++k) {
        if ((ie & bit) == 0) break;
        v = __fadd_rn(lvl[k], v);
      }
      lvl[k] = v;
    }
  }
  return lvl[kLv - 1];
}

// Scale code of an aligned 16-value block of p' = c p with block maximum
// a >= 0: E4M3(a / 2) when kUnder and a < tau (amax2_or_amax6), otherwise
// E4M3(a / 6) (amax6).
template <bool kUnder>
__device__ __forceinline__ uint32_t p_scale_code(float a, float tau) {
  return e4m3_encode((kUnder && a < tau) ? __fmul_rn(a, 0.5f) : div6(a));
}

__device__ __forceinline__ float absmax16(const float* x) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(x[i]));
  return a;
}

// NVFP4 block of 16: amax6 or four_six. Returns the E4M3 scale code.
template <bool kFourSix>
__device__ __forceinline__ uint32_t nv_block(const float* x, uint32_t* packed) {
  const float a = absmax16(x);
  const uint32_t c6 = e4m3_encode(div6(a));
  if (!kFourSix) {
    quant_block_normal<16, false>(x, e4m3_value(c6), packed);
    return c6;
  }
  const uint32_t c4 = e4m3_encode(a * 0.25f);
  uint32_t p6[2], p4[2];
  const float err6 = quant_block_normal<16, true>(x, e4m3_value(c6), p6);
  __builtin_amdgcn_sched_barrier(0);   // keep the two candidates from interleaving
  const float err4 = quant_block_normal<16, true>(x, e4m3_value(c4), p4);
  const bool take4 = err4 < err6;
  packed[0] = take4 ? p4[0] : p6[0];
  packed[1] = take4 ? p4[1] : p6[1];
  return take4 ? c4 : c6;
}

// MXFP4 block of 32 with the two-candidate exponent search. Returns the E8M0 code.
__device__ __forceinline__ uint32_t mx_block(const float* x, uint32_t* packed) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(x[i]));
  if (!(a > 0.0f)) {
#pragma unroll
    for (int w = 0; w < 4; ++w) packed[w] = 0u;
    return 0u;
  }
  int ehi = mx_exponent_hi(a);
  ehi = ehi < -127 ? -127 : (ehi > 127 ? 127 : ehi);
  const int elo = ehi - 1 < -127 ? -127 : ehi - 1;
  uint32_t phi[4], plo[4];
  float err_hi, err_lo;
  if (elo >= -126) {
    // both scales normal powers of two: the direct convert
    err_hi = quant_block_normal<32, true, true>(x, pow2_f32(ehi), phi);
    __builtin_amdgcn_sched_barrier(0);   // keep the two candidates from interleaving
    err_lo = quant_block_normal<32, true, true>(x, pow2_f32(elo), plo);
  } else {
    // a candidate at the float32 subnormal 2^-127: the threshold search
    err_hi = quant_block<32, true>(x, pow2_f32(ehi), phi);
    err_lo = quant_block<32, true>(x, pow2_f32(elo), plo);
  }
  const bool take_lo = (err_lo < err_hi) && (elo < ehi);
#pragma unroll
  for (int w = 0; w < 4; ++w) packed[w] = take_lo ? plo[w] : phi[w];
  return (uint32_t)((take_lo ? elo : ehi) + 127);
}

// Dequantized values (float32, exact) of 8 codes in a uint32 with scale s.
__device__ __forceinline__ void deq8(uint32_t w, float s, float* out) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t nib = (w >> (4 * i)) & 0xFu;
    const float g = e2m1_grid(nib & 7u) * s;
    out[i] = (nib & 8u) ? -g : g;
  }
}

// ---------------------------------------------------------------- Hadamard

// In-lane stages h = 1 .. N/2 of the fast Walsh-Hadamard transform on N
// consecutive elements (pairs (i, i+h) with bit h of i clear -> (a+b, a-b)).
template <int N>
__device__ __forceinline__ void fwht_inlane(float* x) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = __fadd_rn(a, b);
        x[i + h] = __fsub_rn(a, b);
      }
    }
  }
}

// DPP lane permutations: quad_perm within groups of 4 lanes, mirrors
// within 8 and 16 lanes.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Maximum / sum over aligned groups of 8 or 16 lanes (every lane gets it).
__device__ __forceinline__ float max8(float v) {
  v = __builtin_fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = __builtin_fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  return __builtin_fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
}
__device__ __forceinline__ float max16(float v) {
  v = max8(v);
  return __builtin_fmaxf(v, dpp_f32<kDppRowMirror>(v));
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowHalfMirror>(v);
  return v + dpp_f32<kDppRowMirror>(v);
}

// Cross-lane butterfly stage: the lane whose selector bit is clear keeps
// own + partner, the other partner - own (the (a+b, a-b) pair of the stage).
// Written as partner + (+-own): the upper lane's p - x is p + (-x) exactly,
// and the DPP read folds into the addition.
// All sign flips are formed first, so that no DPP read follows closely on
// the write of its register.
template <int N, int kCtrl>
__device__ __forceinline__ void fwht_xlane(float* x, bool upper) {
  const uint32_t flip = upper ? 0x80000000u : 0u;
  float own[N];
#pragma unroll
  for (int i = 0; i < N; ++i) own[i] = __uint_as_float(__float_as_uint(x[i]) ^ flip);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = __fadd_rn(dpp_f32<kCtrl>(x[i]), own[i]);
}

// Rotation of a 128-element row held as 32 consecutive elements per lane in
// 4 consecutive lanes (lane q of the quad holds elements [32q, 32q+32)):
// stages 1..16 in-lane, 32 across lanes q^1, 64 across q^2, then * 1/sqrt(128).
__device__ __forceinline__ void rotate_row_quad(float* x, int q) {
  fwht_inlane<32>(x);
  fwht_xlane<32, kDppQuadXor1>(x, (q & 1) != 0);
  fwht_xlane<32, kDppQuadXor2>(x, (q & 2) != 0);
  const float c = inv_sqrt_d();
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = __fmul_rn(x[i], c);
}

// Widen 32 bf16 (four 16-byte words) to float32.
__device__ __forceinline__ void widen32(const uint4* w, float* x) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t v[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[8 * k + 2 * i] = bf16_lo(v[i]);
      x[8 * k + 2 * i + 1] = bf16_hi(v[i]);
    }
  }
}

}  // namespace bdfp4
