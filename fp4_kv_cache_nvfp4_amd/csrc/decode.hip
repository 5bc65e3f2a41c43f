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
// (1..4) consecutive full pages. Workgroup j serves (sequence, KV head)
// j mod (batch * KV heads) in column j / (batch * KV heads). The BF16
// partition (sink + tail tokens, exact float32 attention of the raw query)
// runs in a workgroup of its own in column 0 when one more column still fits
// the chip at the kernel's occupancy (that column is dispatched first, or
// last when the FP4 workgroups outnumber the compute units), and is
// otherwise folded into the first FP4 workgroup, computed before that
// workgroup requests its first K pages. A grid larger than the chip holds is
// compacted: workgroup j takes the j-th (column, sequence) unit that has
// pages (compact_vj), so that no resident slot goes to a unit without work.
// Every partition computes, for the 4 query heads of its KV head,
// m = max logit, l = sum exp(t - m) and o = sum P_hat v_hat; a workgroup
// merges its four waves in LDS, stores one partial and takes a ticket; the
// last of a (sequence, KV head) merges all of them (merge.hpp).
//
// FP4 partition, per wave:
//  * page ids: lane i reads page i of the partition's block-table run; the
//    wave then fills both K buffers (the two halves of its first page, or
//    its first two whole pages);
//  * prologue: wave g rotates (128-point Hadamard, float32) and quantizes
//    query row g as Q1 + Q2 (amax6 per 16 or mxfp4_search per 32), two
//    elements per lane. NVFP4: the dequantized terms are exact in 16 bits
//    and become the A operands of v_mfma_f32_16x16x32_f16; MXFP4: the codes
//    and E8M0 scale codes themselves are the A operand of the scaled FP4
//    MFMA. Row 2g + t holds term t of head g and rows 8..15 repeat rows
//    0..7. q . mu (raw float32 query, key means) seeds the term-1 rows of the
//    accumulator.
//  * pass 1 (QK^T): the wave streams its K pages, then its V pages, through
//    two buffers per kind: half pages (K tiles 0-3 / 4-7, V chunks 0-1 / 2-3)
//    in all kernels but the 1- and 2-slot channel-key-scale ones, which hold
//    whole pages; a buffer is refilled as soon as its contents are used, so
//    one buffer is in flight while the other is consumed. Per 16-token tile a
//    lane holds 16 code bytes (one coalesced 1 KiB run per wave) and the
//    page's scales come in one 16-byte load per lane. Four
//    f16 MFMAs (NVFP4) or one v_mfma_scale_f32_16x16x128_f8f6f4 (MXFP4: the
//    page's code bytes and E8M0 scales used as they are) give both terms of
//    all four heads; their sum, the raw logit
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
// exponent of their float32 scale. MXFP4 scales are powers of two: K and the
// query enter the scaled FP4 MFMA as codes, and V converts exactly to bf16 in
// one step (its E8M0 scales run along the channels, not along the token sum
// whose blocks the MFMA's scales would have to follow). For NVFP4 the codes
// are converted with scale 1 to f16 and multiplied, two at a time, by their
// E4M3 scales converted to f16 by the hardware E4M3 convert; the product has
// at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in f16. The NVFP4 V page stores tokens
// t, t+1 of one channel in a byte, so a converted pair is directly one 32-bit
// word of the PV B operand.
#include <atomic>
#include <mutex>

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

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

// D += (A 2^(sa - 127)) (B 2^(sb - 127)) on a 16x16x128 tile of E2M1 codes
// (v_mfma_scale_f32_16x16x128_f8f6f4, both operands FP4): lane l supplies
// row / column l & 15, channels 32 (l >> 4) .. +32 as 16 bytes (element 2i in
// the low nibble) and the E8M0 code of that 32-channel block; sa is byte 0
// of its word, sb byte kSel of its word. The products are exact, the sums
// float32.
template <int kSel>
__device__ __forceinline__ f32x4_t mfma_fp4_scaled(u32x4_t a, uint32_t sa, u32x4_t b, uint32_t sb, f32x4_t c) {
  const i32x8_t a8 = {(int32_t)a[0], (int32_t)a[1], (int32_t)a[2], (int32_t)a[3], 0, 0, 0, 0};
  const i32x8_t b8 = {(int32_t)b[0], (int32_t)b[1], (int32_t)b[2], (int32_t)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, 0, (int32_t)sa, kSel, (int32_t)sb);
}

__device__ __forceinline__ f32x4_t mfma_fp4_scaled_byte(int sel, u32x4_t a, uint32_t sa, u32x4_t b, uint32_t sb,
                                                        f32x4_t c) {
  switch (sel) {
    case 0: return mfma_fp4_scaled<0>(a, sa, b, sb, c);
    case 1: return mfma_fp4_scaled<1>(a, sa, b, sb, c);
    case 2: return mfma_fp4_scaled<2>(a, sa, b, sb, c);
    default: return mfma_fp4_scaled<3>(a, sa, b, sb, c);
  }
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
  uint8_t qcode[2][4][kD / 2];              // MXFP4: E2M1 codes of the query terms [term][head][byte]
  uint32_t qsc[2][4][4];                    // MXFP4: their E8M0 scale codes [term][head][32-channel block]
  uint32_t pst[4][16][16];                  // per wave: P_hat staging [row][token pair]; rows 4..15 stay 0
  float qmu[4];
  float red[4][4];                          // per wave, per head: partition maximum (raw logit)
  float lsum[4][4];                         // per wave, per head: sum of c p
  float rcp[8];                             // RN(1 / (1 + k/8)), k = 0..7
  int bad[4];                               // per wave: its block table names an invalid page
  int tick;
  float tmax[4][4][kWaveTok / 16];          // running-max variant: per wave, head, 16-token block: raw maximum
  uint32_t ksc[4][256];                     // channel key geometry: per wave, the K page's scales [token block][channel]
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
// tail page: exact float32 attention of the raw query. QK^T runs on
// v_mfma_f32_16x16x32_bf16 (bf16 x bf16 products are exact, the sums float32,
// as in a float32 dot product of the bf16 inputs): wave w takes the 16-token
// tiles w, w + 4, ..., rows 0..3 of A are the 4 query heads. The maximum and
// l come from DPP row reductions and one LDS exchange across the waves; PV is
// float32 on the VALU, thread (wave w, lane l) taking channels 2l, 2l + 1 of
// the tokens w, w + 4, .... The query, K and V rows of up to 144 tokens are
// all requested before the first wait, so the partition costs one memory
// round trip; longer sink + tail spans read their remaining V rows after.
constexpr int kBfTilesPerWave = 4;                 // 16 tiles of 16 tokens: up to 256 tokens
constexpr int kBfVPerThread = 36;                  // V rows per thread requested up front (144 tokens)

__device__ Partial bf16_partition(const DecArgs& A, Smem& sm, int b, int h, int L, int n_full) {
  const DecodeLaunch& P = A.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = P.sink;
  const int nsink = L < S ? L : S;
  const int tail_lo = S > kPage * n_full ? S : kPage * n_full;
  const int ntail = L > tail_lo ? L - tail_lo : 0;
  const int nb = nsink + ntail;                      // <= 128 + 127 < 256
  const size_t bhk = (size_t)b * P.hkv + h;
  const int tail0 = tail_lo - kPage * n_full;
  auto row_of = [&](const uint16_t* sink, const uint16_t* tail, int j) -> const uint16_t* {
    return j < nsink ? sink + (bhk * S + j) * kD : tail + (bhk * kPage + tail0 + (j - nsink)) * kD;
  };
  const int row = lane & 15, kg = lane >> 4;
  // A: query head `row` (rows 4..15 zero), channels 32 c + 8 kg .. + 8 for MFMA c
  u32x4_t aq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (row < kGroup) {
      const uint4 t = *reinterpret_cast<const uint4*>(P.q + ((size_t)b * P.hq + h * kGroup + row) * kD + 32 * c + 8 * kg);
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
    aq[c] = v;
  }
  // B: token 16 tile + row of each of this wave's tiles, same channels.
  // Whole tiles are taken or skipped by a wave-uniform test (a skipped
  // tile's logits are masked below); inside a taken tile a row past nb reads
  // row nb - 1 instead (masked too), so no load sits behind a per-lane branch
  u32x4_t bk[kBfTilesPerWave][4];
#pragma unroll
  for (int k = 0; k < kBfTilesPerWave; ++k) {
    const int t16 = 16 * (wave + 4 * k);
    const int j = min(t16 + row, nb - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) bk[k][c] = (u32x4_t){0u, 0u, 0u, 0u};
    if (t16 < nb) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 t = *reinterpret_cast<const uint4*>(row_of(P.sink_k, P.tail_k, j) + 32 * c + 8 * kg);
        bk[k][c] = (u32x4_t){t.x, t.y, t.z, t.w};
      }
    }
  }
  // V: channels 2 lane, 2 lane + 1 of tokens wave + 4 m (a wave-uniform test)
  uint32_t vv[kBfVPerThread];
#pragma unroll
  for (int m = 0; m < kBfVPerThread; ++m) {
    const int j = wave + 4 * m;
    vv[m] = 0u;
    if (j < nb) vv[m] = reinterpret_cast<const uint32_t*>(row_of(P.sink_v, P.tail_v, j))[lane];
  }
  // logits: lanes 0..15 hold token 16 tile + lane, heads 0..3 in acc[0..3]
  const float sigma = P.softmax_scale;
  float t[kBfTilesPerWave][4];
  float mx[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
  for (int k = 0; k < kBfTilesPerWave; ++k) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) acc = mfma<true>(aq[c], bk[k][c], acc);
    const bool live = lane < 16 && 16 * (wave + 4 * k) + lane < nb;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      t[k][g] = live ? sigma * acc[g] : kNegInf;
      mx[g] = fmaxf(mx[g], t[k][g]);
    }
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) mx[g] = max16(mx[g]);  // lanes 0..15: this wave's maximum
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) sm.red[wave][g] = mx[g];
  }
  __syncthreads();
  float m[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) m[g] = fmaxf(fmaxf(sm.red[0][g], sm.red[1][g]), fmaxf(sm.red[2][g], sm.red[3][g]));
  // p of the wave's tokens into LDS [token][head]; l per wave
  float* flat = &sm.logit[0][0];
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kBfTilesPerWave; ++k) {
    float pv[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      pv[g] = t[k][g] == kNegInf ? 0.0f : __expf(t[k][g] - m[g]);
      ls[g] += pv[g];
    }
    const int j = 16 * (wave + 4 * k) + lane;
    if (lane < 16 && j < nb) reinterpret_cast<float4*>(flat)[j] = make_float4(pv[0], pv[1], pv[2], pv[3]);
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) ls[g] = sum16(ls[g]);
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) sm.lsum[wave][g] = ls[g];
  }
  __syncthreads();
  // PV over the tokens wave + 4 m
  float o[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
  auto pv_token = [&](int j, uint32_t w) {
    const float4 p = reinterpret_cast<const float4*>(flat)[j];
    const float v0 = bf16_lo(w), v1 = bf16_hi(w);
    o[0][0] = fmaf(p.x, v0, o[0][0]); o[0][1] = fmaf(p.x, v1, o[0][1]);
    o[1][0] = fmaf(p.y, v0, o[1][0]); o[1][1] = fmaf(p.y, v1, o[1][1]);
    o[2][0] = fmaf(p.z, v0, o[2][0]); o[2][1] = fmaf(p.z, v1, o[2][1]);
    o[3][0] = fmaf(p.w, v0, o[3][0]); o[3][1] = fmaf(p.w, v1, o[3][1]);
  };
#pragma unroll
  for (int mm = 0; mm < kBfVPerThread; ++mm) {
    const int j = wave + 4 * mm;
    if (j < nb) pv_token(j, vv[mm]);
  }
  for (int j = wave + 4 * kBfVPerThread; j < nb; j += 4)        // spans longer than 144 tokens
    pv_token(j, reinterpret_cast<const uint32_t*>(row_of(P.sink_v, P.tail_v, j))[lane]);
  float* so = flat + 1024;                           // [wave][head][128], past the p values
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<float2*>(so + (wave * 4 + g) * kD + 2 * lane) = make_float2(o[g][0], o[g][1]);
  __syncthreads();
  const int head = tid >> 6, d = (tid & 63) * 2;
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    o0 += so[(w * 4 + head) * kD + d];
    o1 += so[(w * 4 + head) * kD + d + 1];
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
// same functions of the rotated values. With exp_codes / exp_scales (the
// debug entry bdfp4_decode_query_codes, never the decode itself) the codes
// and scale codes of each term are also written out: codes [term][64] (byte
// i = elements 2i, 2i + 1), scales [term][nb].
template <bool kMx, int kTerms, bool kExport = false>
__device__ __forceinline__ void query_prologue(const DecodeLaunch& P, uint32_t qw, float2 mu, Smem& sm, int g,
                                               int i, uint8_t* exp_codes = nullptr, uint8_t* exp_scales = nullptr) {
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
      // the codes and the E8M0 code (in [0, 254]; an all-zero block's codes
      // are zero whatever its scale) are the scaled FP4 MFMA's A operand
      sm.qcode[term][g][i] = (uint8_t)pk;
      if ((i & 15) == 0) sm.qsc[term][g][i >> 4] = (uint32_t)((take_lo ? elo : ehi) + 127);
      if (kExport) {
        exp_codes[term * 64 + i] = (uint8_t)pk;
        if ((i & 15) == 0) exp_scales[term * 4 + (i >> 4)] = (uint8_t)((take_lo ? elo : ehi) + 127);
      }
    } else {
      // 16-element block = 8 lanes
      a = max8(a);
      const uint32_t sc = e4m3_encode(div6(a));
      s = e4m3_value(sc);
      quant_block<2, false>(xx, s, &pk);
      if (kExport) {
        exp_codes[term * 64 + i] = (uint8_t)pk;
        if ((i & 7) == 0) exp_scales[term * 8 + (i >> 3)] = (uint8_t)sc;
      }
    }
    float deq[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t nib = (pk >> (4 * k)) & 0xFu;
      const float gv = __fmul_rn(e2m1_grid(nib & 7u), s);
      deq[k] = (nib & 8u) ? -gv : gv;
    }
    if (!kMx) reinterpret_cast<uint32_t*>(&sm.qhat[term][g][0])[i] = op16<kMx>(deq[0]) | (op16<kMx>(deq[1]) << 16);
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

// Half h of a K page (tiles 4 h .. 4 h + 3, and the page's scales) or V page
// (chunks 2 h, 2 h + 1 and their scales) into the page buffer, for the
// half-page stream of fp4_wg; the other half of the buffer is never written
// or read, so it takes no registers.
template <bool kMx>
__device__ __forceinline__ void load_k_half(KPage& k, const DecodeLaunch& P, size_t blk, int lane, int half) {
  const uint4* kc = reinterpret_cast<const uint4*>(P.k_codes + blk * 8192) + lane;
#pragma unroll
  for (int t = 0; t < 4; ++t) k.code[4 * half + t] = kc[(4 * half + t) * 64];
  if (kMx) {
    const uint2 t2 = *reinterpret_cast<const uint2*>(P.k_scales + blk * 512 + lane * 8);
    k.sc = make_uint4(t2.x, t2.y, 0u, 0u);
  } else {
    k.sc = *reinterpret_cast<const uint4*>(P.k_scales + blk * 1024 + lane * 16);
  }
}
template <bool kMx>
__device__ __forceinline__ void load_v_half(VPage& v, const DecodeLaunch& P, size_t blk, int lane, int half) {
  const uint4* vc = reinterpret_cast<const uint4*>(P.v_codes + blk * 8192 + lane * 32);
  const int kg = lane >> 4, n = lane & 15;
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int c = 2 * half + cc;
    v.code[2 * c] = vc[c * 128];
    v.code[2 * c + 1] = vc[c * 128 + 1];
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

// What a wave of an FP4 workgroup reads before anything else, issued at the
// start of the kernel so that these loads, the sequence length and the
// kernel arguments share one memory round trip instead of following each
// other: lane i's block-table entry of the wave's partition (page p0 + i,
// for i < pages_per_partition inside the table's row, else 0), the wave's
// query row (two bf16 per lane) and the key means (from a zero row without
// smoothing, so the load is unconditional and no branch waits on it).
struct Early {
  int pid;
  uint32_t qw;
  float2 mu;
};

// Key means of a call without key smoothing: zero (static storage), so the
// key-mean load is the same unconditional load either way.
__device__ float g_zero_means[kD];

__device__ __forceinline__ Early early_loads(const DecodeLaunch& P, int b, int h, int sp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Early E;
  const int pg = (4 * sp + wave) * P.ppp + lane;
  E.pid = (lane < P.ppp && pg < P.max_pages_per_seq) ? P.block_tables[(size_t)b * P.max_pages_per_seq + pg] : 0;
  const uint16_t* qrow = P.q + ((size_t)b * P.hq + h * kGroup + wave) * kD;
  E.qw = reinterpret_cast<const uint32_t*>(qrow)[lane];
  const float* mp = P.key_smoothing ? P.key_shift + h * kD : g_zero_means;
  E.mu = reinterpret_cast<const float2*>(mp)[lane];
  return E;
}

// The four FP4 partitions 4 sp + w (w = wave) of one (sequence, KV head):
// each wave streams its own pages_per_partition consecutive pages through
// pass 1, its own maximum and pass 2 with no workgroup barrier in between
// (kSlots = 1, 2 or 4 page slots per kind, the plan's pages_per_partition
// rounded up, so that no slot is loaded for a page the plan never has);
// the four (m, l, o) are then merged by log-sum-exp in LDS and stored as the
// workgroup's partial (returned; the caller stores it). With bf16 the
// workgroup first computes the (sequence, KV head)'s BF16 partition, then
// requests its first K pages, and folds the partition into the same partial.
template <bool kMx, int kTerms, bool kUnder, bool kRunMax, int kSlots, bool kChan>
__device__ Partial fp4_wg(const DecArgs& A, Smem& sm, int b, int h, int sp, int L, bool bf16, const Early& E) {
  const DecodeLaunch& P = A.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_full = L / kPage;
  const int p0 = (4 * sp + wave) * P.ppp;                       // first page of this wave's partition
  const int npg = max(0, min(n_full, p0 + P.ppp) - p0);         // its pages, 0 .. pages_per_partition
  const size_t hkv = P.hkv;

  // physical pages of the partition: lane i < npg holds page p0 + i (read
  // before the sequence length was known; lanes past npg are dropped here)
  int pid = lane < npg ? E.pid : 0;
  const bool bad_lane = lane < npg && (pid < 0 || pid >= P.num_pages);
  const bool bad = __ballot(bad_lane) != 0;
  if (bad_lane) pid = 0;                                        // keep addresses inside the cache
  auto blk_of = [&](int pi) -> size_t { return (size_t)__builtin_amdgcn_readlane(pid, pi) * hkv + h; };

  // the query row of this wave and the key means
  const uint32_t qw = E.qw;
  const float2 mu = E.mu;
  if (tid < 8) sm.rcp[tid] = rcp_significand((uint32_t)tid);
  {
    uint32_t* pz = &sm.pst[0][0][0];       // rows 4 .. 15 of every wave's staging tile
    for (int i = tid; i < 4 * 192; i += 256) pz[(i / 192) * 256 + 64 + (i % 192)] = 0u;
  }
  // The wave reads a stream of 2 kSlots slots, K pages 0..kSlots-1 then V
  // pages 0..kSlots-1 (kHalf, every kernel but the channel-scale ones with 1
  // or 2 slots: half pages, 4 kSlots slots, see there), keeping the next
  // slot in flight while one is used:
  // K page i lands in kb[i % 2], V page j in vb[j % 2], and the load of a
  // slot is issued once the slot two before it (same buffer) has been used
  // (with one page per partition, K and V page 0 are both requested at the
  // start). One page in flight per wave measured faster than two, and half
  // a page (kHalf) faster still: with 8 waves per CU the memory pipe is
  // already full, and deeper queues only delay the waves dispatched second. The loads are unconditional (a slot
  // of a page past npg, in the partition that ends the sequence, reads
  // physical page 0, which always exists, and is never used) so the compiler
  // can count the loads in flight exactly and wait only for the slot about
  // to be used.
  KPage kb0, kb1;
  VPage vb0, vb1;
  // A workgroup that also computes the BF16 partition does so before it
  // requests its first K pages, so that waiting for the partition's rows
  // does not also wait for those pages (every workgroup of the grid requests
  // its first pages at once, and they take several µs to drain)
  constexpr bool kHalf = !kChan || kSlots == 4;          // half pages (see the stream below)
  Partial bfp;
  if (bf16) {
    bfp = bf16_partition(A, sm, b, h, L, n_full);
    if constexpr (kHalf) load_k_half<kMx>(kb0, P, blk_of(0), lane, 0);
    else load_k<kMx>(kb0, P, blk_of(0), lane);
  } else {
    if constexpr (kHalf) load_k_half<kMx>(kb0, P, blk_of(0), lane, 0);
    else load_k<kMx>(kb0, P, blk_of(0), lane);
  }
  if constexpr (kHalf)
    load_k_half<kMx>(kb1, P, blk_of(0), lane, 1);
  else if constexpr (kSlots == 1)
    load_v<kMx>(vb0, P, blk_of(0), lane);
  else
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
    if (!kMx && (qr & 1) < kTerms) {
      const uint4 t = *reinterpret_cast<const uint4*>(&sm.qhat[qr & 1][qr >> 1][32 * kg + 8 * c]);
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
    aq[c] = v;
  }
  // MXFP4: the query's E2M1 codes (channels 32 kg .. +32) and E8M0 code,
  // one scaled FP4 MFMA per 16-token tile
  u32x4_t aq4 = {0u, 0u, 0u, 0u};
  uint32_t sa4 = 127u;
  if (kMx && (qr & 1) < kTerms) {
    const uint4 t = *reinterpret_cast<const uint4*>(&sm.qcode[qr & 1][qr >> 1][16 * kg]);
    aq4 = (u32x4_t){t.x, t.y, t.z, t.w};
    sa4 = sm.qsc[qr & 1][qr >> 1][kg];
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
  auto k_page = [&](const KPage& cur, int pi, int t_lo = 0, int t_hi = 8) {
    const int skip = pi == 0 ? sink_tiles : 0;                  // uniform
    float pa = kNegInf, pb = kNegInf;
    // channel key geometry: the page's 1 KiB of scales, [token block][channel],
    // in this wave's LDS (the wave reads it back in order); tile t takes the
    // 32 scales of its lanes' channels 32 kg .. +32 from block t
    if (kChan && t_lo == 0) reinterpret_cast<uint4*>(&sm.ksc[wave][0])[lane] = cur.sc;
#pragma unroll
    for (int t = t_lo; t < t_hi; ++t) {
      const int local = pi * kPage + t * 16;                    // first token of the tile - 128 p0
      u32x4_t bk[4];
      f32x4_t acc = acc0;
      if (kMx) {
        // the page's codes are the B operand as they are; byte t & 3 of
        // scale word t >> 2 is this lane's (token, channel block) E8M0 code
        const uint4 cw = cur.code[t];
        acc = mfma_fp4_scaled_byte(t & 3, aq4, sa4, (u32x4_t){cw.x, cw.y, cw.z, cw.w}, word_of(cur.sc, t >> 2), acc);
      } else if (kChan) {
        // the scale of channels 32 kg + 8 c + 2 b, +1 is the byte pair
        // 8 c + 2 b of the lane's 32: dword 2 c + (b >> 1), half b & 1
        const uint4 s_lo = *reinterpret_cast<const uint4*>(&sm.ksc[wave][32 * t + 8 * kg]);
        const uint4 s_hi = *reinterpret_cast<const uint4*>(&sm.ksc[wave][32 * t + 8 * kg + 4]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t cw = word_of(cur.code[t], c);
          const uint32_t sw0 = word_of(c < 2 ? s_lo : s_hi, (2 * c) & 3);
          const uint32_t sw1 = word_of(c < 2 ? s_lo : s_hi, (2 * c + 1) & 3);
          bk[c] = (u32x4_t){u32_of(grid_f16_pair(cw, 0) * e4m3_pair_f16(sw0, false)),
                            u32_of(grid_f16_pair(cw, 1) * e4m3_pair_f16(sw0, true)),
                            u32_of(grid_f16_pair(cw, 2) * e4m3_pair_f16(sw1, false)),
                            u32_of(grid_f16_pair(cw, 3) * e4m3_pair_f16(sw1, true))};
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
      if (!kMx) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = mfma<kMx>(aq[c], bk[c], acc);
      }
      const bool sink = t < skip;                               // uniform: a sink tile of page 0
      const float ta = sink ? kNegInf : __fadd_rn(acc[0], acc[1]);
      const float tb = sink ? kNegInf : __fadd_rn(acc[2], acc[3]);
      lg_a[local] = ta;
      lg_b[local] = tb;
      pa = __builtin_fmaxf(pa, ta);
      pb = __builtin_fmaxf(pb, tb);
      if (kRunMax) {
        // the block's maximum per head (rows of 16 lanes = the tile's tokens)
        const float xa = max16(ta), xb = max16(tb);
        if (lane < 32 && row == 0) {
          sm.tmax[wave][2 * hp][(pi * kPage + t * 16) >> 4] = xa;
          sm.tmax[wave][2 * hp + 1][(pi * kPage + t * 16) >> 4] = xb;
        }
      }
    }
    ma = __builtin_fmaxf(ma, pa);
    mb = __builtin_fmaxf(mb, pb);
  };
  static_assert(kMaxPpw == 4 && (kSlots == 1 || kSlots == 2 || kSlots == 4),
                "the stream below is unrolled for 1, 2 or 4 pages");
  if constexpr (kHalf) {
    // half pages: slot 2 p + h is half h of K page p (buffer kb_h), then
    // half h of V page p (vb_h); the load of a slot follows the use of the
    // slot two before it, in the same buffer. Against whole pages this holds
    // one page of K and V at a time instead of two (NVFP4 160 against 167
    // VGPRs: the room the compacted grid needs; MXFP4 163 against 184: 3
    // waves per SIMD instead of 2), and measured faster at 128K (NVFP4
    // 0.4-0.8 us with bit-identical output, MXFP4 1.4-1.7 us) and for the
    // 32K layer's 2 pages per partition (0.3-0.9 us, bit-identical). With
    // channel key scales (the page's scales staged in LDS by the first half)
    // it gains with 4 slots (the batch of 16: 57.6 -> 55.2 us) and loses with
    // 2 (32K: +0.8 us), so those kernels keep whole pages.
#pragma unroll
    for (int p = 0; p < kSlots; ++p) {
      if (npg > p) k_page(kb0, p, 0, 4);
      if (p < kSlots - 1) load_k_half<kMx>(kb0, P, blk_of(p + 1), lane, 0);
      else load_v_half<kMx>(vb0, P, blk_of(0), lane, 0);
      if (npg > p) k_page(kb1, p, 4, 8);
      if (p < kSlots - 1) load_k_half<kMx>(kb1, P, blk_of(p + 1), lane, 1);
      else load_v_half<kMx>(vb1, P, blk_of(0), lane, 1);
    }
  } else if constexpr (kSlots == 1) {
    if (npg > 0) k_page(kb0, 0);
  } else if constexpr (kSlots == 2) {
    if (npg > 0) k_page(kb0, 0);
    load_v<kMx>(vb0, P, blk_of(0), lane);
    if (npg > 1) k_page(kb1, 1);
    load_v<kMx>(vb1, P, blk_of(1), lane);
  } else {
    if (npg > 0) k_page(kb0, 0);
    load_k<kMx>(kb0, P, blk_of(2), lane);
    if (npg > 1) k_page(kb1, 1);
    load_k<kMx>(kb1, P, blk_of(3), lane);
    if (npg > 2) k_page(kb0, 2);
    load_v<kMx>(vb0, P, blk_of(0), lane);
    if (npg > 3) k_page(kb1, 3);
    load_v<kMx>(vb1, P, blk_of(1), lane);
  }
  // debug export of the raw logits q . mu + q_hat . k_hat of this partition
  // (bdfp4_decode_attention_logits; null in every other call)
  if (P.dbg_logits != nullptr) {
    float* dst = P.dbg_logits + (size_t)(b * P.hkv + h) * kGroup * P.dbg_stride + (size_t)p0 * kPage;
    for (int g = 0; g < kGroup; ++g)
      for (int j = lane; j < npg * kPage; j += 64) dst[(size_t)g * P.dbg_stride + j] = lgw[g * kWaveTok + j];
  }
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
  float mrun = kNegInf;              // running-max variant: maximum of the blocks before this chunk
  f32x4_t acco[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acco[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  auto v_page = [&](const VPage& vcur, int pi, int c_lo = 0, int c_hi = 4) {
#pragma unroll
    for (int ch = c_lo; ch < c_hi; ++ch) {
      // p' = c exp(sigma (t - m)) of tokens 2 pj, 2 pj + 1 of the chunk, head ph
      const float2 tt = *reinterpret_cast<const float2*>(lrow + pi * kPage + ch * 32);
      // the reference maximum: the partition's, or (running-max variant) the
      // maximum over this partition's 16-token blocks up to this lane's block,
      // with w = exp(sigma (mref - m)) weighting its P back to the partition's
      float mref = mh, w = 1.0f;
      if (kRunMax) {
        const int blk = (pi * kPage + ch * 32) >> 4;
        const float mA = __builtin_fmaxf(mrun, sm.tmax[wave][ph][blk]);
        const float mB = __builtin_fmaxf(mA, sm.tmax[wave][ph][blk + 1]);
        mref = pj < 8 ? mA : mB;
        mrun = mB;
        w = __builtin_amdgcn_exp2f(__fmul_rn(__fsub_rn(mref, mh), ks));   // mref = -inf gives 0
      }
      const bool live = !kRunMax || mref != kNegInf;             // a block of sink slots only
      const float x0 = live ? __fmul_rn(cf, __builtin_amdgcn_exp2f(__fmul_rn(__fsub_rn(tt.x, mref), ks))) : 0.0f;
      const float x1 = live ? __fmul_rn(cf, __builtin_amdgcn_exp2f(__fmul_rn(__fsub_rn(tt.y, mref), ks))) : 0.0f;
      lacc = kRunMax ? __fadd_rn(lacc, __fmul_rn(__fadd_rn(x0, x1), w)) : __fadd_rn(lacc, __fadd_rn(x0, x1));
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
      } else if (kRunMax) {
        // P_hat w, rounded once to f16 (P_hat = s e2m1 is exact in float32)
        const e2m1_f32x2_t g = e2m1_grid_pair(byte, 0);
        const _Float16 h0 = (_Float16)__fmul_rn(__fmul_rn(g[0], sv), w);
        const _Float16 h1 = (_Float16)__fmul_rn(__fmul_rn(g[1], sv), w);
        word = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
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
  if constexpr (kHalf) {
#pragma unroll
    for (int p = 0; p < kSlots; ++p) {
      if (npg > p) v_page(vb0, p, 0, 2);
      if (p < kSlots - 1) load_v_half<kMx>(vb0, P, blk_of(p + 1), lane, 0);
      if (npg > p) v_page(vb1, p, 2, 4);
      if (p < kSlots - 1) load_v_half<kMx>(vb1, P, blk_of(p + 1), lane, 1);
    }
  } else if constexpr (kSlots == 1) {
    if (npg > 0) v_page(vb0, 0);
  } else if constexpr (kSlots == 2) {
    if (npg > 0) v_page(vb0, 0);
    if (npg > 1) v_page(vb1, 1);
  } else {
    if (npg > 0) v_page(vb0, 0);
    load_v<kMx>(vb0, P, blk_of(2), lane);
    if (npg > 1) v_page(vb1, 1);
    load_v<kMx>(vb1, P, blk_of(3), lane);
    if (npg > 2) v_page(vb0, 2);
    if (npg > 3) v_page(vb1, 3);
  }
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
  // ---- log-sum-exp merge of the four partitions, and of the BF16 partition
  // when this workgroup computed it: thread (head, channel pair). The FP4
  // part is formed against its own maximum as without the BF16 partition,
  // then both parts are weighted against the overall maximum (a factor of
  // exactly 1 for the larger one).
  const float sigma = P.softmax_scale;
  const float invc = 1.0f / cf;      // exact (c is a power of two)
  float mm[4], ll[4], wgt[4][4], fa[4], fb[4];
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
    const float mf = sigma * M;                  // FP4 maximum (sigma included; -inf if empty)
    const float mb = bf16 ? bfp.m[g] : kNegInf;  // BF16 maximum
    const float mx = fmaxf(mf, mb);
    fa[g] = M == kNegInf ? 0.0f : __expf(mf - mx);
    fb[g] = mb == kNegInf ? 0.0f : __expf(mb - mx);
    mm[g] = mx;
    ll[g] = fmaf(fa[g], l * invc, bf16 ? fb[g] * bfp.l[g] : 0.0f);
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
  const float fah = head == 0 ? fa[0] : (head == 1 ? fa[1] : (head == 2 ? fa[2] : fa[3]));
  const float fbh = head == 0 ? fb[0] : (head == 1 ? fb[1] : (head == 2 ? fb[2] : fb[3]));
  // with rotated values the FP4 part is in the rotated domain: the BF16
  // partition (raw values) is rotated into it before the two are added
  float bo0 = bf16 ? bfp.o0 : 0.0f, bo1 = bf16 ? bfp.o1 : 0.0f;
  if (bf16 && P.rotate_v) wave_rotate2(bo0, bo1);       // uniform per workgroup
  o0 = fmaf(fah, o0 * invc, bf16 ? fbh * bo0 : 0.0f);
  o1 = fmaf(fah, o1 * invc, bf16 ? fbh * bo1 : 0.0f);
  const bool poisoned = (sm.bad[0] | sm.bad[1] | sm.bad[2] | sm.bad[3]) != 0;
  const float nan = __builtin_nanf("");
  Partial r;
  r.o0 = poisoned ? nan : o0;
  r.o1 = poisoned ? nan : o1;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    r.m[g] = poisoned ? 0.0f : mm[g];
    r.l[g] = poisoned ? 1.0f : ll[g];
  }
  return r;
}

// FP4 workgroups of a sequence of length L (0 for an invalid length, whose
// rows column 0 poisons, or for a sequence without a full page).
__device__ __forceinline__ int seq_fp4_wgs(const DecodeLaunch& P, int L) {
  if (L < 1 || L > P.max_seq_len || L / kPage > P.max_pages_per_seq) return 0;
  const int n_full = L / kPage;
  return n_full > 0 ? fp4_wgs((n_full + P.ppp - 1) / P.ppp) : 0;
}
// A compacted launch: the grid of every (sequence, KV head, column) is
// larger than the chip holds at once. Workgroups are dispatched in index
// order, and a slot that a workgroup without work frees is not taken by the
// next one until workgroups with work end, so the columns that only the
// longest sequences have would start late and end the launch (measured on
// the batch of 16: columns 6-7 entered at 2-35 us). Workgroup j instead
// serves the j-th unit with work, as the virtual index col * B Hkv + bh that
// an uncompacted grid would give it: column 0 for every sequence (it also
// computes the BF16 partition, or the NaN rows of an invalid sequence), then
// by column the columns c >= 1 that are not a sequence's last, then by
// column each sequence's last column (c >= 1), all in sequence order, KV
// head j mod Hkv (so a head's workgroups keep their place in the dispatch
// rotation). The last columns hold 1..ppp x 4 pages, the others all of
// them: dispatched last, the lighter units are the ones a compute unit
// takes as its third workgroup (the batch of 16: 46.0-47.8 against
// 48.1-49.7 us with the last columns in column order). Every wave computes
// the same mapping from the sequence lengths (up to kCompactChunks x 64
// sequences, in registers). Returns -1 for a workgroup past the units with
// work.
constexpr int kCompactChunks = 4;
__device__ __forceinline__ int compact_vj(const DecodeLaunch& P, int j) {
  const int lane = threadIdx.x & 63;
  const int BH = P.batch * P.hkv;
  int u = j / P.hkv;
  const int h = j - u * P.hkv;
  if (u < P.batch) return j;
  u -= P.batch;
  int nw[kCompactChunks];
#pragma unroll
  for (int k = 0; k < kCompactChunks; ++k) {
    const int b = 64 * k + lane;
    nw[k] = b < P.batch ? seq_fp4_wgs(P, P.seq_lens[b]) : 0;
  }
  const int wgs = fp4_wgs(P.max_parts);
  for (int last = 0; last < 2; ++last) {
    for (int c = 1; c < wgs; ++c) {
#pragma unroll
      for (int k = 0; k < kCompactChunks; ++k) {
        const bool has = last ? nw[k] == c + 1 : nw[k] > c + 1;   // column c is (not) the sequence's last
        const uint64_t m = __ballot(has);
        const int cnt = __popcll(m);
        if (u < cnt) {
          const int below =
              __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
          const uint64_t pick = __ballot(has && below == u);
          return c * BH + (64 * k + __builtin_ctzll(pick)) * P.hkv + h;
        }
        u -= cnt;
      }
    }
  }
  return -1;
}

// Workgroup j works for (sequence, KV head) bh = j % (B Hkv) in grid column
// c = j / (B Hkv) (j the virtual index: of compact_vj in a compacted launch,
// rotated by one column under bf16_last). A launch whose grid has room for
// one more column (split_bf16: it still fits the chip at the kernel's
// occupancy) gives every BF16 partition (sink + tail) a workgroup of its own
// in column 0 (the first B Hkv workgroups of the grid, or under bf16_last the
// last), which runs beside the FP4 workgroups instead of delaying one of
// them; FP4 workgroup
// sp then sits in column sp + 1. Otherwise FP4 workgroup sp sits in column
// sp, and workgroup 0 also computes the BF16 partition, before it requests
// its first K pages, and folds it into its partial. FP4 workgroup sp stores
// its partial in slot sp, a BF16 workgroup in slot nwg (nwg = the sequence's
// FP4 workgroups), and each takes the (sequence, KV head)'s ticket; the last
// merges all partials (the BF16 one as the merge's extra slot). Without BF16
// workgroups a sequence with one FP4 workgroup writes its o / l directly (no
// partial, ticket or merge: the merge of a single partial is that quotient).
// A sequence without a full page has only the BF16 partition, written
// straight to the output by column 0.
// 3 waves per SIMD (at most 168 VGPRs) for every kernel that streams half
// pages, without spilling; 2 for the whole-page channel-key-scale kernels.
template <bool kMx, int kTerms, bool kUnder, bool kRunMax, int kSlots, bool kChan>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kChan && kSlots != 4 ? 2 : 3)))
decode_kernel(DecArgs A) {
  __shared__ __align__(16) Smem sm;
  const DecodeLaunch& P = A.L;
  const MergeCtx C = merge_ctx(A);
  const int BH = P.batch * P.hkv;
  int vj = (int)blockIdx.x;                                // grid position (compacted: of the j-th unit with work)
  if (P.bf16_last) {
    // the FP4 columns take workgroups 0 .. nfp - 1, the BF16 column the rest
    const int nfp = (int)gridDim.x - BH;
    vj = vj < nfp ? vj + BH : vj - nfp;
  }
  if (P.compact) {
    vj = __builtin_amdgcn_readfirstlane(compact_vj(P, vj));
    if (vj < 0) return;
  }
  const int bh = vj % BH, col = vj / BH;
  const int b = bh / P.hkv, h = bh - b * P.hkv;
  const int split = P.split_bf16;                          // 0 or 1, uniform per launch
  const int sp = col - split;                              // FP4 workgroup of this column (-1: BF16)
  const Early E = early_loads(P, b, h, sp < 0 ? 0 : sp);
  const int L = P.seq_lens[b];
  if (L < 1 || L > P.max_seq_len || L / kPage > P.max_pages_per_seq) {
    if (col == 0) poison_rows(P.out, P.hq, b, h);
    return;
  }
  const int n_full = L / kPage;
  const int nwg = n_full > 0 ? fp4_wgs((n_full + P.ppp - 1) / P.ppp) : 0;   // FP4 workgroups of this sequence
  if (nwg == 0 || sp < 0) {
    // the BF16 partition alone: the whole attention of a sequence without a
    // full page, else its own workgroup (one call site for both)
    if (col != 0) return;
    Partial r = bf16_partition(A, sm, b, h, L, n_full);
    if (nwg == 0) {
      const int head = threadIdx.x >> 6, d = 2 * (threadIdx.x & 63);
      const float l = of_head(r.l[0], r.l[1], r.l[2], r.l[3], head);
      float* out = P.out + ((size_t)b * P.hq + h * kGroup + head) * kD + d;
      *reinterpret_cast<float2*>(out) = make_float2(r.o0 / l, r.o1 / l);
      return;
    }
    // with rotated values its o enters the merge in the rotated domain, like
    // the FP4 partials
    if (P.rotate_v) wave_rotate2(r.o0, r.o1);            // uniform per workgroup
    write_partial(partial_writer(C, bh, nwg), r);
  } else {
    if (sp >= nwg) return;
    const Partial mine =
        fp4_wg<kMx, kTerms, kUnder, kRunMax, kSlots, kChan>(A, sm, b, h, sp, L, split == 0 && sp == 0, E);
    if (split == 0 && nwg == 1) {
      const int head = threadIdx.x >> 6, d = 2 * (threadIdx.x & 63);
      const float l = of_head(mine.l[0], mine.l[1], mine.l[2], mine.l[3], head);
      float o0 = mine.o0, o1 = mine.o1;
      if (P.rotate_v) wave_rotate2(o0, o1);              // uniform per workgroup
      float* out = P.out + ((size_t)b * P.hq + h * kGroup + head) * kD + d;
      *reinterpret_cast<float2*>(out) = make_float2(o0 / l, o1 / l);
      return;
    }
    write_partial(partial_writer(C, bh, sp), mine);
  }
  uint32_t* ticket = C.counters + (size_t)bh * C.counter_stride;
  if (take_ticket(ticket, 1, &sm.tick) == nwg - 1 + split) {
    merge_out(C, b, h, nwg, P.rotate_v != 0, split ? nwg : -1);
    reset_ticket(ticket);
  }
}

// ------------------------------------------------------------ debug: the decode's query codes

// Workgroup (sequence, KV head), wave g = query head g of the group: the
// decode's own query prologue on each query row, its codes and scale codes
// written out ([row][term][64] and [row][term][nb], row = b * hq + query head).
template <bool kMx, int kTerms>
__global__ void __launch_bounds__(256) query_codes_kernel(DecodeLaunch P, uint8_t* codes, uint8_t* scales) {
  __shared__ __align__(16) Smem sm;
  const int bh = blockIdx.x, b = bh / P.hkv, h = bh - b * P.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t row = (size_t)b * P.hq + h * kGroup + wave;
  const uint32_t qw = reinterpret_cast<const uint32_t*>(P.q + row * kD)[lane];
  const float2 mu = make_float2(0.0f, 0.0f);
  constexpr int nb = kMx ? 4 : 8;
  query_prologue<kMx, kTerms, true>(P, qw, mu, sm, wave, lane, codes + row * kTerms * 64,
                                    scales + row * kTerms * nb);
}

hipError_t launch_query_codes(const DecodeLaunch& L, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const dim3 grid((unsigned)(L.batch * L.hkv)), block(256u);
  if (L.mx) {
    if (L.terms == 2) hipLaunchKernelGGL((query_codes_kernel<true, 2>), grid, block, 0, stream, L, codes, scales);
    else hipLaunchKernelGGL((query_codes_kernel<true, 1>), grid, block, 0, stream, L, codes, scales);
  } else {
    if (L.terms == 2) hipLaunchKernelGGL((query_codes_kernel<false, 2>), grid, block, 0, stream, L, codes, scales);
    else hipLaunchKernelGGL((query_codes_kernel<false, 1>), grid, block, 0, stream, L, codes, scales);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ allocation-free entry

// Workspace of bdfp4_decode_attention_noalloc: device memory of fixed size
// in this file, one copy per GPU, held until the process ends. Host code
// reaches it only through the address hipGetSymbolAddress returns for the
// current device (the array's name in host code is not a device address).
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
bool g_scratch_zeroed[kMaxDevices];

__global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  if (!g_scratch_zeroed[dev]) {
    // the ticket words must start at zero (every call leaves them zero);
    // a fill kernel rather than a memset, so a captured first call holds
    // only kernel nodes
    const int n = (int)(kTicketBytes / sizeof(uint32_t));
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256u), 0, stream,
                       static_cast<uint32_t*>(g_scratch_ptr[dev]), n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_zeroed[dev] = true;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// Compute units of the current device (cached per device).
static hipError_t device_cus(int* cus) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return hipSuccess;
}

// One decode instantiation: BF16 partition workgroups of their own when one
// more grid column still fits the chip at the kernel's occupancy (with a full
// chip the extra column would wait for a free slot and end the kernel later;
// the occupancy, from its registers and LDS, is asked once per
// instantiation), then the launch.
template <bool kMx, int kTerms, bool kUnder, bool kRunMax, int kSlots, bool kChan>
static hipError_t launch_one(DecArgs A, int cus, hipStream_t stream) {
  static std::atomic<int> occupancy{0};
  int per_cu = occupancy.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, decode_kernel<kMx, kTerms, kUnder, kRunMax, kSlots, kChan>, 256, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    occupancy.store(per_cu, std::memory_order_relaxed);
  }
  const long long bh = (long long)A.L.batch * A.L.hkv;
  const int wgs = fp4_wgs(A.L.max_parts);
  A.L.split_bf16 = wgs >= 2 && bh * (wgs + 1) <= (long long)per_cu * cus ? 1 : 0;
  // a grid the chip does not hold at once takes its units with work first
  A.L.compact = !A.L.split_bf16 && wgs >= 2 && bh * wgs > (long long)per_cu * cus && A.L.batch <= 64 * kCompactChunks
                    ? 1 : 0;
  // With more FP4 workgroups than compute units, a BF16 workgroup shares its
  // compute unit with two FP4 workgroups; dispatched last it is the youngest
  // there, so its issue comes after theirs rather than before (the 128K
  // layer: 34.9-35.0 against 35.4-35.6 us). With one FP4 workgroup per
  // compute unit it stays first (the 32K layer: 0.15-0.3 us faster so).
  A.L.bf16_last = A.L.split_bf16 && bh * wgs > cus ? 1 : 0;
  // the FP4 workgroups of the longest sequence, after a column of BF16
  // partition workgroups when the launch has them
  const dim3 grid((unsigned)(bh * (wgs + A.L.split_bf16))), block(256u);
  hipLaunchKernelGGL((decode_kernel<kMx, kTerms, kUnder, kRunMax, kSlots, kChan>), grid, block, 0, stream, A);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  DecArgs A;
  A.L = L;
  int cus = 0;
  const hipError_t ce = device_cus(&cus);
  if (ce != hipSuccess) return ce;
  const bool under = L.p_mode == 4;
  // page slots per kind: the plan's pages_per_partition rounded up to 1, 2, 4
  const int slots = L.ppp <= 1 ? 1 : (L.ppp == 2 ? 2 : 4);
#define BDFP4_LAUNCH_S(MX, T, U, R, C)                                               \
  return slots == 1   ? launch_one<MX, T, U, R, 1, C>(A, cus, stream)                  \
         : slots == 2 ? launch_one<MX, T, U, R, 2, C>(A, cus, stream)                  \
                      : launch_one<MX, T, U, R, 4, C>(A, cus, stream)
#define BDFP4_LAUNCH(MX, T, U) BDFP4_LAUNCH_S(MX, T, U, false, false)
#define BDFP4_LAUNCH_CH(T, U) BDFP4_LAUNCH_S(false, T, U, false, true)
  if (L.k_chan) {
    // the host admits the channel key geometry for NVFP4 pages without the
    // running-maximum variant only
    if (L.mx || L.run_max) return hipErrorInvalidValue;
    if (L.terms == 2) { if (under) BDFP4_LAUNCH_CH(2, true); else BDFP4_LAUNCH_CH(2, false); }
    else { if (under) BDFP4_LAUNCH_CH(1, true); else BDFP4_LAUNCH_CH(1, false); }
  } else if (L.run_max) {
    // the host admits the running-max variant only for NVFP4, two query
    // terms and amax2_or_amax6 P
    if (L.mx || L.terms != 2 || !under) return hipErrorInvalidValue;
    BDFP4_LAUNCH_S(false, 2, true, true, false);
  } else if (L.mx) {
    if (L.terms == 2) { if (under) BDFP4_LAUNCH(true, 2, true); else BDFP4_LAUNCH(true, 2, false); }
    else { if (under) BDFP4_LAUNCH(true, 1, true); else BDFP4_LAUNCH(true, 1, false); }
  } else {
    if (L.terms == 2) { if (under) BDFP4_LAUNCH(false, 2, true); else BDFP4_LAUNCH(false, 2, false); }
    else { if (under) BDFP4_LAUNCH(false, 1, true); else BDFP4_LAUNCH(false, 1, false); }
  }
#undef BDFP4_LAUNCH
#undef BDFP4_LAUNCH_CH
#undef BDFP4_LAUNCH_S
}

}  // namespace bdfp4
