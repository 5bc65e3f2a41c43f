// KV page writer for gfx950: key centering, 128-point Hadamard rotation and
// NVFP4 / MXFP4 block quantization of whole 128-token pages.
//
// "How openbitsys/bitdecoding-fp4 works" (gitdiagram): the KV cache writer
// quantizes pages through KV quantization, which uses block scaling and scale
// modes. "kv-landlords scripts/quant_ab.py", PageSim: a page is quantized
// once when it fills. "BitDecoding-FP4 evaluation/config.py": RECIPE
// outlier_aware_key_quantization (key smoothing, Hadamard rotation, adaptive
// block-scale search), recipe_additional_config (key four_six, value amax6),
// KV_MODES bitdecoding-mxfp4 (mxfp4_search).
//
// One workgroup of 256 threads quantizes one (page, KV head) of either K or
// V (page_head, shared by the bulk writer and the decode-time append). Each row of 128 elements sits in four consecutive lanes, 32 elements per
// lane, so the rotation needs only two cross-lane (DPP quad) stages and every
// NVFP4 block (16) / MXFP4 block (32) lies inside one lane. A wave covers a
// 16-token tile, whose K codes are one contiguous 1 KiB run of the page
// layout, written straight from registers; V codes and all scales are
// assembled in LDS and written as contiguous 16-byte stores.
#include "codec.hpp"
#include "launch.hpp"

namespace bdfp4 {

struct WriterArgs {
  const uint16_t* k;       // [n_pages*128][hkv][128] bf16
  const uint16_t* v;
  const int32_t* page_ids;
  const float* key_shift;  // [hkv][128] or null
  uint8_t* k_codes;
  uint8_t* k_scales;
  uint8_t* v_codes;
  uint8_t* v_scales;
  int32_t num_pages;
  int32_t hkv;
  int32_t n_pages;
  int32_t rotation;
  int32_t rotate_v;          // values rotated before quantization (recipe variant)
  int32_t k_chan;            // channel key scale geometry (blocks of 16 tokens of one channel)
};

// Row t (token 0..127) of input page in_page of the bulk writer's
// [pages * 128][hkv][128] input, for KV head h.
struct WriterRows {
  const uint16_t* src;
  int in_page, hkv, h;
  __device__ const uint16_t* operator()(int t) const {
    return src + (((size_t)in_page * kPage + t) * hkv + h) * kD;
  }
};

// Row t of the BF16 tail [128][128] of one (sequence, KV head), except row
// 127, which is the token being appended.
struct TailRows {
  const uint16_t* tail;
  const uint16_t* last;
  __device__ const uint16_t* operator()(int t) const { return t == kPage - 1 ? last : tail + (size_t)t * kD; }
};

// Quantizes one (page, KV head) of K (is_v false) or V into cache block blk
// (= physical page * hkv + h); rows(t) is the address of the page's row t
// (128 bf16). All 256 threads of the workgroup call it (it has barriers).
// kKMode / kVMode: 1 amax6, 2 four_six, 3 mxfp4_search.
//
// kChan: the channel key scale geometry ("BitDecoding-FP4
// evaluation/config.py", KV_MODES key_scale_geometry; "kv-landlords
// scripts/quant_ab.py", SCHEMES per-channel keys): a key block is 16 tokens of
// one channel. Each wave puts its tile's centered, rotated rows in LDS
// (float32 [token][channel], tbuf: 16 x 128 floats per wave), and lane l
// quantizes the 16-token columns of channels 2l and 2l + 1 with the same
// block quantizer; the codes keep the K page layout (a byte holds channels
// 2l, 2l + 1 of one token), the scales are stored [token block][channel].
template <int kKMode, int kVMode, bool is_v, bool kChan, class Rows>
__device__ __forceinline__ void page_head(const WriterArgs& a, const Rows& rows, int h, size_t blk,
                                          uint8_t* s_codes, uint8_t* s_scales, float* tbuf) {
  constexpr bool kKMx = kKMode == 3, kVMx = kVMode == 3;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int q = lane & 3;          // quarter of the row: elements [32q, 32q+32)
  const int n = lane >> 2;         // token within the 16-token tile

  float mu[32];
  if (!is_v && a.key_shift != nullptr) {
    const float4* m4 = reinterpret_cast<const float4*>(a.key_shift + h * kD + 32 * q);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 t = m4[i];
      mu[4 * i] = t.x; mu[4 * i + 1] = t.y; mu[4 * i + 2] = t.z; mu[4 * i + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) mu[i] = 0.0f;
  }
  const bool center = !is_v && a.key_shift != nullptr;

#pragma unroll 1
  for (int it = 0; it < 2; ++it) {
    const int tile = wave * 2 + it;
    const int t = tile * 16 + n;
    const uint4* p = reinterpret_cast<const uint4*>(rows(t) + 32 * q);
    uint4 w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = p[k];
    float x[32];
    widen32(w, x);

    if (!is_v) {
      if (center) {
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = __fsub_rn(x[i], mu[i]);
      }
      if (a.rotation) rotate_row_quad(x, q);
      if constexpr (kChan) {
        float* tb = tbuf + wave * (16 * kD);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<float4*>(tb + n * kD + 32 * q + 4 * i) =
              make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
        // the wave reads back its own LDS rows (a wave's LDS operations
        // complete in order): the column of channels 2 lane, 2 lane + 1
        float xa[16], xb[16];
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
          const float2 v2 = *reinterpret_cast<const float2*>(tb + tt * kD + 2 * lane);
          xa[tt] = v2.x;
          xb[tt] = v2.y;
        }
        uint32_t pa[2], pb[2];
        const uint32_t sa = nv_block<kKMode == 2>(xa, pa);
        const uint32_t sb = nv_block<kKMode == 2>(xb, pb);
        *reinterpret_cast<uint16_t*>(&s_scales[tile * kD + 2 * lane]) = (uint16_t)(sa | (sb << 8));
        // token t's byte of channels 2 lane (low nibble), 2 lane + 1
        uint8_t* cb = s_codes + tile * 1024 + (lane >> 4) * 256 + (lane & 15);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t ev = (pa[k] & 0x0F0F0F0Fu) | ((pb[k] & 0x0F0F0F0Fu) << 4);            // tokens 8k + 2m
          const uint32_t od = ((pa[k] >> 4) & 0x0F0F0F0Fu) | (((pb[k] >> 4) & 0x0F0F0F0Fu) << 4);  // 8k + 2m + 1
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            cb[(8 * k + 2 * m) * 16] = (uint8_t)(ev >> (8 * m));
            cb[(8 * k + 2 * m + 1) * 16] = (uint8_t)(od >> (8 * m));
          }
        }
        continue;
      }
      uint32_t pk[4];
      if (kKMx) {
        const uint32_t sc = mx_block(x, pk);
        s_scales[(q * 16 + n) * 8 + tile] = (uint8_t)sc;
      } else {
        const uint32_t s0 = nv_block<kKMode == 2>(x, pk);
        const uint32_t s1 = nv_block<kKMode == 2>(x + 16, pk + 2);
        *reinterpret_cast<uint16_t*>(&s_scales[((q * 16 + n) * 8 + tile) * 2]) =
            (uint16_t)(s0 | (s1 << 8));
      }
      uint4* dstc = reinterpret_cast<uint4*>(a.k_codes + blk * 8192 + tile * 1024 + q * 256 + n * 16);
      *dstc = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    } else {
      if (a.rotate_v) rotate_row_quad(x, q);
      uint32_t pk[4];
      const int chunk = t >> 5, qq = (t >> 3) & 3, i8 = t & 7;
      if (kVMx) {
        const uint32_t sc = mx_block(x, pk);
        s_scales[((chunk * 4 + qq) * 4 + q) * 8 + i8] = (uint8_t)sc;
      } else {
        const uint32_t s0 = nv_block<false>(x, pk);
        const uint32_t s1 = nv_block<false>(x + 16, pk + 2);
        s_scales[((chunk * 4 + qq) * 8 + 2 * q) * 8 + i8] = (uint8_t)s0;
        s_scales[((chunk * 4 + qq) * 8 + 2 * q + 1) * 8 + i8] = (uint8_t)s1;
      }
      if (kVMx) {
        // element pairs per byte: the lane's 4 words are d-octets 4q .. 4q+3 of token t
#pragma unroll
        for (int o = 0; o < 4; ++o) {
          const int oct = 4 * q + o;
          *reinterpret_cast<uint32_t*>(&s_codes[(((chunk * 4 + qq) * 16 + oct) * 8 + i8) * 4]) = pk[o];
        }
      } else {
        // token pairs per byte: tokens t (even) and t + 1 live in lanes l and
        // l ^ 4; the even lane writes channels [32q, 32q+16), the odd lane
        // [32q+16, 32q+32), low nibble = even token
        uint32_t other[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) other[w] = (uint32_t)__shfl_xor((int)pk[w], 4, 64);
        const bool odd = (t & 1) != 0;
        const int te = t & ~1;
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          const int w = odd ? 2 + w2 : w2;
          const uint32_t mine = odd ? pk[2 + w2] : pk[w2];          // static indices only
          const uint32_t theirs = odd ? other[2 + w2] : other[w2];
          const uint32_t lo_tok = odd ? theirs : mine;
          const uint32_t hi_tok = odd ? mine : theirs;
          const uint32_t even_b = (lo_tok & 0x0F0F0F0Fu) | ((hi_tok & 0x0F0F0F0Fu) << 4);   // elements 0,2,4,6
          const uint32_t odd_b = ((lo_tok >> 4) & 0x0F0F0F0Fu) | (hi_tok & 0xF0F0F0F0u);    // elements 1,3,5,7
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int d = 32 * q + 8 * w + e;
            const uint32_t byte = ((e & 1) ? odd_b : even_b) >> (8 * (e >> 1));
            s_codes[(te >> 5) * 2048 + (((te >> 3) & 3) * 16 + (d >> 3)) * 32 + (d & 7) * 4 + ((te & 7) >> 1)] =
                (uint8_t)byte;
          }
        }
      }
    }
  }
  __syncthreads();
  if (!is_v) {
    const int sbytes = kKMx ? 512 : 1024;
    if (tid * 16 < sbytes)
      *reinterpret_cast<uint4*>(a.k_scales + blk * sbytes + tid * 16) =
          *reinterpret_cast<const uint4*>(&s_scales[tid * 16]);
    if constexpr (kChan) {
      uint4* dc = reinterpret_cast<uint4*>(a.k_codes + blk * 8192);
      const uint4* sc4 = reinterpret_cast<const uint4*>(s_codes);
      dc[tid] = sc4[tid];
      dc[tid + 256] = sc4[tid + 256];
    }
  } else {
    const int sbytes = kVMx ? 512 : 1024;
    uint4* dc = reinterpret_cast<uint4*>(a.v_codes + blk * 8192);
    const uint4* sc4 = reinterpret_cast<const uint4*>(s_codes);
    dc[tid] = sc4[tid];
    dc[tid + 256] = sc4[tid + 256];
    if (tid * 16 < sbytes)
      *reinterpret_cast<uint4*>(a.v_scales + blk * sbytes + tid * 16) =
          *reinterpret_cast<const uint4*>(&s_scales[tid * 16]);
  }
}

// One workgroup per (input page, KV head) quantizes the K page, then the V
// page, through the same LDS staging (the barrier between them keeps the K
// block's copy-out ahead of the V block's first LDS writes). Measured
// against one workgroup per page of one kind (twice the grid): 150-154 us
// instead of 161 us (NVFP4) and 147 us instead of 158 us (MXFP4) for
// 131,072 tokens x 8 heads, with bit-identical output.
// At least 3 (MXFP4) / 4 (NVFP4) waves per SIMD: the MXFP4 body would take
// 171 VGPRs (2 waves) unbounded and fits 168 without spilling; NVFP4 fits
// 4 waves as it is (at 5 it would spill).
template <int kKMode, int kVMode, bool kChan>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kKMode == 3 || kChan ? 3 : 4)))
writer_kernel(WriterArgs a) {
  __shared__ __align__(16) uint8_t s_codes[8192];
  __shared__ __align__(16) uint8_t s_scales[1024];
  __shared__ __align__(16) float tbuf[kChan ? 4 * 16 * kD : 4];
  const int ph = blockIdx.x;       // input page * hkv + head
  const int in_page = ph / a.hkv, h = ph - in_page * a.hkv;
  const int dst = a.page_ids[in_page];
  if (dst < 0 || dst >= a.num_pages) return;
  const size_t blk = (size_t)dst * a.hkv + h;
  const WriterRows krows{a.k, in_page, a.hkv, h};
  page_head<kKMode, kVMode, false, kChan>(a, krows, h, blk, s_codes, s_scales, tbuf);
  __syncthreads();
  const WriterRows vrows{a.v, in_page, a.hkv, h};
  page_head<kKMode, kVMode, true, kChan>(a, vrows, h, blk, s_codes, s_scales, tbuf);
}

// Decode-time append with freeze-at-fill ("kv-landlords scripts/quant_ab.py"
// PageSim: the hot page stays BF16 and is quantized once, when it fills).
// Workgroup (sequence b, KV head h) of K (y = 0) or V (y = 1): the new row
// goes to tail slot pos mod 128 (and to the sink when pos < sink_tokens);
// when it fills slot 127, the workgroup quantizes the tail as one page into
// block_tables[b][pos / 128], taking row 127 from the new row itself (the
// tail rows 0..126 were written by earlier launches).
struct AppendArgs {
  WriterArgs w;                 // cache, key_shift, rotation, num_pages, hkv
  const uint16_t* k_new;        // [B][hkv][128]
  const uint16_t* v_new;
  const int32_t* positions;     // [B]
  const int32_t* block_tables;  // [B][max_pages_per_seq]
  uint16_t* sink_k;             // [B][hkv][sink_tokens][128]
  uint16_t* sink_v;
  uint16_t* tail_k;             // [B][hkv][128][128]
  uint16_t* tail_v;
  int32_t max_pages_per_seq, sink_tokens;
};

template <int kKMode, int kVMode, bool kChan>
__global__ void __launch_bounds__(256) append_kernel(AppendArgs a) {
  __shared__ __align__(16) uint8_t s_codes[8192];
  __shared__ __align__(16) uint8_t s_scales[1024];
  __shared__ __align__(16) float tbuf[kChan ? 4 * 16 * kD : 4];
  const int hkv = a.w.hkv;
  const int bh = blockIdx.x, b = bh / hkv, h = bh - b * hkv;
  const bool is_v = blockIdx.y != 0;
  const int pos = a.positions[b];
  if (pos < 0 || pos >= kPage * a.max_pages_per_seq) return;   // padding row or past the block table
  const int slot = pos & (kPage - 1);
  const uint16_t* nrow = (is_v ? a.v_new : a.k_new) + (size_t)bh * kD;
  uint16_t* tail = (is_v ? a.tail_v : a.tail_k) + (size_t)bh * kPage * kD;
  if (threadIdx.x < 16) {
    const uint4 w = reinterpret_cast<const uint4*>(nrow)[threadIdx.x];
    reinterpret_cast<uint4*>(tail + (size_t)slot * kD)[threadIdx.x] = w;
    if (pos < a.sink_tokens)
      reinterpret_cast<uint4*>((is_v ? a.sink_v : a.sink_k) + ((size_t)bh * a.sink_tokens + pos) * kD)[threadIdx.x] = w;
  }
  if (slot != kPage - 1) return;
  const int dst = a.block_tables[(size_t)b * a.max_pages_per_seq + pos / kPage];
  if (dst < 0 || dst >= a.w.num_pages) return;
  const TailRows rows{tail, nrow};
  if (is_v) page_head<kKMode, kVMode, true, kChan>(a.w, rows, h, (size_t)dst * hkv + h, s_codes, s_scales, tbuf);
  else page_head<kKMode, kVMode, false, kChan>(a.w, rows, h, (size_t)dst * hkv + h, s_codes, s_scales, tbuf);
}

// Quantization diagnostics ("kv-landlords scripts/quant_ab.py" compares cache
// schemes by reconstruction error): workgroup (input page, head) of K (y = 0)
// or V (y = 1) recomputes the float32 rows that were quantized (keys centered
// and rotated exactly as page_head does, values as they are), dequantizes
// the stored page through the byte layout of the cache (codes and scales
// staged in LDS) and adds (x_hat - x)^2 and x^2 in float64: thread sums in
// element order, then a fixed tree. part[y][page-head][2] holds the sums.
__device__ __forceinline__ double e2m1_f64(uint32_t nib) {
  const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  const double m = mag[nib & 7u];
  return (nib & 8u) ? -m : m;
}

template <bool kMx>
__device__ __forceinline__ double scale_f64(uint32_t code) {
  if (kMx) return ldexp(1.0, (int)code - 127);              // E8M0
  return (double)e4m3_value(code);                          // E4M3 (exact in float32)
}

template <bool kKMx, bool kVMx, bool is_v, bool kChan>
__device__ __forceinline__ void page_error(const WriterArgs& a, int in_page, int h, size_t blk, uint8_t* s_codes,
                                           uint8_t* s_scales, double& err, double& ref) {
  constexpr bool kMx = is_v ? kVMx : kKMx;
  constexpr int sbytes = kMx ? 512 : 1024;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane & 3, n = lane >> 2;
  const uint4* codes = reinterpret_cast<const uint4*>((is_v ? a.v_codes : a.k_codes) + blk * 8192);
  const uint4* scales = reinterpret_cast<const uint4*>((is_v ? a.v_scales : a.k_scales) + blk * sbytes);
  reinterpret_cast<uint4*>(s_codes)[tid] = codes[tid];
  reinterpret_cast<uint4*>(s_codes)[tid + 256] = codes[tid + 256];
  if (tid * 16 < sbytes) reinterpret_cast<uint4*>(s_scales)[tid] = scales[tid];
  float mu[32];
  const bool center = !is_v && a.key_shift != nullptr;
#pragma unroll
  for (int i = 0; i < 32; ++i) mu[i] = center ? a.key_shift[h * kD + 32 * q + i] : 0.0f;
  __syncthreads();
  const WriterRows rows{is_v ? a.v : a.k, in_page, a.hkv, h};
#pragma unroll 1
  for (int it = 0; it < 2; ++it) {
    const int t = (wave * 2 + it) * 16 + n;
    const uint4* p = reinterpret_cast<const uint4*>(rows(t) + 32 * q);
    uint4 w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = p[k];
    float x[32];
    widen32(w, x);
    if (!is_v) {
      if (center) {
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = __fsub_rn(x[i], mu[i]);
      }
      if (a.rotation) rotate_row_quad(x, q);
    } else if (a.rotate_v) {
      rotate_row_quad(x, q);
    }
#pragma unroll 4
    for (int e = 0; e < 32; ++e) {
      const int d = 32 * q + e;
      int cb, sb, shift;
      if (!is_v) {
        cb = (t >> 4) * 1024 + (d >> 5) * 256 + (t & 15) * 16 + ((d & 31) >> 1);
        shift = 4 * (d & 1);
        sb = kChan ? (t >> 4) * kD + d
                   : (kMx ? ((d >> 5) * 16 + (t & 15)) * 8 + (t >> 4)
                          : ((((d >> 4) >> 1) * 16 + (t & 15)) * 8 + (t >> 4)) * 2 + ((d >> 4) & 1));
      } else {
        const int g = (t >> 5) * 4 + ((t >> 3) & 3);
        if (kMx) {
          cb = ((g * 16 + (d >> 3)) * 8 + (t & 7)) * 4 + ((d & 7) >> 1);
          shift = 4 * (d & 1);
          sb = (g * 4 + (d >> 5)) * 8 + (t & 7);
        } else {
          cb = (t >> 5) * 2048 + (((t >> 3) & 3) * 16 + (d >> 3)) * 32 + (d & 7) * 4 + ((t & 7) >> 1);
          shift = 4 * (t & 1);
          sb = (g * 8 + (d >> 4)) * 8 + (t & 7);
        }
      }
      const double xh = e2m1_f64(((uint32_t)s_codes[cb] >> shift) & 15u) * scale_f64<kMx>(s_scales[sb]);
      const double xv = (double)x[e];
      err = fma(xh - xv, xh - xv, err);
      ref = fma(xv, xv, ref);
    }
  }
}

template <bool kKMx, bool kVMx, bool kChan>
__global__ void __launch_bounds__(256) page_error_kernel(WriterArgs a, double* part) {
  __shared__ __align__(16) uint8_t s_codes[8192];
  __shared__ __align__(16) uint8_t s_scales[1024];
  __shared__ double s_e[256], s_r[256];
  const int ph = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int in_page = ph / a.hkv, h = ph - in_page * a.hkv;
  const int dst = a.page_ids[in_page];
  double err = 0.0, ref = 0.0;
  if (dst >= 0 && dst < a.num_pages) {
    const size_t blk = (size_t)dst * a.hkv + h;
    if (is_v) page_error<kKMx, kVMx, true, kChan>(a, in_page, h, blk, s_codes, s_scales, err, ref);
    else page_error<kKMx, kVMx, false, kChan>(a, in_page, h, blk, s_codes, s_scales, err, ref);
  }
  s_e[threadIdx.x] = err;
  s_r[threadIdx.x] = ref;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      s_e[threadIdx.x] += s_e[threadIdx.x + w];
      s_r[threadIdx.x] += s_r[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double* o = part + ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * 2;
    o[0] = s_e[0];
    o[1] = s_r[0];
  }
}

// out[2 y + c] = sum over page-heads i of part[y][i][c]: thread t adds
// i = t, t + 256, ... in order, then a fixed tree (workgroup y).
__global__ void __launch_bounds__(256) page_error_total_kernel(const double* part, int n, double* out) {
  __shared__ double s_e[256], s_r[256];
  const double* py = part + (size_t)blockIdx.x * n * 2;
  double e = 0.0, r = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) {
    e += py[2 * i];
    r += py[2 * i + 1];
  }
  s_e[threadIdx.x] = e;
  s_r[threadIdx.x] = r;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      s_e[threadIdx.x] += s_e[threadIdx.x + w];
      s_r[threadIdx.x] += s_r[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = s_e[0];
    out[2 * blockIdx.x + 1] = s_r[0];
  }
}

static WriterArgs writer_args(const WriterLaunch& L) {
  WriterArgs a;
  a.k = static_cast<const uint16_t*>(L.k);
  a.v = static_cast<const uint16_t*>(L.v);
  a.page_ids = L.page_ids;
  a.key_shift = L.key_shift;
  a.k_codes = static_cast<uint8_t*>(L.k_codes);
  a.k_scales = static_cast<uint8_t*>(L.k_scales);
  a.v_codes = static_cast<uint8_t*>(L.v_codes);
  a.v_scales = static_cast<uint8_t*>(L.v_scales);
  a.num_pages = L.num_pages;
  a.hkv = L.hkv;
  a.n_pages = L.n_pages;
  a.rotation = L.rotation;
  a.rotate_v = L.rotate_v;
  a.k_chan = L.k_chan;
  return a;
}

hipError_t launch_writer(const WriterLaunch& L, hipStream_t stream) {
  if (L.n_pages == 0) return hipSuccess;
  const WriterArgs a = writer_args(L);
  const dim3 grid((unsigned)(L.n_pages * L.hkv)), block(256u);
  if (L.k_chan && L.k_mode == 2 && L.v_mode == 1)
    hipLaunchKernelGGL((writer_kernel<2, 1, true>), grid, block, 0, stream, a);
  else if (L.k_chan && L.k_mode == 1 && L.v_mode == 1)
    hipLaunchKernelGGL((writer_kernel<1, 1, true>), grid, block, 0, stream, a);
  else if (L.k_chan)
    return hipErrorInvalidValue;
  else if (L.k_mode == 2 && L.v_mode == 1)
    hipLaunchKernelGGL((writer_kernel<2, 1, false>), grid, block, 0, stream, a);
  else if (L.k_mode == 1 && L.v_mode == 1)
    hipLaunchKernelGGL((writer_kernel<1, 1, false>), grid, block, 0, stream, a);
  else if (L.k_mode == 3 && L.v_mode == 3)
    hipLaunchKernelGGL((writer_kernel<3, 3, false>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_append(const AppendLaunch& L, hipStream_t stream) {
  if (L.batch == 0) return hipSuccess;
  AppendArgs a;
  a.w = writer_args(L.w);
  a.k_new = static_cast<const uint16_t*>(L.k_new);
  a.v_new = static_cast<const uint16_t*>(L.v_new);
  a.positions = L.positions;
  a.block_tables = L.block_tables;
  a.sink_k = static_cast<uint16_t*>(L.sink_k);
  a.sink_v = static_cast<uint16_t*>(L.sink_v);
  a.tail_k = static_cast<uint16_t*>(L.tail_k);
  a.tail_v = static_cast<uint16_t*>(L.tail_v);
  a.max_pages_per_seq = L.max_pages_per_seq;
  a.sink_tokens = L.sink_tokens;
  const dim3 grid((unsigned)(L.batch * L.w.hkv), 2u), block(256u);
  const int km = L.w.k_mode, vm = L.w.v_mode;
  const bool ch = L.w.k_chan != 0;
  if (ch && km == 2 && vm == 1)
    hipLaunchKernelGGL((append_kernel<2, 1, true>), grid, block, 0, stream, a);
  else if (ch && km == 1 && vm == 1)
    hipLaunchKernelGGL((append_kernel<1, 1, true>), grid, block, 0, stream, a);
  else if (ch)
    return hipErrorInvalidValue;
  else if (km == 2 && vm == 1)
    hipLaunchKernelGGL((append_kernel<2, 1, false>), grid, block, 0, stream, a);
  else if (km == 1 && vm == 1)
    hipLaunchKernelGGL((append_kernel<1, 1, false>), grid, block, 0, stream, a);
  else if (km == 3 && vm == 3)
    hipLaunchKernelGGL((append_kernel<3, 3, false>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

size_t page_errors_workspace_bytes(int n_pages, int hkv) { return (size_t)n_pages * hkv * 2 * 2 * sizeof(double); }

hipError_t launch_page_errors(const WriterLaunch& L, void* workspace, double* out, hipStream_t stream) {
  const WriterArgs a = writer_args(L);
  double* part = static_cast<double*>(workspace);
  const int n = L.n_pages * L.hkv;
  const dim3 grid((unsigned)n, 2u), block(256u);
  if (L.k_chan && L.k_mode != 3 && L.v_mode != 3)
    hipLaunchKernelGGL((page_error_kernel<false, false, true>), grid, block, 0, stream, a, part);
  else if (L.k_chan)
    return hipErrorInvalidValue;
  else if (L.k_mode == 3 && L.v_mode == 3)
    hipLaunchKernelGGL((page_error_kernel<true, true, false>), grid, block, 0, stream, a, part);
  else if (L.k_mode != 3 && L.v_mode != 3)
    hipLaunchKernelGGL((page_error_kernel<false, false, false>), grid, block, 0, stream, a, part);
  else
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(page_error_total_kernel, dim3(2u), dim3(256u), 0, stream, part, n, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- debug codec

// One row per quad of lanes: optional shift, optional rotation, then the
// scale mode, and for terms == 2 the residual r = y - deq(Q1) quantized again.
template <int kMode>
__global__ void __launch_bounds__(256) rows_kernel(const uint16_t* rows, int n_rows, const float* shift,
                                                   int rotation, int terms, uint8_t* codes, uint8_t* scales) {
  constexpr bool kMx = kMode == 3;
  constexpr int nb = kMx ? 4 : 8;
  const int gl = blockIdx.x * 256 + threadIdx.x;
  const int row = gl >> 2, q = gl & 3;
  const bool live = row < n_rows;
  const int r = live ? row : 0;   // dead quads compute on row 0 and store nothing
  const uint4* p = reinterpret_cast<const uint4*>(rows + (size_t)r * kD + 32 * q);
  uint4 w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = p[k];
  float x[32];
  widen32(w, x);
  if (shift != nullptr) {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = __fsub_rn(x[i], shift[32 * q + i]);
  }
  if (rotation) rotate_row_quad(x, q);
  for (int term = 0; term < terms; ++term) {
    uint32_t pk[4];
    float deq[32];
    if (kMx) {
      const uint32_t sc = mx_block(x, pk);
      if (live) scales[((size_t)row * terms + term) * nb + q] = (uint8_t)sc;
      const float s = pow2_f32((int)sc - 127);   // an all-zero block dequantizes to 0
#pragma unroll
      for (int k = 0; k < 4; ++k) deq8(pk[k], s, deq + 8 * k);
    } else {
      uint32_t s0 = nv_block<kMode == 2>(x, pk);
      uint32_t s1 = nv_block<kMode == 2>(x + 16, pk + 2);
      if (live) {
        scales[((size_t)row * terms + term) * nb + 2 * q] = (uint8_t)s0;
        scales[((size_t)row * terms + term) * nb + 2 * q + 1] = (uint8_t)s1;
      }
      deq8(pk[0], e4m3_value(s0), deq);
      deq8(pk[1], e4m3_value(s0), deq + 8);
      deq8(pk[2], e4m3_value(s1), deq + 16);
      deq8(pk[3], e4m3_value(s1), deq + 24);
    }
    if (live)
      *reinterpret_cast<uint4*>(codes + ((size_t)row * terms + term) * 64 + 16 * q) =
          make_uint4(pk[0], pk[1], pk[2], pk[3]);
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = __fsub_rn(x[i], deq[i]);
  }
}

hipError_t launch_rows(const void* rows, int n_rows, const float* shift, int rotation, int mode,
                       int terms, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_rows * 4 + 255) / 256)), block(256u);
  const uint16_t* r = static_cast<const uint16_t*>(rows);
  if (mode == 1)
    hipLaunchKernelGGL((rows_kernel<1>), grid, block, 0, stream, r, n_rows, shift, rotation, terms, codes, scales);
  else if (mode == 2)
    hipLaunchKernelGGL((rows_kernel<2>), grid, block, 0, stream, r, n_rows, shift, rotation, terms, codes, scales);
  else if (mode == 3)
    hipLaunchKernelGGL((rows_kernel<3>), grid, block, 0, stream, r, n_rows, shift, rotation, terms, codes, scales);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bdfp4

namespace bdfp4 {

// One 16-value block of p' per lane: block max, the probability scale rule
// (amax2_or_amax6: E4M3(a/2) if a < tau else E4M3(a/6); amax6: E4M3(a/6)),
// then the E2M1 codes.
__global__ void __launch_bounds__(256) p_blocks_kernel(const float* pp, int n_blocks, int mode, float tau,
                                                       uint8_t* codes, uint8_t* scales) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= n_blocks) return;
  float x[16];
  const float4* p4 = reinterpret_cast<const float4*>(pp + (size_t)b * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 t = p4[i];
    x[4 * i] = t.x; x[4 * i + 1] = t.y; x[4 * i + 2] = t.z; x[4 * i + 3] = t.w;
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = __builtin_fmaxf(a, x[i]);
  const uint32_t sc = mode == 4 ? p_scale_code<true>(a, tau) : p_scale_code<false>(a, tau);
  uint32_t pk[2];
  quant_block<16, false>(x, e4m3_value(sc), pk);
  *reinterpret_cast<uint2*>(codes + (size_t)b * 8) = make_uint2(pk[0], pk[1]);
  scales[b] = (uint8_t)sc;
}

hipError_t launch_p_blocks(const float* pp, int n_blocks, int mode, float tau, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream) {
  if (n_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(p_blocks_kernel, dim3((unsigned)((n_blocks + 255) / 256)), dim3(256u), 0, stream,
                     pp, n_blocks, mode, tau, codes, scales);
  return hipGetLastError();
}

}  // namespace bdfp4
