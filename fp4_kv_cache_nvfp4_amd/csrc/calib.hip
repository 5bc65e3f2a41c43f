// Calibration kernels: per-channel key means and output-error sums.
//
// "BitDecoding-FP4 evaluation/config.py", RECIPE outlier_aware_key_quantization:
// key smoothing subtracts a static per-(KV head, channel) key shift, which a
// calibration pass creates when it is missing; probability_environment:
// tau is searched ("calibrate") before it is used. The key shift here is the
// mean of the calibration keys; the tau search compares decode outputs with
// exact attention through the error sums below.
//
// Both reductions run in float64 in a fixed order (per thread in token or
// index order, then fixed trees and sequential passes), so results do not
// depend on scheduling.
#include "codec.hpp"
#include "launch.hpp"

namespace bdfp4 {

namespace {

constexpr int kMeanChunk = 2048;  // tokens per workgroup of the first pass
constexpr int kRound = 16;        // loads in flight per thread

// The sums start from +0.0 and absent entries add +0.0, as the plain sum
// 0 + x_0 + x_1 + ... does (a channel of zeros of either sign sums to +0.0).

// Pass 1: workgroup (chunk c, head h) sums tokens [2048 c, 2048 c + 2048) of
// head h. Thread (r = tid >> 4, octet o = tid & 15) takes channels 8 o .. 8 o
// + 7 of tokens 2048 c + r + 16 k (k = 0..127, in order; 16 loads in flight
// per round), one 16-byte load per token; the 16 token lanes of a channel are
// then added in lane order.
__global__ void __launch_bounds__(256) key_sum_kernel(const uint16_t* k, int tokens, int hkv, double* part) {
  __shared__ double s[16][128];
  const int c = blockIdx.x, h = blockIdx.y;
  const int r = threadIdx.x >> 4, o = threadIdx.x & 15;
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  for (int k0 = 0; k0 < kMeanChunk / 16; k0 += kRound) {
    uint4 w[kRound];
#pragma unroll
    for (int kk = 0; kk < kRound; ++kk) {
      const int t = c * kMeanChunk + r + 16 * (k0 + kk);
      w[kk] = t < tokens ? *reinterpret_cast<const uint4*>(k + ((size_t)t * hkv + h) * kD + 8 * o)
                         : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int kk = 0; kk < kRound; ++kk) {
      const uint32_t ws[4] = {w[kk].x, w[kk].y, w[kk].z, w[kk].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += (double)__uint_as_float(ws[j] << 16);
        acc[2 * j + 1] += (double)__uint_as_float(ws[j] & 0xFFFF0000u);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) s[r][8 * o + j] = acc[j];
  __syncthreads();
  if (threadIdx.x < kD) {
    double v = 0.0;
    for (int i = 0; i < 16; ++i) v += s[i][threadIdx.x];
    part[((size_t)c * hkv + h) * kD + threadIdx.x] = v;
  }
}

// Pass 2: thread (h, channel) adds the chunk sums in chunk order (16 loads in
// flight per round) and rounds the float64 mean to float32.
__global__ void __launch_bounds__(128) key_mean_kernel(const double* part, int nchunks, int tokens, int hkv,
                                                       float* mu) {
  const int h = blockIdx.x, ch = threadIdx.x;
  double v = 0.0;
  for (int c0 = 0; c0 < nchunks; c0 += kRound) {
    double x[kRound];
#pragma unroll
    for (int j = 0; j < kRound; ++j)
      x[j] = c0 + j < nchunks ? part[((size_t)(c0 + j) * hkv + h) * kD + ch] : 0.0;
#pragma unroll
    for (int j = 0; j < kRound; ++j) v += x[j];
  }
  mu[h * kD + ch] = (float)(v / (double)tokens);
}

// One workgroup: thread t adds (got - ref)^2 and ref^2 over i = t, t + 256,
// ... in float64, then a fixed tree over the 256 threads.
__global__ void __launch_bounds__(256) error_sums_kernel(const float* got, const float* ref, int64_t n,
                                                         double* out) {
  __shared__ double se[256], sr[256];
  double e = 0.0, q = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    const double g = (double)got[i], f = (double)ref[i];
    e += (g - f) * (g - f);
    q += f * f;
  }
  se[threadIdx.x] = e;
  sr[threadIdx.x] = q;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      se[threadIdx.x] += se[threadIdx.x + w];
      sr[threadIdx.x] += sr[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[0] = se[0];
    out[1] = sr[0];
  }
}

}  // namespace

size_t key_means_workspace_bytes(int tokens, int hkv) {
  const size_t nchunks = ((size_t)tokens + kMeanChunk - 1) / kMeanChunk;
  return nchunks * (size_t)hkv * kD * sizeof(double);
}

hipError_t launch_key_means(const void* k, int tokens, int hkv, void* workspace, float* mu, hipStream_t stream) {
  const int nchunks = (tokens + kMeanChunk - 1) / kMeanChunk;
  double* part = static_cast<double*>(workspace);
  hipLaunchKernelGGL(key_sum_kernel, dim3((unsigned)nchunks, (unsigned)hkv), dim3(256u), 0, stream,
                     static_cast<const uint16_t*>(k), tokens, hkv, part);
  hipLaunchKernelGGL(key_mean_kernel, dim3((unsigned)hkv), dim3(128u), 0, stream, part, nchunks, tokens, hkv, mu);
  return hipGetLastError();
}

hipError_t launch_error_sums(const float* got, const float* ref, int64_t n, double* out, hipStream_t stream) {
  hipLaunchKernelGGL(error_sums_kernel, dim3(1u), dim3(256u), 0, stream, got, ref, n, out);
  return hipGetLastError();
}

}  // namespace bdfp4
