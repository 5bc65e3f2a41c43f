// Plain streaming read of a device buffer: the practical HBM read ceiling the
// decode is measured against (the same byte count through the simplest
// access pattern there is). Grid-stride over 16-byte words: in one step the
// grid reads kStreamUnroll consecutive grid-wide runs, every wave a 1 KiB
// piece of each, four loads in flight per thread; each thread folds its
// words into one 32-bit value so the loads cannot be dropped.
#include "launch.hpp"

namespace bdfp4 {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

__global__ void __launch_bounds__(kStreamThreads) stream_read_kernel(const uint4* __restrict__ src, size_t words,
                                                                     uint32_t* __restrict__ sink) {
  const size_t nth = (size_t)gridDim.x * kStreamThreads;
  const size_t tid = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  uint32_t x = 0;
  for (size_t base = tid; base < words; base += nth * kStreamUnroll) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t i = base + (size_t)u * nth;
      v[u] = i < words ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[tid] = x;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kStreamThreads), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace bdfp4
