// Streaming-read probe: reads a buffer once with 16-byte non-temporal loads,
// eight per thread in flight, grid-strided (a measured HBM read ceiling to set
// beside the nominal peak). The loaded words are folded and written to *sink
// only for one improbable value, so the loads cannot be dropped.
#include "common.h"
#include "internal.h"

namespace beam {

constexpr int kReadThreads = 256;
constexpr int kReadBlocks = 8192;

__global__ __launch_bounds__(kReadThreads) void hbm_read_kernel(const uint4* __restrict__ p,
                                                                size_t n16,
                                                                unsigned* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  unsigned acc = 0;
  for (size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x; i < n16; i += stride * 8) {
    uint4 v[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const size_t j = i + b * stride;
      v[b] = j < n16 ? ld16_nt(p + j) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) acc ^= v[b].x ^ v[b].y ^ v[b].z ^ v[b].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// Zeroes n 32-bit words (a workspace's counter block) with vector stores: a
// kernel rather than a memset node, so the clear also replays correctly from
// a captured graph.
__global__ __launch_bounds__(256) void zero_words_kernel(unsigned* __restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

int launch_zero_words(unsigned* p, int n, hipStream_t st) {
  hipLaunchKernelGGL(zero_words_kernel, dim3(std::max(1, std::min((n + 255) / 256, 64))),
                     dim3(256), 0, st, p, n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_hbm_read(const void* p, size_t bytes, unsigned* sink, hipStream_t st) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(kReadBlocks), dim3(kReadThreads), 0, st,
                     (const uint4*)p, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace beam
