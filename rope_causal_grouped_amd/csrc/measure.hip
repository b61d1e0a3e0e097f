// Streaming-read helper for benchmarks: how fast a plain kernel reads HBM
// on this device, as context for the HBM-bound kernels' roofline figures.
// Not part of the attention path.

#include "common.h"
#include "launch.h"

namespace gqa {

namespace {

// Grid-stride, four 16-byte non-temporal loads in flight per lane; the XOR
// of everything read keeps the loads live (written out only if it equals
// a value the caller's data does not produce, which still forces the reads).
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n,
                                                          unsigned* __restrict__ sink) {
  unsigned acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* p, size_t bytes, unsigned* sink, hipStream_t st) {
  stream_read_kernel<<<8192, 256, 0, st>>>((const u32x4*)p, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace gqa
