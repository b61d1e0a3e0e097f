// Streaming-read helper for benchmarks: how fast a plain kernel reads HBM
// on this device, as context for the HBM-bound kernels' roofline figures.
// Not part of the attention path.

#include "common.h"
#include "launch.h"

namespace gqa {

namespace {

// Each workgroup reads one contiguous block, eight 16-byte non-temporal
// loads in flight per lane (a grid-stride loop over the whole buffer reads
// about 11% slower on MI355X: 6.3 against 7.0 TB/s); the XOR of everything
// read keeps the loads live (written out only if it equals a value the
// caller's data does not produce, which still forces the reads).
constexpr int kStreamU = 8;
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n,
                                                          size_t per, unsigned* __restrict__ sink) {
  unsigned acc = 0;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n ? b0 + per : n;
  size_t i = b0 + threadIdx.x;
  for (; i + (kStreamU - 1) * 256 < b1; i += kStreamU * 256) {
    u32x4 v[kStreamU];
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < b1; i += 256) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* p, size_t bytes, unsigned* sink, hipStream_t st) {
  const size_t n = bytes / 16;
  const unsigned grid = 8192;
  const size_t per = ((n + grid - 1) / grid + 255) / 256 * 256;   // elements per workgroup
  stream_read_kernel<<<grid, 256, 0, st>>>((const u32x4*)p, n, per, sink);
  return hipGetLastError();
}

}  // namespace gqa
