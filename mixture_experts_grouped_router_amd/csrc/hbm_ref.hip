// Achievable-bandwidth reference for the HBM-bound kernels (a measurement
// aid, not a step of the path): a stream that reads a buffer once and
// writes k copies of it, the traffic shape of the permute's row gather
// (each token row read once, written to its k expert rows) without the
// gather's indexing.  The best of a sweep on MI355X (64 and 128 MiB
// buffers, k = 2, caches flushed): streaming (non-temporal) 16-byte loads
// and stores -- plain ones reached only 3.6-4.3 TB/s -- with each block
// taking a contiguous 16 KiB per trip (four vectors per thread) and 32
// blocks per CU: 5.43 TB/s at 64 MiB, 5.80 TB/s at 128 MiB; one block per
// 8 KiB row (the gather's shape) 5.18 / 5.59 TB/s.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "timer.hpp"

namespace moe {

namespace {
constexpr int kStreamUnroll = 4;

__global__ __launch_bounds__(256) void hbm_stream_kernel(
    const uint4* __restrict__ src, int64_t n16, int k,
    uint4* __restrict__ dst) {
  constexpr int64_t per = 256 * kStreamUnroll;   // vectors per block trip
  for (int64_t b0 = (int64_t)blockIdx.x * per; b0 < n16;
       b0 += (int64_t)gridDim.x * per) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t i = b0 + 256 * u + threadIdx.x;
      if (i < n16) v[u] = ld_nt(src + i);
    }
    for (int j = 0; j < k; ++j) {
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const int64_t i = b0 + 256 * u + threadIdx.x;
        if (i < n16) st_nt(dst + (int64_t)j * n16 + i, v[u]);
      }
    }
  }
}
}  // namespace

hipError_t launch_hbm_stream(const void* src, int64_t bytes, int k, void* dst,
                             int cu_count, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0 || k <= 0) return hipSuccess;
  KernelScope ks("hbm_stream_reference", stream);
  const int64_t want = (n16 + 256 * kStreamUnroll - 1) / (256 * kStreamUnroll);
  const int64_t grid = std::min<int64_t>(want, (int64_t)cu_count * 32);
  hipLaunchKernelGGL(hbm_stream_kernel, dim3((unsigned)grid), dim3(256), 0,
                     stream, static_cast<const uint4*>(src), n16, k,
                     static_cast<uint4*>(dst));
  return hipGetLastError();
}

}  // namespace moe
