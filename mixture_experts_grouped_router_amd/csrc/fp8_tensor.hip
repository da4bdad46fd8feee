// Tensor-scaled FP8: one float32 scale per tensor from an amax pass
// ("NVIDIA presents an efficient path for training biological MoE models",
// section "Reducing memory and quantisation cost", and "Efficient MoE
// training for biological foundation models (NVIDIA)", section "3)
// Quantisation overhead in low-precision training": 8-bit formats with
// scales, quantised from 16-bit masters).  s = amax / 448 (1 for an
// all-zero tensor), code = E4M3(float32(v / s)) with round to nearest even
// and saturation.  A buffer of n_seg equal segments holds n_seg tensors
// (each expert's weight matrix is its own tensor).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "timer.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// amax (as float32 bits of a non-negative value) of each segment; blocks
// stride over their segment, 8 bf16 per 16-byte load
__global__ __launch_bounds__(256) void seg_amax_kernel(
    const uint16_t* __restrict__ src, int64_t seg_elems,
    uint32_t* __restrict__ amax_bits) {
  const int seg = blockIdx.y;
  const uint4* s = reinterpret_cast<const uint4*>(src + seg * seg_elems);
  const int64_t n8 = seg_elems / 8;
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * 256) {
    const uint4 v = s[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = w[j] & 0x7fffu, hi = (w[j] >> 16) & 0x7fffu;
      m = max(m, max(lo, hi));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    // bf16 magnitude -> float32 bits (order preserving)
    atomicMax(amax_bits + seg, m << 16);
  }
}

__device__ __forceinline__ float tensor_scale(uint32_t amax_bits) {
  const float a = __uint_as_float(amax_bits);
  return a > 0.0f ? a / 448.0f : 1.0f;
}

// codes of each segment with its scale; scales[seg] = s
__global__ __launch_bounds__(256) void tensor_quant_kernel(
    const uint16_t* __restrict__ src, int64_t seg_elems,
    const uint32_t* __restrict__ amax_bits, uint8_t* __restrict__ codes,
    float* __restrict__ scales) {
  const int seg = blockIdx.y;
  const float sc = tensor_scale(amax_bits[seg]);
  if (blockIdx.x == 0 && threadIdx.x == 0) scales[seg] = sc;
  const uint4* s = reinterpret_cast<const uint4*>(src + seg * seg_elems);
  uint2* d = reinterpret_cast<uint2*>(codes + seg * seg_elems);
  const int64_t n8 = seg_elems / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * 256) {
    const uint4 v = s[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float q[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      q[2 * j] = bf16lo(w[j]) / sc;        // IEEE float32 division
      q[2 * j + 1] = bf16hi(w[j]) / sc;
    }
    d[i] = make_uint2(e4m3x4_hw_f32(q[0], q[1], q[2], q[3], 1.0f),
                      e4m3x4_hw_f32(q[4], q[5], q[6], q[7], 1.0f));
  }
}

unsigned blocks_per_seg(int64_t seg_elems, int n_seg) {
  const int64_t want = (seg_elems / 8 + 255) / 256;
  const int64_t cap = (2048 + n_seg - 1) / n_seg;   // ~8 blocks per CU
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(want, cap));
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  KernelScope ks("fp8_amax_clear", stream);
  hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     stream, p, n);
  return hipGetLastError();
}

hipError_t launch_seg_amax(const void* src, int64_t seg_elems, int n_seg,
                           uint32_t* amax_bits, hipStream_t stream) {
  if (n_seg <= 0 || seg_elems <= 0) return hipSuccess;
  KernelScope ks("fp8_amax", stream);
  hipLaunchKernelGGL(seg_amax_kernel,
                     dim3(blocks_per_seg(seg_elems, n_seg), n_seg), dim3(256),
                     0, stream, static_cast<const uint16_t*>(src), seg_elems,
                     amax_bits);
  return hipGetLastError();
}

hipError_t launch_tensor_quant(const void* src, int64_t seg_elems, int n_seg,
                               const uint32_t* amax_bits, uint8_t* codes,
                               float* scales, hipStream_t stream) {
  if (n_seg <= 0) return hipSuccess;
  KernelScope ks("fp8_tensor_quantize", stream);
  hipLaunchKernelGGL(tensor_quant_kernel,
                     dim3(blocks_per_seg(std::max<int64_t>(seg_elems, 8), n_seg),
                          n_seg),
                     dim3(256), 0, stream, static_cast<const uint16_t*>(src),
                     seg_elems, amax_bits, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
