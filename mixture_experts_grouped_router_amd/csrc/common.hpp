// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_codec.hpp"
#include "offsets_check.hpp"

namespace moe {

constexpr int kWave = 64;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) 16-byte global load / store.
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u32x4_t v =
      __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(uint4* p, const uint4 v) {
  u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

// bfloat16 storage <-> float32.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t pair) {
  return __uint_as_float(pair << 16);
}
__device__ __forceinline__ float bf16hi(uint32_t pair) {
  return __uint_as_float(pair & 0xffff0000u);
}
// float -> bf16 with round to nearest even (v_cvt_pk_bf16_f32)
typedef __bf16 moe_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float moe_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(
      uint32_t, __builtin_convertvector(moe_f32x2_t{lo, hi}, moe_bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// ---- MXFP8 encoding with the gfx950 scaled conversion ----------------------
// v_cvt_scalef32_pk_fp8_bf16 converts two bf16 values divided by a float
// scale to E4M3 with round to nearest even.  For every finite bf16 value v
// and block exponent s with |v| < 2^(s+9) (all values a block with scale s
// can hold) it returns the same code as e4m3_from_bf16(v, s), except that a
// value rounding above 448 gives the NaN code 0x7F / 0xFF where the
// encoding saturates to 448 (0x7E / 0xFE); sat_e4m3x4 repairs those bytes.
// 2^-127 is passed as the subnormal float it is.
__device__ __forceinline__ float mx_scale_f32(int s) {
  return s > -127 ? __uint_as_float((uint32_t)(127 + s) << 23)
                  : __uint_as_float(0x00400000u);
}
// bytes 0x7F / 0xFF -> 0x7E / 0xFE, other bytes unchanged
__device__ __forceinline__ uint32_t sat_e4m3x4(uint32_t x) {
  const uint32_t m = ((x & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;
  return x ^ (m >> 7);
}
typedef short mx_v2i16 __attribute__((ext_vector_type(2)));
typedef __bf16 mx_v2bf16 __attribute__((ext_vector_type(2)));
// four E4M3 codes from two dwords of packed bf16 pairs (low halves first)
__device__ __forceinline__ uint32_t e4m3x4_hw(uint32_t lo2, uint32_t hi2,
                                              float scale) {
  mx_v2i16 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      r, __builtin_bit_cast(mx_v2bf16, lo2), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      r, __builtin_bit_cast(mx_v2bf16, hi2), scale, true);
  return sat_e4m3x4(__builtin_bit_cast(uint32_t, r));
}
// four E4M3 codes from four floats (first value in the low byte)
__device__ __forceinline__ uint32_t e4m3x4_hw_f32(float a, float b, float c,
                                                  float d, float scale) {
  mx_v2i16 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, a, b, scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c, d, scale, true);
  return sat_e4m3x4(__builtin_bit_cast(uint32_t, r));
}
// MXFP8 encoding of one block of 32 float32 values held by a quad of lanes
// (4 consecutive lanes starting at a multiple of 4, 8 consecutive values
// each, in lane order): the block exponent from the quad's amax (two lane
// swaps, float32 magnitudes compared as integers), then the E4M3 codes with
// the scaled conversion and the 448 fix-up.  Every lane of the quad must be
// active.  Returns the lane's 8 codes (first value in the low byte) and the
// block exponent in *sx.
__device__ __forceinline__ uint2 mx_quad_encode_f32(const float (&v)[8],
                                                    int* sx) {
  uint32_t am = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t a = __float_as_uint(v[c]) & 0x7fffffffu;
    am = am > a ? am : a;
  }
  uint32_t o = __shfl_xor(am, 1, 64);
  am = am > o ? am : o;
  o = __shfl_xor(am, 2, 64);
  am = am > o ? am : o;
  const int s = e8m0_exp_from_f32_amax(am);
  const float sc = mx_scale_f32(s);
  *sx = s;
  return make_uint2(e4m3x4_hw_f32(v[0], v[1], v[2], v[3], sc),
                    e4m3x4_hw_f32(v[4], v[5], v[6], v[7], sc));
}

// 8 bf16 (one uint4) -> 8 E4M3 codes with block exponent s
__device__ __forceinline__ uint2 e4m3x8_hw(const uint4 v, int s) {
  const float sc = mx_scale_f32(s);
  return make_uint2(e4m3x4_hw(v.x, v.y, sc), e4m3x4_hw(v.z, v.w, sc));
}

// Record the first device-side data error (first error wins).
__device__ __forceinline__ void report_error(int32_t* status, int32_t code) {
  if (status) atomicCAS(status, 0, code);
}

// Block-wide check of a segment offsets array [n_seg + 1] against `rows`,
// by a block of exactly 256 threads, thread t taking pairs 4t .. 4t+3
// (n_seg <= 1024).  Every thread of the block must call it; all get the
// same answer.  An invalid array is recorded once, by block (0, 0, 0).
__device__ __forceinline__ bool seg_offsets_ok(const int32_t* off, int n_seg,
                                               int64_t rows, int t,
                                               int32_t* status) {
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sg = 4 * t + i;
    if (sg < n_seg) ok = ok && offsets_pair_ok(off, sg, n_seg, rows);
  }
  const bool bad = __syncthreads_or(!ok);
  if (bad && t == 0 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    report_error(status, kDevErrOffsets);
  return !bad;
}

// Exclusive scan of one int per thread over a block of exactly 256 threads.
// Returns the thread's exclusive prefix and the block total in *total.
__device__ __forceinline__ int32_t block_exclusive_scan_256(int32_t v,
                                                            int32_t* total) {
  __shared__ int32_t wsum[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int32_t s = wsum[w];
    if (w < wid) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return incl - v + before;
}

}  // namespace moe
