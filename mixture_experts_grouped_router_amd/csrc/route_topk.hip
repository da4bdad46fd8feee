// Router top-k: 16 lanes per token (k <= 16, E <= 256), else one wave64
// per token.
//
// Top-k routing over the E router logits of each token ("Nous Research
// scales expert parallelism with DeepEP", practical-implications paragraph;
// "Efficient MoE training for biological foundation models (NVIDIA)",
// section "Why dense and MoE models differ": a small subset of experts per
// token).  Weights: softmax restricted to the chosen experts (or over all E),
// evaluated in float64 and rounded to float32.
//
// Each lane holds E/16 (or E/64) logits in registers.  k rounds of an
// argmax over the token's lanes (larger value first, lower expert id on
// ties) pick the experts; lane j keeps slot j.  No LDS; a NaN or infinite
// logit (a precondition violation) records MOE_DEVERR_LOGITS in the device
// status word.
#include "common.hpp"
#include "kernels.hpp"
#include "timer.hpp"

namespace moe {

namespace {

// device status code (include/moe.h: MOE_DEVERR_LOGITS)
constexpr int32_t kDevErrLogits = 3;

struct Cand {
  float v;
  int e;
};

// a beats b: larger logit, or equal logit and lower expert id.  +0 == -0
// under float comparison, so signed zeros tie and fall to the id rule.
__device__ __forceinline__ bool beats(float av, int ae, float bv, int be) {
  return av > bv || (av == bv && ae < be);
}

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* status) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + t * (int64_t)E;

  float v[VPL];
  uint32_t taken = 0;  // bit i: v[i] already selected
  bool bad = false;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : 0.0f;
    if (e >= E) taken |= 1u << i;
    bad |= !__builtin_isfinite(v[i]);
  }
  if (bad) report_error(status, kDevErrLogits);

  float my_v = 0.0f;  // lane j < k: logit of slot j
  int my_e = 0;
  float top_v = 0.0f;
  for (int j = 0; j < k; ++j) {
    // lane-local best among not-yet-taken values
    float bv = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (!(taken >> i & 1u) && (be == 0x7fffffff || beats(v[i], e, bv, be))) {
        bv = v[i];
        be = e;
      }
    }
    // wave-wide argmax (butterfly: every lane ends with the winner)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (oe != 0x7fffffff && (be == 0x7fffffff || beats(ov, oe, bv, be))) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
    if (j == 0) top_v = bv;
  }

  // weights in float64: exp(l - max) / sum
  const double m = (double)top_v;
  double num = 0.0;
  if (lane < k) num = exp((double)my_v - m);
  double part;
  if (renorm) {
    part = num;
  } else {
    part = 0.0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) part += exp((double)v[i] - m);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
  if (lane < k) {
    topk_idx[t * k + lane] = my_e;
    topk_w[t * k + lane] = (float)(num / part);
  }
}

// ---- 16 lanes per token (k <= 16, E <= 256) -------------------------------
// Four tokens per wave.  Lane s of a token's 16 holds the logits of experts
// s, s + 16, ...; the reductions across the 16 lanes use DPP lane moves
// (VALU only): quad swaps (xor 1, xor 2), then the half-row and row
// mirrors.  Each step pairs lanes that hold equal partial results, so every
// lane ends with the same value, bit for bit, also for the float64 sum.
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;       // lane i <- 15 - i within 16

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const uint64_t u = __double_as_longlong(x);
  const int lo = dpp_i<CTRL>((int)(uint32_t)u);
  const int hi = dpp_i<CTRL>((int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) |
                                          (uint32_t)lo));
}
// (bv, be) <- the better of it and the candidate of the lane CTRL names
template <int CTRL>
__device__ __forceinline__ void best_step(float& bv, int& be) {
  const float ov = dpp_f<CTRL>(bv);
  const int oe = dpp_i<CTRL>(be);
  if (oe != 0x7fffffff && (be == 0x7fffffff || beats(ov, oe, bv, be))) {
    bv = ov;
    be = oe;
  }
}
template <int CTRL>
__device__ __forceinline__ void sum_step(double& v) {
  v += dpp_d<CTRL>(v);
}

template <int VPL>
__global__ __launch_bounds__(256) void route_topk16_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* status) {
  const int s = threadIdx.x & 15;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 4) + (threadIdx.x >> 4);
  if (t >= T) return;   // whole 16-lane rows leave together
  const float* row = logits + t * (int64_t)E;

  float v[VPL];
  uint32_t taken = 0;  // bit i: v[i] already selected (or no expert)
  bool bad = false;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = s + 16 * i;
    v[i] = e < E ? row[e] : 0.0f;
    if (e >= E) taken |= 1u << i;
    bad |= !__builtin_isfinite(v[i]);
  }
  if (bad) report_error(status, kDevErrLogits);

  float my_v = 0.0f;  // lane j < k: logit of slot j
  int my_e = 0;
  float top_v = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = s + 16 * i;
      if (!(taken >> i & 1u) && (be == 0x7fffffff || beats(v[i], e, bv, be))) {
        bv = v[i];
        be = e;
      }
    }
    best_step<kDppXor1>(bv, be);
    best_step<kDppXor2>(bv, be);
    best_step<kDppHalfMirror>(bv, be);
    best_step<kDppMirror>(bv, be);
    if ((be & 15) == s) taken |= 1u << (be >> 4);
    if (s == j) {
      my_v = bv;
      my_e = be;
    }
    if (j == 0) top_v = bv;
  }

  // weights in float64: exp(l - max) / sum
  const double m = (double)top_v;
  double num = 0.0;
  if (s < k) num = exp((double)my_v - m);
  double part;
  if (renorm) {
    part = num;
  } else {
    part = 0.0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = s + 16 * i;
      if (e < E) part += exp((double)v[i] - m);
    }
  }
  sum_step<kDppXor1>(part);
  sum_step<kDppXor2>(part);
  sum_step<kDppHalfMirror>(part);
  sum_step<kDppMirror>(part);
  if (s < k) {
    topk_idx[t * k + s] = my_e;
    topk_w[t * k + s] = (float)(num / part);
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k,
                             int renorm, int32_t* idx, float* w,
                             int32_t* status, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (k <= 16 && E <= 256) {
    // 16 tokens per block of 256 threads
    const dim3 grid16((unsigned)((T + 15) / 16));
    const int v16 = (E + 15) / 16;
    KernelScope ks("route_topk", stream);
    if (v16 <= 1)
      hipLaunchKernelGGL(route_topk16_kernel<1>, grid16, dim3(256), 0, stream,
                         logits, T, E, k, renorm, idx, w, status);
    else if (v16 <= 2)
      hipLaunchKernelGGL(route_topk16_kernel<2>, grid16, dim3(256), 0, stream,
                         logits, T, E, k, renorm, idx, w, status);
    else if (v16 <= 4)
      hipLaunchKernelGGL(route_topk16_kernel<4>, grid16, dim3(256), 0, stream,
                         logits, T, E, k, renorm, idx, w, status);
    else if (v16 <= 8)
      hipLaunchKernelGGL(route_topk16_kernel<8>, grid16, dim3(256), 0, stream,
                         logits, T, E, k, renorm, idx, w, status);
    else
      hipLaunchKernelGGL(route_topk16_kernel<16>, grid16, dim3(256), 0, stream,
                         logits, T, E, k, renorm, idx, w, status);
    return hipGetLastError();
  }
  const int tokens_per_block = 4;
  const dim3 grid((unsigned)((T + tokens_per_block - 1) / tokens_per_block));
  const int vpl = (E + 63) / 64;
  KernelScope ks("route_topk", stream);
#define MOE_ROUTE_CASE(N)                                                      \
  case N:                                                                      \
    hipLaunchKernelGGL(route_topk_kernel<N>, grid, dim3(256), 0, stream,      \
                       logits, T, E, k, renorm, idx, w, status);               \
    break;
  switch (vpl) {
    MOE_ROUTE_CASE(1)
    MOE_ROUTE_CASE(2)
    MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(16)
    case 3:
      hipLaunchKernelGGL(route_topk_kernel<4>, grid, dim3(256), 0, stream,
                         logits, T, E, k, renorm, idx, w, status);
      break;
    default:
      if (vpl <= 8)
        hipLaunchKernelGGL(route_topk_kernel<8>, grid, dim3(256), 0, stream,
                           logits, T, E, k, renorm, idx, w, status);
      else
        hipLaunchKernelGGL(route_topk_kernel<16>, grid, dim3(256), 0, stream,
                           logits, T, E, k, renorm, idx, w, status);
  }
#undef MOE_ROUTE_CASE
  return hipGetLastError();
}

}  // namespace moe
