// Router projection and router backward: the step in front of the top-k
// ("Nous Research scales expert parallelism with DeepEP", paragraph on
// practical implications: Top-k routing; "NVIDIA NeMo AutoModel ...",
// section "Background": tokens are routed across many experts).
//
// Forward: logits[t, e] = sum_h x[t, h] * W_r[e, h] (+ bias[e]), each logit
// accumulated in float64 one term at a time in ascending h, bias added
// last, rounded once to float32.  Products of two bf16 values are exact in
// float64, so an FMA chain in that order is the same sum term by term: the
// logits, and the routing decided on them, do not depend on the launch
// shape.
//
// Backward: dlogits from the routing-weight gradient through the softmax
// the forward used (over the chosen set, or over all experts); then
// dW_r = dlogits^T x and the router's dx = dlogits W_r, float32.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "timer.hpp"

namespace moe {
namespace {

constexpr int kLgH = 64;   // h per LDS chunk

// Block tile: EB experts x TB tokens, 256 threads.  Thread (tt, te) owns
// experts te + NE * j (j < EPT) and tokens tt + NT * i (i < TPT).  Each
// output is one sequential chain of H FMAs, so the tile shape trades
// parallelism (one chain per thread when there are few) against
// independent chains per thread (latency hiding when there are many).
// Chunks of 64 h go through LDS as float64; the next chunk's bf16 values
// are loaded (16-byte vectors, H % 8 == 0) while the current one is used.
template <int EB, int TPB, int EPT>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const float* __restrict__ bias, int64_t T, int H, int E,
    float* __restrict__ logits) {
  constexpr int TPT = TPB;
  constexpr int NE = EB / EPT;      // threads along experts
  constexpr int NT = 256 / NE;      // threads along tokens
  constexpr int TB = NT * TPT;
  constexpr int XQ = (TB * 8 + 255) / 256;   // 16-byte x loads per thread
  constexpr int WQ = (EB * 8 + 255) / 256;   // 16-byte w loads per thread
  static_assert(NE * NT == 256 && NE * EPT == EB, "tile shape");
  __shared__ double xs[TB][kLgH + 1];
  __shared__ double ws[EB][kLgH + 1];
  const int tid = threadIdx.x;
  const int tt = tid / NE, te = tid % NE;
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const int e0 = blockIdx.y * EB;
  uint4 xr[XQ], wr[WQ];
  // 16-byte vector q of the chunk at h0 (zeros past T, E and H)
  auto load = [&](int h0) {
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const int idx = tid + 256 * q;
      const int r = idx >> 3, h = h0 + 8 * (idx & 7);
      const int64_t t = t0 + r;
      xr[q] = (idx < TB * 8 && t < T && h < H)
                  ? *reinterpret_cast<const uint4*>(x + t * H + h)
                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < WQ; ++q) {
      const int idx = tid + 256 * q;
      const int r = idx >> 3, h = h0 + 8 * (idx & 7);
      const int e = e0 + r;
      wr[q] = (idx < EB * 8 && e < E && h < H)
                  ? *reinterpret_cast<const uint4*>(w + (int64_t)e * H + h)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto put = [&](double* row, uint4 v) {
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      row[2 * i] = (double)bf16lo(p[i]);
      row[2 * i + 1] = (double)bf16hi(p[i]);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const int idx = tid + 256 * q;
      if (idx < TB * 8) put(&xs[idx >> 3][8 * (idx & 7)], xr[q]);
    }
#pragma unroll
    for (int q = 0; q < WQ; ++q) {
      const int idx = tid + 256 * q;
      if (idx < EB * 8) put(&ws[idx >> 3][8 * (idx & 7)], wr[q]);
    }
  };
  // -0.0 + p == p for every p (a sum that starts at its first term)
  double acc[TPT][EPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc[i][j] = -0.0;
  auto term = [&](int c) {
    double xv[TPT], wv[EPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) xv[i] = xs[tt + NT * i][c];
#pragma unroll
    for (int j = 0; j < EPT; ++j) wv[j] = ws[te + NE * j][c];
#pragma unroll
    for (int i = 0; i < TPT; ++i)
#pragma unroll
      for (int j = 0; j < EPT; ++j) acc[i][j] = fma(xv[i], wv[j], acc[i][j]);
  };
  load(0);
  for (int h0 = 0; h0 < H; h0 += kLgH) {
    store();
    __syncthreads();
    if (h0 + kLgH < H) load(h0 + kLgH);
    const int hn = min(kLgH, H - h0);
    if (hn == kLgH) {
      // whole chunk unrolled: the LDS reads go out ahead of the FMA chain
#pragma unroll
      for (int c = 0; c < kLgH; ++c) term(c);
    } else {   // columns past H are never read
      for (int c = 0; c < hn; ++c) term(c);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int64_t t = t0 + tt + NT * i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = e0 + te + NE * j;
      if (e >= E) continue;
      double s = acc[i][j];
      if (bias) s += (double)bias[e];
      logits[t * E + e] = (float)s;
    }
  }
}

// One wave per token: dlogits[t, :] from dtopk_w[t, :] (float64 inside).
__global__ __launch_bounds__(256) void router_dlogits_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ dw, int64_t T, int E, int k, int renorm,
    float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* lg = logits + t * E;
  double m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmax(m, (double)lg[e] + 0.0);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
  // expert ids are clamped for reading (an id outside [0, E) gives an
  // unspecified result, never an out-of-range access)
  auto sel = [&](int j) { return min(max(idx[t * k + j], 0), E - 1); };
  // the chosen experts' exp(l - m) and the normaliser
  double den = 0.0;
  if (renorm) {
    for (int j = 0; j < k; ++j) den += exp((double)lg[sel(j)] - m);
  } else {
    double part = 0.0;
    for (int e = lane; e < E; e += 64) part += exp((double)lg[e] - m);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    den = part;
  }
  // dot = sum_j w_j dw_j over the chosen set
  double dot = 0.0;
  for (int j = 0; j < k; ++j)
    dot += exp((double)lg[sel(j)] - m) / den * (double)dw[t * k + j];
  for (int e = lane; e < E; e += 64) {
    double g = 0.0;
    bool chosen = false;
    for (int j = 0; j < k; ++j)
      if (sel(j) == e) {
        g = (double)dw[t * k + j];
        chosen = true;
      }
    double v = 0.0;
    if (chosen || !renorm) {
      const double p = exp((double)lg[e] - m) / den;
      v = p * (g - dot);
    }
    dl[t * E + e] = (float)v;
  }
}

// C[m, n] (+)= sum over k in [k0, k1) of A(m, k) B(k, n), float32.
// A is float32: A(m, k) = a[m * a_m + k * a_k]; B is bf16 [K, N] row-major.
// 64 x 64 tile per block, k in chunks of 16 through LDS; thread (tm, tn)
// owns rows 4 tm .. +3 and columns 4 tn .. +3.  The k order is ascending
// inside a split; split z writes its own partial slice c + z * M * N.
constexpr int kGT = 64;
constexpr int kGK = 16;

__global__ __launch_bounds__(256) void router_gemm_kernel(
    const float* __restrict__ a, int64_t a_m, int64_t a_k,
    const uint16_t* __restrict__ b, int64_t M, int64_t N, int64_t K,
    int64_t k_per_split, float* __restrict__ c) {
  __shared__ float as[kGK][kGT + 4];
  __shared__ float bs[kGK][kGT + 4];
  const int tid = threadIdx.x;
  const int tm = tid >> 4, tn = tid & 15;
  const int64_t m0 = (int64_t)blockIdx.y * kGT;
  const int64_t n0 = (int64_t)blockIdx.x * kGT;
  const int64_t k0 = (int64_t)blockIdx.z * k_per_split;
  const int64_t k1 = min(K, k0 + k_per_split);
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int64_t kc = k0; kc < k1; kc += kGK) {
    // A chunk: 16 k x 64 m; B chunk: 16 k x 64 n (zeros past the edges)
#pragma unroll
    for (int q = 0; q < (kGK * kGT) / 256; ++q) {
      const int idx = tid + 256 * q;
      // consecutive threads along the operand's contiguous direction
      int kk, mm;
      if (a_m == 1) { kk = idx / kGT; mm = idx % kGT; }
      else { mm = idx / kGK; kk = idx % kGK; }
      const int64_t gk = kc + kk, gm = m0 + mm;
      as[kk][mm] = (gk < k1 && gm < M) ? a[gm * a_m + gk * a_k] : 0.0f;
      const int bk = idx / kGT, bn = idx % kGT;
      const int64_t hk = kc + bk, hn = n0 + bn;
      bs[bk][bn] = (hk < k1 && hn < N) ? bf16_to_f32(b[hk * N + hn]) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = as[kk][4 * tm + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = bs[kk][4 * tn + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* cz = c + (int64_t)blockIdx.z * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gm = m0 + 4 * tm + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gn = n0 + 4 * tn + j;
      if (gn < N) cz[gm * N + gn] = acc[i][j];
    }
  }
}

// out[i] = sum over splits s = 0, 1, ... of part[s][i]
__global__ __launch_bounds__(256) void router_split_sum_kernel(
    const float* __restrict__ part, int splits, int64_t n,
    float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int z = 0; z < splits; ++z) s += part[(int64_t)z * n + i];
  out[i] = s;
}

// splits of the dW_r reduction over tokens: enough blocks for the chip
int dw_splits(int64_t T, int E, int H) {
  const int64_t tiles = ((E + kGT - 1) / kGT) * ((H + kGT - 1) / kGT);
  int64_t s = (1024 + tiles - 1) / tiles;
  s = std::min<int64_t>(s, (T + 255) / 256);
  return (int)std::max<int64_t>(1, std::min<int64_t>(s, 64));
}

}  // namespace

hipError_t launch_router_logits(const void* x, const void* w_r,
                                const float* bias, int64_t T, int H, int E,
                                float* logits, hipStream_t stream) {
  KernelScope ks("router_logits", stream);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* wp = static_cast<const uint16_t*>(w_r);
  auto go = [&](auto kern, int eb, int tb) {
    const dim3 grid((unsigned)((T + tb - 1) / tb), (unsigned)((E + eb - 1) / eb));
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, xp, wp, bias, T, H, E,
                       logits);
  };
  // up to 2^20 chains: one per thread; more: 32 per thread (4 tokens x 8
  // experts of a 128 x 64 tile: 12 LDS reads per 32 FMAs)
  if (T * (int64_t)E > ((int64_t)1 << 20)) go(router_logits_kernel<64, 4, 8>, 64, 128);
  else if (E <= 8) go(router_logits_kernel<8, 1, 1>, 8, 32);
  else if (E <= 16) go(router_logits_kernel<16, 1, 1>, 16, 16);
  else if (E <= 32) go(router_logits_kernel<32, 1, 1>, 32, 8);
  else go(router_logits_kernel<64, 1, 1>, 64, 4);
  return hipGetLastError();
}

size_t router_bwd_ws_bytes(int64_t T, int H, int E) {
  const int s = dw_splits(T, E, H);
  return s > 1 ? (size_t)s * E * H * sizeof(float) : 0;
}

hipError_t launch_router_bwd(const float* logits, const int32_t* topk_idx,
                             const float* dtopk_w, const void* x,
                             const void* w_r, int64_t T, int H, int E, int k,
                             bool renorm, float* dlogits, float* dw_r,
                             float* dx, void* ws, hipStream_t stream) {
  {
    KernelScope ks("router_dlogits", stream);
    hipLaunchKernelGGL(router_dlogits_kernel,
                       dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream,
                       logits, topk_idx, dtopk_w, T, E, k, renorm ? 1 : 0,
                       dlogits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dx) {
    // dx[t, h] = sum_e dl[t, e] W_r[e, h]
    KernelScope ks("router_dx", stream);
    const dim3 grid((unsigned)((H + kGT - 1) / kGT),
                    (unsigned)((T + kGT - 1) / kGT), 1);
    hipLaunchKernelGGL(router_gemm_kernel, grid, dim3(256), 0, stream,
                       dlogits, (int64_t)E, (int64_t)1,
                       static_cast<const uint16_t*>(w_r), T, (int64_t)H,
                       (int64_t)E, (int64_t)E, dx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dw_r) {
    // dW_r[e, h] = sum_t dl[t, e] x[t, h], split over tokens, then summed
    // over the splits in order
    const int s = dw_splits(T, E, H);
    const int64_t kps = ((T + s - 1) / s + kGK - 1) / kGK * kGK;
    float* part = s > 1 ? static_cast<float*>(ws) : dw_r;
    {
      KernelScope ks("router_dw", stream);
      const dim3 grid((unsigned)((H + kGT - 1) / kGT),
                      (unsigned)((E + kGT - 1) / kGT), (unsigned)s);
      hipLaunchKernelGGL(router_gemm_kernel, grid, dim3(256), 0, stream,
                         dlogits, (int64_t)1, (int64_t)E,
                         static_cast<const uint16_t*>(x), (int64_t)E,
                         (int64_t)H, T, kps, part);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (s > 1) {
      KernelScope ks("router_dw_sum", stream);
      const int64_t n = (int64_t)E * H;
      hipLaunchKernelGGL(router_split_sum_kernel,
                         dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                         stream, part, s, n, dw_r);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace moe
