// The per-expert loop: the expert MLP computed the way an eager framework's
// Python loop over experts does it, as the baseline the grouped path is
// measured against ("NVIDIA presents an efficient path for training
// biological MoE models", section "Grouped experts instead of a Python
// loop": the loop launches separate small kernels per expert, which the
// grouped GEMM replaces).  The caller has read the per-expert row counts
// back to the host; then for every expert with rows, in ascending order: a gate/up GEMM writing (g, u) in bf16, a SwiGLU kernel
// writing a = w * silu(g) * u in bf16, a down GEMM.  The GEMM launches use
// the grouped kernel on one expert at a time; nothing is fused.
#include "grouped_gemm.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

using namespace gg;

// Tile tables of one-expert launches: t[2e] = 0, t[2e+1] = tiles of e.
__global__ __launch_bounds__(256) void loop_tile_tables_kernel(
    const int32_t* __restrict__ offsets, int E, int tn1, int tn2,
    int32_t* __restrict__ t1, int32_t* __restrict__ t2) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int mt = (offsets[e + 1] - offsets[e] + BM - 1) / BM;
  t1[2 * e] = 0;
  t1[2 * e + 1] = mt * tn1;
  t2[2 * e] = 0;
  t2[2 * e + 1] = mt * tn2;
}

// a[r, f] = w[r] * silu(g) * u for rows [row0, row0 + nrows), g = h1[r, f],
// u = h1[r, F + f] (bf16), float32 arithmetic, one bf16 rounding.  One
// thread per 8 consecutive f.
__global__ __launch_bounds__(256) void loop_swiglu_kernel(
    const uint16_t* __restrict__ h1, const float* __restrict__ w, int F,
    int64_t row0, int64_t nrows, uint16_t* __restrict__ a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = F / 8;
  if (i >= nrows * per_row) return;
  const int64_t r = row0 + i / per_row;
  const int f = (int)(i % per_row) * 8;
  const uint4 g4 = *reinterpret_cast<const uint4*>(h1 + r * 2 * F + f);
  const uint4 u4 = *reinterpret_cast<const uint4*>(h1 + r * 2 * F + F + f);
  const float wr = w ? w[r] : 1.0f;
  const uint32_t gw[4] = {g4.x, g4.y, g4.z, g4.w};
  const uint32_t uw[4] = {u4.x, u4.y, u4.z, u4.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float g0 = bf16lo(gw[j]), g1 = bf16hi(gw[j]);
    const float v0 = wr * (g0 * fast_sigmoid(g0)) * bf16lo(uw[j]);
    const float v1 = wr * (g1 * fast_sigmoid(g1)) * bf16hi(uw[j]);
    o[j] = pack_bf16x2(v0, v1);
  }
  *reinterpret_cast<uint4*>(a + r * F + f) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

size_t expert_loop_fwd_ws_bytes(int E, int F, int64_t rows, bool need_h1,
                                bool need_a) {
  size_t b = 2 * align256((size_t)2 * E * sizeof(int32_t));
  if (need_h1) b += align256((size_t)rows * 2 * F * 2);
  if (need_a) b += align256((size_t)rows * F * 2);
  return b;
}

hipError_t launch_expert_loop_fwd(int E, int H, int F, int64_t rows,
                                  const void* x_perm, const void* w_gu,
                                  const void* w_dn, const float* w_perm,
                                  const int32_t* offsets,
                                  const int32_t* offsets_host, void* z_perm,
                                  void* h1_save, void* a_save, void* ws,
                                  hipStream_t stream) {
  const int tn1 = (2 * F + BN - 1) / BN;
  const int tn2 = (H + BN - 1) / BN;
  char* wp = static_cast<char*>(ws);
  int32_t* t1 = reinterpret_cast<int32_t*>(wp);
  wp += align256((size_t)2 * E * sizeof(int32_t));
  int32_t* t2 = reinterpret_cast<int32_t*>(wp);
  wp += align256((size_t)2 * E * sizeof(int32_t));
  uint16_t* h1 = static_cast<uint16_t*>(h1_save);
  if (!h1) {
    h1 = reinterpret_cast<uint16_t*>(wp);
    wp += align256((size_t)rows * 2 * F * 2);
  }
  uint16_t* a = static_cast<uint16_t*>(a_save);
  if (!a) a = reinterpret_cast<uint16_t*>(wp);

  const int32_t* off = offsets_host;   // the row counts, read back
  hipError_t err;
  {
    KernelScope ks("loop_tile_tables", stream);
    hipLaunchKernelGGL(loop_tile_tables_kernel, dim3((E + 255) / 256),
                       dim3(256), 0, stream, offsets, E, tn1, tn2, t1, t2);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  auto grid = [](int tiles) { return (tiles + kXcds - 1) / kXcds * kXcds; };
  for (int e = 0; e < E; ++e) {
    const int64_t m = off[e + 1] - off[e];
    if (m == 0) continue;
    const int mt = (int)((m + BM - 1) / BM);
    // gate/up: h1 rows [off[e], off[e+1]) = X_e W_gu[e]^T
    Params p{};
    p.a = static_cast<const char*>(x_perm);
    p.lda = 2 * (int64_t)H;
    p.b = static_cast<const char*>(w_gu) + (int64_t)e * 2 * F * H * 2;
    p.ldb = 2 * (int64_t)H;
    p.b_rows = 2 * F;
    p.N = 2 * F;
    p.K = H;
    p.F = F;
    p.E = 1;
    p.offsets = offsets + e;
    p.tile_start = t1 + 2 * e;
    p.tiles_n = tn1;
    p.c = h1;
    p.ldc = 2 * F;
    p.rows = rows;
    err = launch<P_BF16, KC, KC, RAGGED_M, EPI_STORE>(
        "loop_gemm_gate_up", p, grid(mt * tn1), stream);
    if (err != hipSuccess) return err;
    {
      KernelScope ks("loop_swiglu", stream);
      const int64_t n = m * (F / 8);
      hipLaunchKernelGGL(loop_swiglu_kernel, dim3((unsigned)((n + 255) / 256)),
                         dim3(256), 0, stream, h1, w_perm, F,
                         (int64_t)off[e], m, a);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    // down: z rows = a_e W_dn[e]^T
    Params q{};
    q.a = reinterpret_cast<const char*>(a);
    q.lda = 2 * (int64_t)F;
    q.b = static_cast<const char*>(w_dn) + (int64_t)e * H * F * 2;
    q.ldb = 2 * (int64_t)F;
    q.b_rows = H;
    q.N = H;
    q.K = F;
    q.E = 1;
    q.offsets = offsets + e;
    q.tile_start = t2 + 2 * e;
    q.tiles_n = tn2;
    q.c = static_cast<uint16_t*>(z_perm);
    q.ldc = H;
    q.rows = rows;
    err = launch<P_BF16, KC, KC, RAGGED_M, EPI_STORE>(
        "loop_gemm_down", q, grid(mt * tn2), stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
