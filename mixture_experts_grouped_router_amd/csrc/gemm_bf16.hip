// bf16 grouped GEMMs of the expert MLP, forward and backward.
//
// Forward: grouped gate/up GEMM with ScaledSwiGLU times the routing weight
// in its epilogue ("NVIDIA presents an efficient path for training
// biological MoE models", section "Reducing memory and quantisation cost":
// GroupedLinear -> ScaledSwiGLU -> GroupedLinear fused; section "Grouped
// experts instead of a Python loop": routing weights scaled inside the
// grouped MLP), then the grouped down GEMM.  Backward: the counterpart GEMMs
// (dgrad of both projections, the first with the SwiGLU backward and the
// routing-weight gradient in its epilogue; wgrad of both projections with K
// running over each expert's tokens).  Kernels: grouped_gemm.hpp, and for
// the forward GEMMs grouped_gemm_w8.hpp (eight waves per tile).
#include "grouped_gemm.hpp"
#include "grouped_gemm_w8.hpp"
#include "grouped_gemm_w8b.hpp"
#include "kernels.hpp"

namespace moe {
namespace gg {

// Prefix over experts: tile_start[e] = sum_{e' < e} ceil(M_e'/unit) * tn.
// With unit = BM it counts GEMM tiles; with unit = tn = P it gives the
// offsets of segments padded to multiples of P.  Offsets that do not run
// non-decreasing from 0 to rows give an all-zero table (no tile runs, every
// padded segment is empty) and record MOE_DEVERR_OFFSETS.  With mrec (GEMM
// tiles, unit = BM) thread e also writes the records of e's M tiles.
__global__ __launch_bounds__(1024) void tile_table_kernel(
    const int32_t* __restrict__ offsets, int E, int64_t rows, int unit,
    int tn, int32_t* __restrict__ tile_start, uint32_t* __restrict__ zero,
    int nzero, int32_t* status, int32_t* __restrict__ mrec) {
  __shared__ int32_t wsum[16];
  const int e = threadIdx.x;
  for (int i = e; i < nzero; i += 1024) zero[i] = 0u;
  if (__syncthreads_or(e < E && !offsets_pair_ok(offsets, e, E, rows))) {
    for (int i = e; i <= E; i += 1024) tile_start[i] = 0;
    if (e == 0) report_error(status, kDevErrOffsets);
    return;
  }
  const int lane = e & 63, wid = e >> 6;
  int32_t v = 0;
  if (e < E) v = ((offsets[e + 1] - offsets[e] + unit - 1) / unit) * tn;
  int32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  if (e == 0) {
    int32_t acc = 0;
    for (int w = 0; w < 16; ++w) {
      const int32_t s = wsum[w];
      wsum[w] = acc;
      acc += s;
    }
  }
  __syncthreads();
  const int32_t excl = incl - v + wsum[wid];
  if (e < E) tile_start[e] = excl;
  if (e == E - 1) tile_start[E] = excl + v;
  if (mrec && e < E && v > 0) {
    const int32_t first = excl / tn, n = v / tn;
    const int4 r = make_int4(e, first, offsets[e], offsets[e + 1] - offsets[e]);
    for (int i = 0; i < n; ++i)
      reinterpret_cast<int4*>(mrec)[first + i] = r;
  }
}

// Rank of expert e by rows, descending; equal counts keep index order.
// Invalid offsets (as in tile_table_kernel) give order[] = -1: every tile of
// a RAGGED_K launch then exits without work.
__global__ __launch_bounds__(1024) void expert_order_kernel(
    const int32_t* __restrict__ offsets, int E, int64_t rows,
    int32_t* __restrict__ order, int32_t* status) {
  __shared__ int32_t len[1024];
  const int e = threadIdx.x;
  if (__syncthreads_or(e < E && !offsets_pair_ok(offsets, e, E, rows))) {
    if (e < E) order[e] = -1;
    if (e == 0) report_error(status, kDevErrOffsets);
    return;
  }
  if (e < E) len[e] = offsets[e + 1] - offsets[e];
  __syncthreads();
  if (e >= E) return;
  const int le = len[e];
  int r = 0;
  for (int j = 0; j < E; ++j) {
    const int lj = len[j];
    r += (lj > le) | ((lj == le) & (j < e));
  }
  order[r] = e;
}

namespace {
// dw_perm[r] = sum over N tiles (ascending) of the partial row sums.
__global__ __launch_bounds__(256) void reduce_parts_kernel(
    const float* __restrict__ part, int nparts, int64_t rows,
    float* __restrict__ out) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  float s = 0.0f;
  for (int i = 0; i < nparts; ++i) s += part[(int64_t)i * rows + r];
  out[r] = s;
}
}  // namespace

hipError_t launch_tile_table(const int32_t* offsets, int E, int64_t rows,
                             int tn, int32_t* tile_start, int32_t* status,
                             hipStream_t stream, uint32_t* zero, int nzero) {
  KernelScope ks("tile_table", stream);
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, stream,
                     offsets, E, rows, BM, tn, tile_start, zero, nzero,
                     status, tile_start + tile_rec_offset(E));
  return hipGetLastError();
}

hipError_t launch_expert_order(const int32_t* offsets, int E, int64_t rows,
                               int32_t* order, int32_t* status,
                               hipStream_t stream) {
  KernelScope ks("expert_order", stream);
  hipLaunchKernelGGL(expert_order_kernel, dim3(1), dim3(1024), 0, stream,
                     offsets, E, rows, order, status);
  return hipGetLastError();
}

hipError_t launch_padded_offsets(const int32_t* offsets, int E, int64_t rows,
                                 int pad, int32_t* poff, int32_t* status,
                                 hipStream_t stream) {
  KernelScope ks("padded_offsets", stream);
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, stream,
                     offsets, E, rows, pad, pad, poff, nullptr, 0, status,
                     nullptr);
  return hipGetLastError();
}

}  // namespace gg

using namespace gg;

namespace {
// Split slots per XCD of the eight-wave forward GEMMs (the gate/up GEMM
// runs with eight waves up to H = kW8MaxGateUpK).
int fwd_split_slots_x(int E, int H, int F, int64_t rows) {
  const int64_t mt = rows / BM + E;
  const int tn1 = (F + BN / 2 - 1) / (BN / 2);
  const int tn2 = (H + BN - 1) / BN;
  int s = split_slots_x(mt * tn2, F / 64);
  if (H <= kW8MaxGateUpK) s = std::max(s, split_slots_x(mt * tn1, H / 64));
  return s;
}
}  // namespace

size_t mlp_fwd_bf16_ws_bytes(int E, int H, int F, int64_t rows, bool need_a) {
  size_t b = 2 * tile_table_bytes(E, rows);
  if (need_a) b += align256((size_t)rows * F * 2);
  const int sx = fwd_split_slots_x(E, H, F, rows);
  b += split_part_bytes(sx) + counters_bytes(1, sx);
  return b;
}

hipError_t launch_mlp_fwd_bf16(int E, int H, int F, int64_t rows,
                               const void* x_perm, const void* w_gu,
                               const void* w_dn, const float* w_perm,
                               const int32_t* offsets, void* z_perm,
                               void* h1_save, void* a_save, void* ws,
                               int cu_count, int32_t* status,
                               hipStream_t stream) {
  char* wp = static_cast<char*>(ws);
  int32_t* ts1 = reinterpret_cast<int32_t*>(wp);
  wp += tile_table_bytes(E, rows);
  int32_t* ts2 = reinterpret_cast<int32_t*>(wp);
  wp += tile_table_bytes(E, rows);
  uint16_t* a_buf = static_cast<uint16_t*>(a_save);
  if (!a_buf) {
    a_buf = reinterpret_cast<uint16_t*>(wp);
    wp += align256((size_t)rows * F * 2);
  }
  const int sx = fwd_split_slots_x(E, H, F, rows);
  float* split_part = reinterpret_cast<float*>(wp);
  wp += split_part_bytes(sx);
  // the gate/up GEMM's persistent-launch counters, then the split counters
  uint32_t* queues = reinterpret_cast<uint32_t*>(wp);
  uint32_t* split_cnt = queues + kQueueWords;
  if (rows == 0) return hipSuccess;

  const int tn1 = (F + BN / 2 - 1) / (BN / 2);
  const int tn2 = (H + BN - 1) / BN;
  hipError_t err = launch_tile_table(offsets, E, rows, tn1, ts1, status,
                                     stream, queues,
                                     kQueueWords + kXcds * sx);
  if (err == hipSuccess)
    err = launch_tile_table(offsets, E, rows, tn2, ts2, status, stream);
  if (err != hipSuccess) return err;
  // the eight-wave GEMMs split the last, partly filled round of tiles
  auto set_split = [&](Params& p) {
    enable_split(p, split_part, split_cnt, sx, cu_count);
  };

  Params p1{};
  p1.a = static_cast<const char*>(x_perm);
  p1.lda = 2 * (int64_t)H;
  p1.b = static_cast<const char*>(w_gu);
  p1.ldb = 2 * (int64_t)H;
  p1.b_es = (int64_t)4 * F * H;
  p1.N = 2 * F;
  p1.b_rows = 2 * F;
  p1.K = H;
  p1.F = F;
  p1.E = E;
  p1.offsets = offsets;
  p1.tile_start = ts1;
  p1.mrec = tile_records(ts1, E);
  p1.tiles_n = tn1;
  p1.c = a_buf;
  p1.ldc = F;
  p1.c2 = static_cast<uint16_t*>(h1_save);
  p1.w = w_perm;
  p1.rows = rows;
  // Eight waves per tile hide more latency but read 50% more LDS per MFMA;
  // up to H = kW8MaxGateUpK the latency gained pays for it (measured up
  // to H = 4096), above the four-wave kernel runs it.
  if (H <= kW8MaxGateUpK) {
    set_split(p1);
    p1.queue = queues;
    err = launch_w8<EPI_SWIGLU>(
        "gemm_gate_up_swiglu_bf16", p1,
        persistent_grid(cu_count, ragged_m_grid_split(rows, E, tn1, p1)),
        stream);
  } else {
    err = launch<P_BF16, KC, KC, RAGGED_M, EPI_SWIGLU>(
        "gemm_gate_up_swiglu_bf16", p1, ragged_m_grid(rows, E, tn1), stream);
  }
  if (err != hipSuccess) return err;

  Params p2{};
  p2.a = reinterpret_cast<const char*>(a_buf);
  p2.lda = 2 * (int64_t)F;
  p2.b = static_cast<const char*>(w_dn);
  p2.ldb = 2 * (int64_t)F;
  p2.b_es = (int64_t)2 * H * F;
  p2.N = H;
  p2.b_rows = H;
  p2.K = F;
  p2.E = E;
  p2.offsets = offsets;
  p2.tile_start = ts2;
  p2.mrec = tile_records(ts2, E);
  p2.tiles_n = tn2;
  p2.c = static_cast<uint16_t*>(z_perm);
  p2.ldc = H;
  p2.rows = rows;
  set_split(p2);
  return launch_w8<EPI_STORE>("gemm_down_bf16", p2,
                             ragged_m_grid_split(rows, E, tn2, p2), stream);
}

size_t mlp_bwd_bf16_ws_bytes(int E, int H, int F, int64_t rows) {
  const int tnf = (F + BN - 1) / BN;
  size_t b = 2 * tile_table_bytes(E, rows) +
             align256((size_t)(E + 1) * sizeof(int32_t));
  b += align256((size_t)rows * 2 * F * 2);        // dH1
  b += align256((size_t)tnf * rows * sizeof(float));  // dw partials
  return b;
}

hipError_t launch_mlp_bwd_bf16(int E, int H, int F, int64_t rows,
                               const void* x_perm, const void* w_gu,
                               const void* w_dn, const float* w_perm,
                               const int32_t* offsets, const void* h1_save,
                               const void* a_save, const void* dz_perm,
                               void* dx_perm, void* dw_gu, void* dw_dn,
                               float* dw_perm, void* ws, int32_t* status,
                               hipStream_t stream) {
  const int tnf = (F + BN - 1) / BN;
  const int tnh = (H + BN - 1) / BN;
  char* wp = static_cast<char*>(ws);
  int32_t* ts_f = reinterpret_cast<int32_t*>(wp);
  wp += tile_table_bytes(E, rows);
  int32_t* ts_h = reinterpret_cast<int32_t*>(wp);
  wp += tile_table_bytes(E, rows);
  int32_t* order = reinterpret_cast<int32_t*>(wp);
  wp += align256((size_t)(E + 1) * sizeof(int32_t));
  uint16_t* dh1 = reinterpret_cast<uint16_t*>(wp);
  wp += align256((size_t)rows * 2 * F * 2);
  float* part = reinterpret_cast<float*>(wp);

  hipError_t err;
  if (rows > 0) {
    err = launch_tile_table(offsets, E, rows, tnf, ts_f, status, stream);
    if (err == hipSuccess)
      err = launch_tile_table(offsets, E, rows, tnh, ts_h, status, stream);
    if (err != hipSuccess) return err;
    // dgrad2 + SwiGLU backward: dA = dZ W_dn[e]  (B = W_dn[e] [H, F] is
    // N-contiguous)
    Params p{};
    p.a = static_cast<const char*>(dz_perm);
    p.lda = 2 * (int64_t)H;
    p.b = static_cast<const char*>(w_dn);
    p.ldb = 2 * (int64_t)F;
    p.b_es = (int64_t)2 * H * F;
    p.N = F;
    p.K = H;
    p.F = F;
    p.E = E;
    p.offsets = offsets;
    p.tile_start = ts_f;
    p.mrec = tile_records(ts_f, E);
    p.tiles_n = tnf;
    p.c = dh1;
    p.h1 = static_cast<const uint16_t*>(h1_save);
    p.w = w_perm;
    p.dw_part = dw_perm ? part : nullptr;
    p.rows = rows;
    err = launch_w8b<KC, MC, RAGGED_M, EPI_SWIGLU_BWD>(
        "gemm_dgrad_down_swiglu_bwd", p, ragged_m_grid(rows, E, tnf),
                                                   stream);
    if (err != hipSuccess) return err;
    if (dw_perm) {
      KernelScope ks("routing_weight_grad_reduce", stream);
      hipLaunchKernelGGL(reduce_parts_kernel, dim3((unsigned)((rows + 255) / 256)),
                         dim3(256), 0, stream, part, tnf, rows, dw_perm);
    }
    // dgrad1: dX = dH1 W_gu[e]  (B = W_gu[e] [2F, H] is N-contiguous)
    Params q{};
    q.a = reinterpret_cast<const char*>(dh1);
    q.lda = 4 * (int64_t)F;
    q.b = static_cast<const char*>(w_gu);
    q.ldb = 2 * (int64_t)H;
    q.b_es = (int64_t)4 * F * H;
    q.N = H;
    q.K = 2 * F;
    q.E = E;
    q.offsets = offsets;
    q.tile_start = ts_h;
    q.mrec = tile_records(ts_h, E);
    q.tiles_n = tnh;
    q.c = static_cast<uint16_t*>(dx_perm);
    q.ldc = H;
    q.rows = rows;
    err = launch_w8b<KC, MC, RAGGED_M>("gemm_dgrad_gate_up", q,
                                       ragged_m_grid(rows, E, tnh), stream);
    if (err != hipSuccess) return err;
  }
  // wgrad2: dW_dn[e] [H, F] = dZ_e^T A_e   (K = rows of expert e)
  err = launch_expert_order(offsets, E, rows, order, status, stream);
  if (err != hipSuccess) return err;
  {
    Params p{};
    p.order = order;
    p.a = static_cast<const char*>(dz_perm);
    p.lda = 2 * (int64_t)H;
    p.b = static_cast<const char*>(a_save);
    p.ldb = 2 * (int64_t)F;
    p.M = H;
    p.N = F;
    p.E = E;
    p.offsets = offsets;
    p.tiles_m = (H + BM - 1) / BM;
    p.tiles_n = (F + BN - 1) / BN;
    p.c = static_cast<uint16_t*>(dw_dn);
    p.ldc = F;
    p.c_es = (int64_t)H * F;
    p.rows = rows;
    const int grid = ragged_k_grid(E, p.tiles_m, p.tiles_n);
    err = launch_w8b<MC, MC, RAGGED_K>("gemm_wgrad_down", p, grid, stream);
    if (err != hipSuccess) return err;
  }
  // wgrad1: dW_gu[e] [2F, H] = dH1_e^T X_e
  {
    Params p{};
    p.order = order;
    p.a = reinterpret_cast<const char*>(dh1);
    p.lda = 4 * (int64_t)F;
    p.b = static_cast<const char*>(x_perm);
    p.ldb = 2 * (int64_t)H;
    p.M = 2 * F;
    p.N = H;
    p.E = E;
    p.offsets = offsets;
    p.tiles_m = (2 * F + BM - 1) / BM;
    p.tiles_n = (H + BN - 1) / BN;
    p.c = static_cast<uint16_t*>(dw_gu);
    p.ldc = H;
    p.c_es = (int64_t)2 * F * H;
    p.rows = rows;
    const int grid = ragged_k_grid(E, p.tiles_m, p.tiles_n);
    err = launch_w8b<MC, MC, RAGGED_K>("gemm_wgrad_gate_up", p, grid, stream);
  }
  return err;
}

}  // namespace moe
