// Tensor-scaled FP8 forward of the expert MLP: x_perm, each expert's W_gu
// and W_dn, and the SwiGLU output A each carry one float32 scale (amax /
// 448; "NVIDIA presents an efficient path for training biological MoE
// models", section "Reducing memory and quantisation cost").  The grouped
// GEMMs run on E4M3 codes with unit MFMA scales and multiply the
// accumulators by the two tensor scales; the gate/up epilogue writes A in
// bf16 and its amax, then A is quantised with its own scale for the down
// GEMM.  Kernel: grouped_gemm.hpp (P_FP8T).
#include "grouped_gemm.hpp"
#include "grouped_gemm_w8q.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

using namespace gg;

struct Fp8tWs {
  uint32_t* amax;   // [2 + 2E]: x, A, W_gu[e], W_dn[e]
  float* scale;     // same order
  int32_t *ts1, *ts2;
  uint8_t *xq, *guq, *dnq, *aq;
  uint16_t* a;      // bf16 A (when a_save is NULL)
  int split_x;          // down GEMM: split slots per XCD
  float* split_part;    // down GEMM: partial tiles of a split tail
  uint32_t* split_cnt;  // down GEMM: arrival counters
  size_t bytes;
};

Fp8tWs carve(void* base, int E, int H, int F, int64_t rows, bool need_a,
             bool quant_w) {
  Fp8tWs w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t n) {
    char* q = p ? p + off : nullptr;
    off += align256(n);
    return q;
  };
  w.amax = reinterpret_cast<uint32_t*>(take((size_t)(2 + 2 * E) * 4));
  w.scale = reinterpret_cast<float*>(take((size_t)(2 + 2 * E) * 4));
  w.ts1 = reinterpret_cast<int32_t*>(take(tile_table_bytes(E, rows)));
  w.ts2 = reinterpret_cast<int32_t*>(take(tile_table_bytes(E, rows)));
  w.xq = reinterpret_cast<uint8_t*>(take((size_t)rows * H));
  if (quant_w) {
    w.guq = reinterpret_cast<uint8_t*>(take((size_t)E * 2 * F * H));
    w.dnq = reinterpret_cast<uint8_t*>(take((size_t)E * H * F));
  }
  w.aq = reinterpret_cast<uint8_t*>(take((size_t)rows * F));
  w.a = need_a ? reinterpret_cast<uint16_t*>(take((size_t)rows * F * 2))
               : nullptr;
  // K steps of 128 values
  w.split_x = split_slots_x((rows / BM + E) * (int64_t)((H + BN - 1) / BN),
                            F / 128);
  w.split_part = reinterpret_cast<float*>(take(split_part_bytes(w.split_x)));
  w.split_cnt = reinterpret_cast<uint32_t*>(take(split_cnt_bytes(w.split_x)));
  w.bytes = off;
  return w;
}

}  // namespace

size_t mlp_fwd_fp8t_ws_bytes(int E, int H, int F, int64_t rows, bool need_a,
                             bool quant_w) {
  return carve(nullptr, E, H, F, rows, need_a, quant_w).bytes;
}

hipError_t launch_mlp_fwd_fp8t(int E, int H, int F, int64_t rows,
                               const void* x_perm, const void* w_gu,
                               const void* w_dn, const uint8_t* w_gu_q,
                               const float* w_gu_ts, const uint8_t* w_dn_q,
                               const float* w_dn_ts, const float* w_perm,
                               const int32_t* offsets, void* z_perm,
                               void* h1_save, void* a_save, void* ws,
                               int cu_count, int32_t* status,
                               hipStream_t stream) {
  const bool quant_w = w_gu_q == nullptr;
  Fp8tWs w = carve(ws, E, H, F, rows, a_save == nullptr, quant_w);
  uint16_t* a = a_save ? static_cast<uint16_t*>(a_save) : w.a;
  // scale slots: 0 x, 1 A, 2 + e W_gu[e], 2 + E + e W_dn[e] (the weights'
  // slots unused when the caller passes their codes and scales)
  const uint8_t* guq = w_gu_q;
  const uint8_t* dnq = w_dn_q;
  const float* gus = w_gu_ts;
  const float* dns = w_dn_ts;
  hipError_t err = launch_zero_u32(w.amax, 2 + 2 * E, stream);
  if (quant_w) {
    guq = w.guq;
    dnq = w.dnq;
    gus = w.scale + 2;
    dns = w.scale + 2 + E;
    if (err == hipSuccess)
      err = launch_seg_amax(w_gu, (int64_t)2 * F * H, E, w.amax + 2, stream);
    if (err == hipSuccess)
      err = launch_seg_amax(w_dn, (int64_t)H * F, E, w.amax + 2 + E, stream);
    if (err == hipSuccess)
      err = launch_tensor_quant(w_gu, (int64_t)2 * F * H, E, w.amax + 2,
                                w.guq, w.scale + 2, stream);
    if (err == hipSuccess)
      err = launch_tensor_quant(w_dn, (int64_t)H * F, E, w.amax + 2 + E,
                                w.dnq, w.scale + 2 + E, stream);
  }
  if (err != hipSuccess || rows == 0) return err;
  err = launch_seg_amax(x_perm, rows * H, 1, w.amax, stream);
  if (err == hipSuccess)
    err = launch_tensor_quant(x_perm, rows * H, 1, w.amax, w.xq, w.scale,
                              stream);
  const int tn1 = (F + BN / 2 - 1) / (BN / 2);
  const int tn2 = (H + BN - 1) / BN;
  if (err == hipSuccess)
    err = launch_tile_table(offsets, E, rows, tn1, w.ts1, status, stream,
                            w.split_cnt, kXcds * w.split_x);
  if (err == hipSuccess)
    err = launch_tile_table(offsets, E, rows, tn2, w.ts2, status, stream);
  if (err != hipSuccess) return err;

  // gate/up + ScaledSwiGLU: A in bf16 (and its amax), (g, u) save optional
  Params p1{};
  p1.a = reinterpret_cast<const char*>(w.xq);
  p1.lda = H;
  p1.b = reinterpret_cast<const char*>(guq);
  p1.ldb = H;
  p1.b_es = (int64_t)2 * F * H;
  p1.N = 2 * F;
  p1.b_rows = 2 * F;
  p1.K = H;
  p1.F = F;
  p1.E = E;
  p1.offsets = offsets;
  p1.tile_start = w.ts1;
  p1.mrec = tile_records(w.ts1, E);
  p1.tiles_n = tn1;
  p1.c = a;
  p1.ldc = F;
  p1.c2 = static_cast<uint16_t*>(h1_save);
  p1.w = w_perm;
  p1.rows = rows;
  p1.tsa = w.scale;
  p1.tsb = gus;
  p1.amax_out = w.amax + 1;
  err = launch_w8q<P_FP8T, EPI_SWIGLU>(
      "gemm_gate_up_swiglu_fp8t", p1, ragged_m_grid(rows, E, tn1), stream);
  if (err == hipSuccess)
    err = launch_tensor_quant(a, rows * F, 1, w.amax + 1, w.aq, w.scale + 1,
                              stream);
  if (err != hipSuccess) return err;

  Params p2{};
  p2.a = reinterpret_cast<const char*>(w.aq);
  p2.lda = F;
  p2.b = reinterpret_cast<const char*>(dnq);
  p2.ldb = F;
  p2.b_es = (int64_t)H * F;
  p2.N = H;
  p2.b_rows = H;
  p2.K = F;
  p2.E = E;
  p2.offsets = offsets;
  p2.tile_start = w.ts2;
  p2.mrec = tile_records(w.ts2, E);
  p2.tiles_n = tn2;
  p2.c = static_cast<uint16_t*>(z_perm);
  p2.ldc = H;
  p2.rows = rows;
  p2.tsa = w.scale + 1;
  p2.tsb = dns;
  enable_split(p2, w.split_part, w.split_cnt, w.split_x, cu_count);
  return launch_w8q<P_FP8T, EPI_STORE>("gemm_down_fp8t", p2,
                            ragged_m_grid_split(rows, E, tn2, p2), stream);
}

}  // namespace moe
