// MXFP8 grouped MLP forward: E4M3 operands with one E8M0 scale per 32
// consecutive values along each GEMM's K ("NVIDIA presents an efficient path
// for training biological MoE models", section "Reducing memory and
// quantisation cost"; "Efficient MoE training for biological foundation
// models (NVIDIA)", sections "2) Model size and activation memory" and
// "3) Quantisation overhead in low-precision training").
//
//   x_perm (codes from the permute, or quantised here)  x  W_gu (quantised
//   from the bf16 masters here unless the caller passes codes)
//     -> scaled-MFMA grouped GEMM, float32 accumulate
//     -> epilogue: ScaledSwiGLU x routing weight in float32, then row-wise
//        MXFP8 quantisation of A along F (one half-wave = one block of 32)
//   A codes  x  W_dn codes -> scaled-MFMA grouped GEMM -> bf16 Z
// Kernel: grouped_gemm.hpp.
#include "grouped_gemm.hpp"
#include "kernels.hpp"

namespace moe {

using namespace gg;

namespace {

struct MxFwdWs {
  int32_t* ts1;
  int32_t* ts2;
  uint8_t* aq;   // A codes [rows, F]
  uint8_t* as;   // A scales [rows, F/32]
  uint8_t* xq;   // x_perm codes [rows, H] (quantised here)
  uint8_t* xs;
  uint8_t* guq;  // W_gu codes [E, 2F, H]
  uint8_t* gus;
  uint8_t* dnq;  // W_dn codes [E, H, F]
  uint8_t* dns;
  size_t bytes;
};

MxFwdWs carve_fwd(void* base, int E, int H, int F, int64_t rows, bool quant_x,
                  bool quant_w) {
  MxFwdWs w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t n) {
    char* q = p ? p + off : nullptr;
    off += align256(n);
    return q;
  };
  w.ts1 = reinterpret_cast<int32_t*>(take((size_t)(E + 1) * 4));
  w.ts2 = reinterpret_cast<int32_t*>(take((size_t)(E + 1) * 4));
  w.aq = reinterpret_cast<uint8_t*>(take((size_t)rows * F));
  w.as = reinterpret_cast<uint8_t*>(take((size_t)rows * F / 32));
  if (quant_x) {
    w.xq = reinterpret_cast<uint8_t*>(take((size_t)rows * H));
    w.xs = reinterpret_cast<uint8_t*>(take((size_t)rows * H / 32));
  }
  if (quant_w) {
    const size_t ngu = (size_t)E * 2 * F * H, ndn = (size_t)E * H * F;
    w.guq = reinterpret_cast<uint8_t*>(take(ngu));
    w.gus = reinterpret_cast<uint8_t*>(take(ngu / 32));
    w.dnq = reinterpret_cast<uint8_t*>(take(ndn));
    w.dns = reinterpret_cast<uint8_t*>(take(ndn / 32));
  }
  w.bytes = off;
  return w;
}

}  // namespace

size_t mlp_fwd_mx_ws_bytes(int E, int H, int F, int64_t rows, bool quant_x,
                           bool quant_w) {
  return carve_fwd(nullptr, E, H, F, rows, quant_x, quant_w).bytes;
}

hipError_t launch_mlp_fwd_mx(int E, int H, int F, int64_t rows,
                             const void* x_perm_bf16, const uint8_t* xq,
                             const uint8_t* xs, const void* w_gu,
                             const void* w_dn, const uint8_t* w_gu_q,
                             const uint8_t* w_gu_s, const uint8_t* w_dn_q,
                             const uint8_t* w_dn_s, const float* w_perm,
                             const int32_t* offsets, void* z_perm,
                             void* h1_save, void* a_save, void* ws,
                             hipStream_t stream) {
  const bool quant_x = xq == nullptr;
  const bool quant_w = w_gu_q == nullptr || w_dn_q == nullptr;
  MxFwdWs w = carve_fwd(ws, E, H, F, rows, quant_x, quant_w);
  hipError_t err = hipSuccess;
  if (quant_w) {
    err = launch_mx_quant_rows(w_gu, (int64_t)E * 2 * F, H, w.guq, w.gus,
                               stream);
    if (err == hipSuccess)
      err = launch_mx_quant_rows(w_dn, (int64_t)E * H, F, w.dnq, w.dns,
                                 stream);
    if (err != hipSuccess) return err;
    w_gu_q = w.guq; w_gu_s = w.gus; w_dn_q = w.dnq; w_dn_s = w.dns;
  }
  if (rows == 0) return hipSuccess;
  if (quant_x) {
    err = launch_mx_quant_rows(x_perm_bf16, rows, H, w.xq, w.xs, stream);
    if (err != hipSuccess) return err;
    xq = w.xq; xs = w.xs;
  }
  const int tn1 = (F + BN / 2 - 1) / (BN / 2);
  const int tn2 = (H + BN - 1) / BN;
  err = launch_tile_table(offsets, E, tn1, w.ts1, stream);
  if (err == hipSuccess) err = launch_tile_table(offsets, E, tn2, w.ts2, stream);
  if (err != hipSuccess) return err;

  Params p1{};
  p1.a = reinterpret_cast<const char*>(xq);
  p1.lda = H;
  p1.sa = xs;
  p1.ldsa = H / 32;
  p1.b = reinterpret_cast<const char*>(w_gu_q);
  p1.ldb = H;
  p1.b_es = (int64_t)2 * F * H;
  p1.sb = w_gu_s;
  p1.ldsb = H / 32;
  p1.sb_es = (int64_t)2 * F * H / 32;
  p1.N = 2 * F;
  p1.b_rows = 2 * F;
  p1.K = H;
  p1.F = F;
  p1.E = E;
  p1.offsets = offsets;
  p1.tile_start = w.ts1;
  p1.tiles_n = tn1;
  p1.c = static_cast<uint16_t*>(a_save);
  p1.ldc = F;
  p1.c2 = static_cast<uint16_t*>(h1_save);
  p1.cq = w.aq;
  p1.cs = w.as;
  p1.w = w_perm;
  p1.rows = rows;
  err = launch<P_FP8, KC, KC, RAGGED_M, EPI_SWIGLU_MX>(
      "gemm_gate_up_swiglu_mxfp8", p1, ragged_m_grid(rows, E, tn1), stream);
  if (err != hipSuccess) return err;

  Params p2{};
  p2.a = reinterpret_cast<const char*>(w.aq);
  p2.lda = F;
  p2.sa = w.as;
  p2.ldsa = F / 32;
  p2.b = reinterpret_cast<const char*>(w_dn_q);
  p2.ldb = F;
  p2.b_es = (int64_t)H * F;
  p2.sb = w_dn_s;
  p2.ldsb = F / 32;
  p2.sb_es = (int64_t)H * F / 32;
  p2.N = H;
  p2.b_rows = H;
  p2.K = F;
  p2.E = E;
  p2.offsets = offsets;
  p2.tile_start = w.ts2;
  p2.tiles_n = tn2;
  p2.c = static_cast<uint16_t*>(z_perm);
  p2.ldc = H;
  p2.rows = rows;
  return launch<P_FP8, KC, KC, RAGGED_M, EPI_STORE>(
      "gemm_down_mxfp8", p2, ragged_m_grid(rows, E, tn2), stream);
}

size_t mlp_bwd_mx_ws_bytes(int, int, int, int64_t) { return 256; }
hipError_t launch_mlp_bwd_mx(int, int, int, int64_t, const void*, const void*,
                             const void*, const float*, const int32_t*,
                             const void*, const void*, const void*, void*,
                             void*, void*, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moe
