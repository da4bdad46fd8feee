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
// Backward: below.  Kernel: grouped_gemm.hpp.
#include "grouped_gemm.hpp"
#include "grouped_gemm_w8q.hpp"
#include "kernels.hpp"

namespace moe {

using namespace gg;

namespace {

struct MxFwdWs {
  int32_t* ts1;
  int32_t* ts2;
  uint8_t* aq;   // A codes [rows, F]
  uint8_t* as;   // A scales (GEMM layout, K = F)
  uint8_t* xq;   // x_perm codes [rows, H] (quantised here)
  uint8_t* xs;   // x_perm scales (GEMM layout, K = H)
  uint8_t* guq;  // W_gu codes [E, 2F, H] (quantised here)
  uint8_t* gus;  // W_gu scales (GEMM layout, K = H)
  uint8_t* dnq;  // W_dn codes [E, H, F] (quantised here)
  uint8_t* dns;  // W_dn scales (GEMM layout, K = F)
  int split_x;          // down GEMM: split slots per XCD
  float* split_part;    // down GEMM: partial tiles of a split tail
  uint32_t* split_cnt;  // down GEMM: arrival counters
  size_t bytes;
};

// Scales always live here in the GEMM layout: quantised in the call, or
// rearranged from the caller's row-major scales.
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
  auto take8 = [&](size_t n) { return reinterpret_cast<uint8_t*>(take(n)); };
  w.ts1 = reinterpret_cast<int32_t*>(take(tile_table_bytes(E, rows)));
  w.ts2 = reinterpret_cast<int32_t*>(take(tile_table_bytes(E, rows)));
  w.aq = take8((size_t)rows * F);
  w.as = take8(mx_tile_bytes(rows, F));
  if (quant_x) w.xq = take8((size_t)rows * H);
  w.xs = take8(mx_tile_bytes(rows, H));
  const size_t ngu = (size_t)E * 2 * F * H, ndn = (size_t)E * H * F;
  if (quant_w) {
    w.guq = take8(ngu);
    w.dnq = take8(ndn);
  }
  w.gus = take8(ngu / 32);
  w.dns = take8(ndn / 32);
  // K steps of 128 values
  w.split_x = split_slots_x((rows / BM + E) * (int64_t)((H + BN - 1) / BN),
                            F / 128);
  w.split_part = reinterpret_cast<float*>(take(split_part_bytes(w.split_x)));
  w.split_cnt = reinterpret_cast<uint32_t*>(take(split_cnt_bytes(w.split_x)));
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
                             void* h1_save, void* a_save, uint8_t* a_q_save,
                             uint8_t* a_s_save, void* ws, int cu_count,
                             int32_t* status, hipStream_t stream) {
  const bool quant_x = xq == nullptr;
  const bool quant_w = w_gu_q == nullptr || w_dn_q == nullptr;
  MxFwdWs w = carve_fwd(ws, E, H, F, rows, quant_x, quant_w);
  // A's codes go to the caller's buffer when it keeps them
  if (a_q_save) w.aq = a_q_save;
  hipError_t err = hipSuccess;
  const int64_t ngu = (int64_t)E * 2 * F, ndn = (int64_t)E * H;  // rows
  if (quant_w) {
    err = launch_mx_quant_rows(w_gu, ngu, H, w.guq, w.gus, stream, true);
    if (err == hipSuccess)
      err = launch_mx_quant_rows(w_dn, ndn, F, w.dnq, w.dns, stream, true);
    w_gu_q = w.guq;
    w_dn_q = w.dnq;
  } else {
    err = launch_mx_scales_retile(w_gu_s, ngu, H, w.gus, stream);
    if (err == hipSuccess)
      err = launch_mx_scales_retile(w_dn_s, ndn, F, w.dns, stream);
  }
  if (err != hipSuccess) return err;
  if (rows == 0) return hipSuccess;
  if (quant_x) {
    err = launch_mx_quant_rows(x_perm_bf16, rows, H, w.xq, w.xs, stream,
                               true);
    xq = w.xq;
  } else {
    err = launch_mx_scales_retile(xs, rows, H, w.xs, stream);
  }
  if (err != hipSuccess) return err;
  const int tn1 = (F + BN / 2 - 1) / (BN / 2);
  const int tn2 = (H + BN - 1) / BN;
  err = launch_tile_table(offsets, E, rows, tn1, w.ts1, status, stream,
                          w.split_cnt, kXcds * w.split_x);
  if (err == hipSuccess)
    err = launch_tile_table(offsets, E, rows, tn2, w.ts2, status, stream);
  if (err != hipSuccess) return err;

  Params p1{};
  p1.a = reinterpret_cast<const char*>(xq);
  p1.lda = H;
  p1.sa = w.xs;
  p1.ldsa = H / 128;
  p1.b = reinterpret_cast<const char*>(w_gu_q);
  p1.ldb = H;
  p1.b_es = (int64_t)2 * F * H;
  p1.sb = w.gus;
  p1.ldsb = H / 128;
  p1.sb_es = (int64_t)2 * F * H / 32;
  p1.N = 2 * F;
  p1.b_rows = 2 * F;
  p1.K = H;
  p1.F = F;
  p1.E = E;
  p1.offsets = offsets;
  p1.tile_start = w.ts1;
  p1.mrec = tile_records(w.ts1, E);
  p1.tiles_n = tn1;
  p1.c = static_cast<uint16_t*>(a_save);
  p1.ldc = F;
  p1.c2 = static_cast<uint16_t*>(h1_save);
  p1.cq = w.aq;
  p1.cs = w.as;
  p1.cs_rm = a_s_save;
  p1.w = w_perm;
  p1.rows = rows;
  err = launch_w8q<P_FP8, EPI_SWIGLU_MX>(
      "gemm_gate_up_swiglu_mxfp8", p1, ragged_m_grid(rows, E, tn1), stream);
  if (err != hipSuccess) return err;

  Params p2{};
  p2.a = reinterpret_cast<const char*>(w.aq);
  p2.lda = F;
  p2.sa = w.as;
  p2.ldsa = F / 128;
  p2.b = reinterpret_cast<const char*>(w_dn_q);
  p2.ldb = F;
  p2.b_es = (int64_t)H * F;
  p2.sb = w.dns;
  p2.ldsb = F / 128;
  p2.sb_es = (int64_t)H * F / 32;
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
  enable_split(p2, w.split_part, w.split_cnt, w.split_x, cu_count);
  return launch_w8q<P_FP8, EPI_STORE>("gemm_down_mxfp8", p2,
                           ragged_m_grid_split(rows, E, tn2, p2), stream);
}

// ---- backward ----------------------------------------------------------------
// Every GEMM operand is quantised along that GEMM's K:
//   dgrad2  dA  = Q_H(dZ) Q_H(W_dn)     dZ row-wise, W_dn [H, F] blocks along H
//   dgrad1  dX  = Q_2F(dH1) Q_2F(W_gu)  dH1 row-wise, W_gu [2F, H] along 2F
//   wgrad2  dW_dn = Q_tok(dZ)^T Q_tok(A)
//   wgrad1  dW_gu = Q_tok(dH1)^T Q_tok(X)
// Token-direction blocks restart at each expert's first row and the last one
// is zero-padded.  Here each expert's token range is padded to whole K steps
// of the GEMM (128): the extra blocks are all zero, so the products are those
// of the 32-padded layout.  The SwiGLU backward runs in float32 in the dgrad2
// epilogue, which writes dH1 in bf16; dH1 is quantised from that bf16 copy.
// dZ and dH1 are each quantised in both directions by one pass that reads
// them once.
namespace {

constexpr int kTokPad = 128;   // token segments padded to one K step

struct MxBwdWs {
  int32_t* ts_f;   // tile prefix, N = F
  int32_t* ts_h;   // tile prefix, N = H
  int32_t* poff;   // padded token offsets [E+1]
  int32_t* order;  // experts by decreasing rows
  uint16_t* dh1;   // bf16 [rows, 2F]
  float* part;     // dw partial sums [tiles along F][rows]
  // codes, and scales in the GEMM layout
  uint8_t *dzq, *dzs;      // dZ row-wise [rows, H]
  uint8_t *wdq, *wds;      // W_dn blocks along H: [E, F, H]
  uint8_t *wgq, *wgs;      // W_gu blocks along 2F: [E, H, 2F]
  uint8_t *hq, *hs;        // dH1 row-wise [rows, 2F]
  uint8_t *dzt, *dzts;     // dZ token-wise [H, ld]
  uint8_t *at, *ats;       // A token-wise [F, ld]
  uint8_t *ht, *hts;       // dH1 token-wise [2F, ld]
  uint8_t *xt, *xts;       // X token-wise [H, ld]
  int64_t ld;              // padded token columns
  size_t bytes;
};

int64_t tok_ld(int64_t rows, int E) {
  // sum_e ceil(n_e / 128) * 128 <= rows + 127 E
  return (rows + (int64_t)kTokPad * E + kTokPad - 1) / kTokPad * kTokPad;
}

MxBwdWs carve_bwd(void* base, int E, int H, int F, int64_t rows,
                  bool quant_w) {
  MxBwdWs w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t n) {
    char* q = p ? p + off : nullptr;
    off += align256(n);
    return q;
  };
  auto take8 = [&](size_t n) { return reinterpret_cast<uint8_t*>(take(n)); };
  const int tnf = (F + BN - 1) / BN;
  const size_t F2 = 2 * (size_t)F;
  w.ld = tok_ld(rows, E);
  const size_t ld = (size_t)w.ld;
  w.ts_f = reinterpret_cast<int32_t*>(take(tile_table_bytes(E, rows)));
  w.ts_h = reinterpret_cast<int32_t*>(take(tile_table_bytes(E, rows)));
  w.poff = reinterpret_cast<int32_t*>(take((size_t)(E + 1) * 4));
  w.order = reinterpret_cast<int32_t*>(take((size_t)(E + 1) * 4));
  w.dh1 = reinterpret_cast<uint16_t*>(take((size_t)rows * F2 * 2));
  w.part = reinterpret_cast<float*>(take((size_t)tnf * rows * 4));
  w.dzq = take8((size_t)rows * H);
  w.dzs = take8(mx_tile_bytes(rows, H));
  if (quant_w) w.wdq = take8((size_t)E * H * F);
  w.wds = take8((size_t)E * H * F / 32);
  if (quant_w) w.wgq = take8((size_t)E * F2 * H);
  w.wgs = take8((size_t)E * F2 * H / 32);
  w.hq = take8((size_t)rows * F2);
  w.hs = take8(mx_tile_bytes(rows, F2));
  w.dzt = take8((size_t)H * ld);
  w.dzts = take8((size_t)H * ld / 32);
  w.at = take8((size_t)F * ld);
  w.ats = take8((size_t)F * ld / 32);
  w.ht = take8(F2 * ld);
  w.hts = take8(F2 * ld / 32);
  w.xt = take8((size_t)H * ld);
  w.xts = take8((size_t)H * ld / 32);
  w.bytes = off;
  return w;
}

// dw_perm[r] = sum over N tiles (ascending) of the partial row sums.
__global__ __launch_bounds__(256) void mx_reduce_parts_kernel(
    const float* __restrict__ part, int nparts, int64_t rows,
    float* __restrict__ out) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  float s = 0.0f;
  for (int i = 0; i < nparts; ++i) s += part[(int64_t)i * rows + r];
  out[r] = s;
}

// Token-direction GEMM dW[e] [M, N] = sum over the expert's padded tokens of
// At[m][tok] Bt[n][tok] (both quantised along tokens).
hipError_t wgrad_mx(const char* name, int E, int M, int N, int64_t ld,
                    const int32_t* poff, const int32_t* order,
                    const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                    const uint8_t* bs, void* dw, hipStream_t stream) {
  Params p{};
  p.order = order;
  p.a = reinterpret_cast<const char*>(aq);
  p.lda = ld;
  p.sa = as;
  p.ldsa = ld / 128;
  p.b = reinterpret_cast<const char*>(bq);
  p.ldb = ld;
  p.sb = bs;
  p.ldsb = ld / 128;
  p.b_rows = N;
  p.M = M;
  p.N = N;
  p.E = E;
  p.offsets = poff;
  p.tiles_m = (M + BM - 1) / BM;
  p.tiles_n = (N + BN - 1) / BN;
  p.c = static_cast<uint16_t*>(dw);
  p.ldc = N;
  p.c_es = (int64_t)M * N;
  return launch_w8q<P_FP8, EPI_STORE, RAGGED_K>(
      name, p, ragged_k_grid(E, p.tiles_m, p.tiles_n), stream);
}

}  // namespace

size_t mlp_bwd_mx_ws_bytes(int E, int H, int F, int64_t rows, bool quant_w) {
  return carve_bwd(nullptr, E, H, F, rows, quant_w).bytes;
}

hipError_t launch_mlp_bwd_mx(int E, int H, int F, int64_t rows,
                             const void* x_perm, const void* w_gu,
                             const void* w_dn, const float* w_perm,
                             const int32_t* offsets, const void* h1_save,
                             const void* a_save, const void* dz_perm,
                             void* dx_perm, void* dw_gu, void* dw_dn,
                             float* dw_perm, const uint8_t* w_gu_qt,
                             const uint8_t* w_gu_st, const uint8_t* w_dn_qt,
                             const uint8_t* w_dn_st, void* ws,
                             int32_t* status, hipStream_t stream) {
  // the weights' codes along the dgrad GEMMs' K come from the caller
  // (quantised once per weight update) or are made here
  const bool quant_w = w_gu_qt == nullptr || w_dn_qt == nullptr;
  MxBwdWs w = carve_bwd(ws, E, H, F, rows, quant_w);
  const int tnf = (F + BN - 1) / BN;
  const int tnh = (H + BN - 1) / BN;
  const int F2 = 2 * F;
  hipError_t err = launch_padded_offsets(offsets, E, rows, kTokPad, w.poff,
                                         status, stream);
  if (err == hipSuccess)
    err = launch_expert_order(offsets, E, rows, w.order, status, stream);
  if (rows > 0) {
    if (err == hipSuccess)
      err = launch_tile_table(offsets, E, rows, tnf, w.ts_f, status, stream);
    if (err == hipSuccess)
      err = launch_tile_table(offsets, E, rows, tnh, w.ts_h, status, stream);
    // dZ for dgrad2 (row-wise) and wgrad2 (along tokens)
    if (err == hipSuccess)
      err = launch_mx_quant_segments(dz_perm, rows, H, offsets, E, kTokPad,
                                     w.ld, w.dzt, w.dzts, status, stream,
                                     true, w.dzq, w.dzs);
    if (quant_w) {
      if (err == hipSuccess)
        err = launch_mx_quant_cols(w_dn, E, H, F, w.wdq, w.wds, stream, true);
      if (err == hipSuccess)
        err = launch_mx_quant_cols(w_gu, E, F2, H, w.wgq, w.wgs, stream, true);
    } else {
      // row-major scales of the caller's codes -> the GEMM layout
      w.wdq = const_cast<uint8_t*>(w_dn_qt);
      w.wgq = const_cast<uint8_t*>(w_gu_qt);
      if (err == hipSuccess)
        err = launch_mx_scales_retile(w_dn_st, (int64_t)E * F, H, w.wds,
                                      stream);
      if (err == hipSuccess)
        err = launch_mx_scales_retile(w_gu_st, (int64_t)E * H, F2, w.wgs,
                                      stream);
    }
    if (err != hipSuccess) return err;

    // dgrad2 + SwiGLU backward: dA = dZ W_dn[e]; B = W_dn[e]^T [F, H]
    Params p{};
    p.a = reinterpret_cast<const char*>(w.dzq);
    p.lda = H;
    p.sa = w.dzs;
    p.ldsa = H / 128;
    p.b = reinterpret_cast<const char*>(w.wdq);
    p.ldb = H;
    p.b_es = (int64_t)F * H;
    p.sb = w.wds;
    p.ldsb = H / 128;
    p.sb_es = (int64_t)F * H / 32;
    p.b_rows = F;
    p.N = F;
    p.K = H;
    p.F = F;
    p.E = E;
    p.offsets = offsets;
    p.tile_start = w.ts_f;
    p.mrec = tile_records(w.ts_f, E);
    p.tiles_n = tnf;
    p.c = w.dh1;
    p.h1 = static_cast<const uint16_t*>(h1_save);
    p.w = w_perm;
    p.dw_part = dw_perm ? w.part : nullptr;
    p.rows = rows;
    err = launch<P_FP8, KC, KC, RAGGED_M, EPI_SWIGLU_BWD>(
        "gemm_dgrad_down_swiglu_bwd_mxfp8", p, ragged_m_grid(rows, E, tnf),
        stream);
    if (err != hipSuccess) return err;
    if (dw_perm) {
      KernelScope ks("routing_weight_grad_reduce", stream);
      hipLaunchKernelGGL(mx_reduce_parts_kernel,
                         dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                         stream, w.part, tnf, rows, dw_perm);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }

    // dgrad1: dX = dH1 W_gu[e]; B = W_gu[e]^T [H, 2F]; dH1 for it
    // (row-wise) and for wgrad1 (along tokens)
    err = launch_mx_quant_segments(w.dh1, rows, F2, offsets, E, kTokPad,
                                   w.ld, w.ht, w.hts, status, stream, true,
                                   w.hq, w.hs);
    if (err != hipSuccess) return err;
    Params q{};
    q.a = reinterpret_cast<const char*>(w.hq);
    q.lda = F2;
    q.sa = w.hs;
    q.ldsa = F2 / 128;
    q.b = reinterpret_cast<const char*>(w.wgq);
    q.ldb = F2;
    q.b_es = (int64_t)H * F2;
    q.sb = w.wgs;
    q.ldsb = F2 / 128;
    q.sb_es = (int64_t)H * F2 / 32;
    q.b_rows = H;
    q.N = H;
    q.K = F2;
    q.E = E;
    q.offsets = offsets;
    q.tile_start = w.ts_h;
    q.mrec = tile_records(w.ts_h, E);
    q.tiles_n = tnh;
    q.c = static_cast<uint16_t*>(dx_perm);
    q.ldc = H;
    q.rows = rows;
    err = launch_w8q<P_FP8, EPI_STORE>(
        "gemm_dgrad_gate_up_mxfp8", q, ragged_m_grid(rows, E, tnh), stream);
    if (err != hipSuccess) return err;

    // the other token-direction operands of the two wgrad GEMMs
    err = launch_mx_quant_segments(a_save, rows, F, offsets, E, kTokPad,
                                   w.ld, w.at, w.ats, status, stream, true);
    if (err == hipSuccess)
      err = launch_mx_quant_segments(x_perm, rows, H, offsets, E, kTokPad,
                                     w.ld, w.xt, w.xts, status, stream, true);
  }
  if (err != hipSuccess) return err;
  // wgrad: every expert gets a tile set; K = its padded token count (0 for
  // an expert without rows, whose weight gradient is then stored as zeros)
  err = wgrad_mx("gemm_wgrad_down_mxfp8", E, H, F, w.ld, w.poff, w.order, w.dzt,
                 w.dzts, w.at, w.ats, dw_dn, stream);
  if (err == hipSuccess)
    err = wgrad_mx("gemm_wgrad_gate_up_mxfp8", E, F2, H, w.ld, w.poff, w.order, w.ht,
                   w.hts, w.xt, w.xts, dw_gu, stream);
  return err;
}

}  // namespace moe
