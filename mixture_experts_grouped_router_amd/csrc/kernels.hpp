// Internal launch wrappers of libmoe (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// router top-k
hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k,
                             int renorm, int32_t* idx, float* w,
                             int32_t* status, hipStream_t stream);

// permutation
size_t permute_ws_bytes(int64_t T, int E, int k);
// the static scratch of moe_permute_noalloc: its size, and its device address
// on `device` (which must be current; looked up once per device)
size_t permute_scratch_bytes();
hipError_t permute_scratch_address(int device, void** out);
hipError_t launch_permute_index(const int32_t* topk_idx, int64_t T, int E,
                                int k, int32_t* row_map, int32_t* src_row,
                                int32_t* split, int32_t* offsets, void* ws,
                                int32_t* status, hipStream_t stream);
hipError_t launch_gather_rows(const void* x, const int32_t* row_map,
                              const float* topk_w, int64_t T, int H, int k,
                              void* x_perm, float* w_perm, hipStream_t stream);
hipError_t launch_gather_rows_mx(const void* x, const int32_t* row_map,
                                 const float* topk_w, int64_t T, int H, int k,
                                 uint8_t* codes, uint8_t* scales,
                                 float* w_perm, hipStream_t stream);
hipError_t launch_unpermute(const void* z, const int32_t* row_map,
                            const float* topk_w, int64_t T, int H, int k,
                            void* y, hipStream_t stream);
hipError_t launch_probs_grad(const float* dw_perm, const int32_t* row_map,
                             int64_t T, int k, float* dprobs,
                             hipStream_t stream);

// MXFP8 quantisation.  tiled: scales in the GEMM layout (mx_tile_off;
// K = cols for rows, K = rows / ld for the transposed outputs, which then
// must be multiples of 128); otherwise row-major [rows][K / 32].
hipError_t launch_mx_quant_rows(const void* src, int64_t rows, int64_t cols,
                                uint8_t* codes, uint8_t* scales,
                                hipStream_t stream, bool tiled = false);
hipError_t launch_mx_quant_cols(const void* src, int64_t batch, int64_t rows,
                                int64_t cols, uint8_t* codes, uint8_t* scales,
                                hipStream_t stream, bool tiled = false);
// pad: segments start at multiples of pad (a multiple of 32) in the output.
// row_codes / row_scales (optional; pad and cols multiples of 128, tiled
// scales): the same pass also writes the row-wise quantisation, codes
// [rows][cols] and scales in the GEMM layout.
hipError_t launch_mx_quant_segments(const void* src, int64_t rows,
                                    int64_t cols, const int32_t* seg_offsets,
                                    int n_seg, int pad, int64_t ld,
                                    uint8_t* codes, uint8_t* scales,
                                    int32_t* status, hipStream_t stream,
                                    bool tiled = false,
                                    uint8_t* row_codes = nullptr,
                                    uint8_t* row_scales = nullptr);
// row-wise MXFP8 of float32 values [n / cols][cols] (n % 32 == 0) with the
// encoder of the MXFP8 gate/up epilogue; row-major scales [n / 32]
hipError_t launch_mx_quant_f32(const float* src, int64_t n, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream);
// row-major scales [rows][k / 32] (k % 128 == 0, 4-byte aligned) -> GEMM
// layout
hipError_t launch_mx_scales_retile(const uint8_t* src, int64_t rows,
                                   int64_t k, uint8_t* dst,
                                   hipStream_t stream);

// achievable-bandwidth reference: read `bytes` once, write k copies
hipError_t launch_hbm_mix(const void* src, int64_t bytes, int reads,
                          int writes, void* dst, int cu_count,
                          hipStream_t stream);
hipError_t launch_hbm_stream(const void* src, int64_t bytes, int k, void* dst,
                             int cu_count, hipStream_t stream);

// bf16 grouped MLP
size_t mlp_fwd_bf16_ws_bytes(int E, int H, int F, int64_t rows, bool need_a);
hipError_t launch_mlp_fwd_bf16(int E, int H, int F, int64_t rows,
                               const void* x_perm, const void* w_gu,
                               const void* w_dn, const float* w_perm,
                               const int32_t* offsets, void* z_perm,
                               void* h1_save, void* a_save, void* ws,
                               int cu_count, int32_t* status,
                               hipStream_t stream);
// tensor-scaled FP8
hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t stream);
hipError_t launch_seg_amax(const void* src, int64_t seg_elems, int n_seg,
                           uint32_t* amax_bits, hipStream_t stream);
hipError_t launch_tensor_quant(const void* src, int64_t seg_elems, int n_seg,
                               const uint32_t* amax_bits, uint8_t* codes,
                               float* scales, hipStream_t stream);
// quant_w: the weights are quantised inside the call (else w_gu_q/_ts and
// w_dn_q/_ts, quantised by the caller, are used)
size_t mlp_fwd_fp8t_ws_bytes(int E, int H, int F, int64_t rows, bool need_a,
                             bool quant_w);
hipError_t launch_mlp_fwd_fp8t(int E, int H, int F, int64_t rows,
                               const void* x_perm, const void* w_gu,
                               const void* w_dn, const uint8_t* w_gu_q,
                               const float* w_gu_ts, const uint8_t* w_dn_q,
                               const float* w_dn_ts, const float* w_perm,
                               const int32_t* offsets, void* z_perm,
                               void* h1_save, void* a_save, void* ws,
                               int cu_count, int32_t* status,
                               hipStream_t stream);

// router projection (float64 accumulation in ascending h) and backward
hipError_t launch_router_logits(const void* x, const void* w_r,
                                const float* bias, int64_t T, int H, int E,
                                float* logits, hipStream_t stream);
size_t router_bwd_ws_bytes(int64_t T, int H, int E);
hipError_t launch_router_bwd(const float* logits, const int32_t* topk_idx,
                             const float* dtopk_w, const void* x,
                             const void* w_r, int64_t T, int H, int E, int k,
                             bool renorm, float* dlogits, float* dw_r,
                             float* dx, void* ws, hipStream_t stream);

// per-expert loop (baseline of the grouped path), bf16; offsets_host is
// the host copy of offsets
size_t expert_loop_fwd_ws_bytes(int E, int F, int64_t rows, bool need_h1,
                                bool need_a);
hipError_t launch_expert_loop_fwd(int E, int H, int F, int64_t rows,
                                  const void* x_perm, const void* w_gu,
                                  const void* w_dn, const float* w_perm,
                                  const int32_t* offsets,
                                  const int32_t* offsets_host, void* z_perm,
                                  void* h1_save, void* a_save, void* ws,
                                  hipStream_t stream);
size_t mlp_bwd_bf16_ws_bytes(int E, int H, int F, int64_t rows);
hipError_t launch_mlp_bwd_bf16(int E, int H, int F, int64_t rows,
                               const void* x_perm, const void* w_gu,
                               const void* w_dn, const float* w_perm,
                               const int32_t* offsets, const void* h1_save,
                               const void* a_save, const void* dz_perm,
                               void* dx_perm, void* dw_gu, void* dw_dn,
                               float* dw_perm, void* ws, int32_t* status,
                               hipStream_t stream);

// MXFP8 grouped MLP
size_t mlp_fwd_mx_ws_bytes(int E, int H, int F, int64_t rows, bool quant_x,
                           bool quant_w);
hipError_t launch_mlp_fwd_mx(int E, int H, int F, int64_t rows,
                             const void* x_perm_bf16, const uint8_t* xq,
                             const uint8_t* xs, const void* w_gu,
                             const void* w_dn, const uint8_t* w_gu_q,
                             const uint8_t* w_gu_s, const uint8_t* w_dn_q,
                             const uint8_t* w_dn_s, const float* w_perm,
                             const int32_t* offsets, void* z_perm,
                             void* h1_save, void* a_save, uint8_t* a_q_save,
                             uint8_t* a_s_save, void* ws, int cu_count,
                             int32_t* status, hipStream_t stream);
size_t mlp_bwd_mx_ws_bytes(int E, int H, int F, int64_t rows, bool quant_w);
hipError_t launch_mlp_bwd_mx(int E, int H, int F, int64_t rows,
                             const void* x_perm, const void* w_gu,
                             const void* w_dn, const float* w_perm,
                             const int32_t* offsets, const void* h1_save,
                             const void* a_save, const void* dz_perm,
                             void* dx_perm, void* dw_gu, void* dw_dn,
                             float* dw_perm, const uint8_t* w_gu_qt,
                             const uint8_t* w_gu_st, const uint8_t* w_dn_qt,
                             const uint8_t* w_dn_st, void* ws,
                             int32_t* status, hipStream_t stream);

}  // namespace moe
