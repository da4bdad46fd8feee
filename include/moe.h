/*
 * moe.h -- C ABI of libmoe: the MoE expert-MLP hot path on one MI355X
 * (gfx950).
 *
 * The path: router top-k -> permute tokens into expert-contiguous order with
 * per-expert split_sizes -> grouped GEMM gate/up -> ScaledSwiGLU times the
 * routing weight -> grouped GEMM down -> unpermute / combine, in bf16 or
 * MXFP8 (E4M3 elements, one E8M0 scale per 32 consecutive values along K),
 * forward and backward.
 *
 * Sources (web pages; cited by title and section):
 *  [PG1] "NVIDIA presents an efficient path for training biological MoE
 *        models" (sitech.ge).
 *  [PG2] "Efficient MoE training for biological foundation models (NVIDIA)"
 *        (news.bpdata.com).
 *  [PG3] "Nous Research scales expert parallelism with DeepEP"
 *        (seventnews.com).
 *  [PG4] "NVIDIA NeMo AutoModel: 3.7x faster MoE fine-tuning with expert
 *        parallelism and DeepEP" (seventnews.com).
 *
 * Conventions for every call
 *  - Memory: every tensor argument is DEVICE memory allocated and owned by
 *    the caller (the library never allocates or frees per call); tensors are
 *    dense row-major with the shapes given, 16-byte aligned.  bf16 tensors
 *    are passed as void* (IEEE bfloat16 bit patterns); E4M3 codes and E8M0
 *    scales as uint8_t*.  Scalars are host values.
 *  - Streams: `stream` is a hipStream_t (NULL = the null stream).  Calls
 *    enqueue work and return; none synchronises the host, except
 *    moe_ctx_check_device_status.  The library creates no streams and never
 *    copies split_sizes/offsets to the host.
 *  - Errors: argument validation happens on the host before anything is
 *    enqueued; a failing call enqueues nothing and returns a non-zero
 *    moe_status_t.  moe_last_error() gives a thread-local message.
 *    Data errors that only the device can see are recorded in the context's
 *    device status word (first error wins) and moe_ctx_check_device_status
 *    reports them: an expert id outside [0, E) (the offending pair is
 *    skipped, its row_map entry is -1), and a per-expert offsets array that
 *    does not run non-decreasing from 0 to the row count (the call then
 *    processes no expert; its outputs are undefined).
 *  - Threading: a context may be used by one host thread at a time.
 *  - Determinism: no floating-point atomics; results are bitwise
 *    reproducible for the same inputs and sizes.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null required pointer, bad sizes, k > E */
  MOE_ERR_UNSUPPORTED = 2,   /* device not gfx950, size outside limits */
  MOE_ERR_WORKSPACE = 3,     /* workspace missing or too small */
  MOE_ERR_HIP = 4,           /* a HIP runtime call or launch failed */
  MOE_ERR_DEVICE_CHECK = 5   /* a device-side data check fired */
} moe_status_t;

typedef enum moe_precision {
  MOE_PREC_BF16 = 0,
  MOE_PREC_MXFP8_E4M3 = 1,
  /* E4M3 with one float32 scale per tensor (forward only) */
  MOE_PREC_FP8_TENSOR = 2
} moe_precision_t;

typedef enum moe_mx_axis {
  MOE_MX_ROWWISE = 0,   /* blocks of 32 run along each row (cols) */
  MOE_MX_COLWISE = 1    /* blocks of 32 run down each column; output transposed */
} moe_mx_axis_t;

/* Device status codes written by kernels into the context status word. */
#define MOE_DEVERR_NONE 0
#define MOE_DEVERR_EXPERT_ID 1     /* topk_idx entry outside [0, E) */
#define MOE_DEVERR_OFFSETS 2       /* offsets not non-decreasing from 0 to rows */
#define MOE_DEVERR_LOGITS 3        /* a router logit is NaN or infinite */

typedef struct moe_ctx* moe_ctx_t;

/* Limits (UNSUPPORTED beyond them). */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32

/* ------------------------------------------------------------------------
 * Context.  moe_ctx_create checks that `device` is a gfx950 GPU, records its
 * compute-unit count and allocates the 4-byte device status word (the only
 * allocation the library makes, freed by moe_ctx_destroy).
 * ---------------------------------------------------------------------- */
moe_status_t moe_ctx_create(int device, moe_ctx_t* ctx);
moe_status_t moe_ctx_destroy(moe_ctx_t ctx);

/* Synchronises `stream`, returns the first device-side error code recorded
 * since the last check in *host_code (MOE_DEVERR_*), and clears it.  Returns
 * MOE_ERR_DEVICE_CHECK when a code was set, MOE_OK otherwise. */
moe_status_t moe_ctx_check_device_status(moe_ctx_t ctx, void* stream,
                                         int32_t* host_code);

const char* moe_status_string(moe_status_t status);
const char* moe_last_error(void);

/* ------------------------------------------------------------------------
 * Per-kernel timing (a measurement aid; off by default).
 * moe_ctx_set_kernel_timing(ctx, 1): every kernel the library launches for
 * this context is bracketed by two HIP events recorded on the launch stream
 * (the stream passed to the call); 0 switches it off.  Records accumulate
 * until moe_ctx_reset_kernel_timing.
 * moe_ctx_kernel_time: waits for the recorded events and returns, for the
 * kernel called `kernel` (e.g. "gemm_gate_up_swiglu_bf16",
 * "gemm_down_bf16", "permute_gather", "unpermute"; the names are listed in
 * the library's sources next to each launch), the number of launches and
 * their summed duration in milliseconds (0 / 0.0 if none).
 * ---------------------------------------------------------------------- */
moe_status_t moe_ctx_set_kernel_timing(moe_ctx_t ctx, int32_t enable);
moe_status_t moe_ctx_reset_kernel_timing(moe_ctx_t ctx);
moe_status_t moe_ctx_kernel_time(moe_ctx_t ctx, const char* kernel,
                                 int64_t* launches, double* total_ms);

/* moe_hbm_stream_reference -- a measurement aid, not a step of the path:
 * reads `bytes` of src once and writes k copies of them to dst
 * ([k][bytes], device memory, 16-byte aligned, bytes % 16 == 0), the
 * traffic shape of moe_permute's row gather without its indexing, as the
 * achievable HBM bandwidth the gather and combine are compared with
 * (kernel name "hbm_stream_reference" for moe_ctx_kernel_time). */
moe_status_t moe_hbm_stream_reference(moe_ctx_t ctx, const void* src,
                                      int64_t bytes, int32_t k, void* dst,
                                      void* stream);

/* moe_hbm_stream_mix -- a measurement aid, not a step of the path: reads
 * `reads` (0..2) buffers of `bytes` each from src ([reads][bytes]) and
 * writes `writes` (0..2) copies of their bitwise xor (of a constant when
 * reads = 0) to dst ([writes][bytes]; with writes = 0 nothing is stored,
 * dst must still hold 4 KiB), reads + writes >= 1, device memory, 16-byte
 * aligned, bytes % 16 == 0: the HBM bandwidth of each traffic mix (read
 * only, write only, copy, one read and two writes as the permute's gather,
 * two reads and one write as the combine) on this device.  Kernel name
 * "hbm_stream_mix" for moe_ctx_kernel_time. */
moe_status_t moe_hbm_stream_mix(moe_ctx_t ctx, const void* src, int64_t bytes,
                                int32_t reads, int32_t writes, void* dst,
                                void* stream);

/* ------------------------------------------------------------------------
 * moe_router_logits -- router projection in front of the top-k.
 * [PG3, practical-implications paragraph: Top-k routing; PG4, section
 *  "Background": tokens are routed across many experts.]  The pages do not
 * give the router's form; the library takes the linear gate reading.
 * logits[t, e] = sum over h in ascending order of x[t, h] * W_r[e, h],
 * accumulated in float64 one term at a time (the bf16 products are exact),
 * plus bias[e], rounded once to float32.  The result does not depend on the
 * launch shape, so the routing decided on it is reproducible bit for bit.
 *
 *  x       bf16    [T, H]
 *  w_r     bf16    [E, H]   the gate
 *  bias    float32 [E] or NULL
 *  logits  float32 [T, E]   out
 *  T >= 0 (T = 0 is a no-op), H >= 8 with H % 8 == 0, 1 <= E <= 1024;
 *  x and w_r 16-byte aligned.
 * Errors: MOE_ERR_INVALID_ARG (null pointer, bad sizes), MOE_ERR_UNSUPPORTED
 * (E > 1024, H % 8 != 0, misaligned x / w_r, T * max(H, E) >= 2^62),
 * MOE_ERR_HIP.
 * ---------------------------------------------------------------------- */
moe_status_t moe_router_logits(moe_ctx_t ctx, const void* x, const void* w_r,
                               const float* bias, int64_t T, int32_t H,
                               int32_t E, float* logits, void* stream);

/* ------------------------------------------------------------------------
 * moe_router_bwd -- router backward.
 * [Same passages as moe_router_logits.]  The routing-weight gradient
 * reaches the logits only through the softmax the forward used (the top-k
 * selection passes no gradient).  With the forward weights recomputed from
 * the logits in float64:
 *   renormalize != 0:  dl_i = w_i (dw_i - sum_j w_j dw_j) on the chosen set,
 *                      0 elsewhere
 *   renormalize == 0:  dl_e = p_e (g_e - sum_j p_j dw_j), p the softmax over
 *                      all E, g_e = dw on the chosen set and 0 elsewhere
 * then dW_r = dlogits^T x and the router's share of dx = dlogits W_r, in
 * float32 with a fixed summation order (deterministic).
 *
 *  logits   float32 [T, E];  topk_idx int32 [T, k] (entries in [0, E): ids
 *           outside are clamped when read and give unspecified values)
 *  dtopk_w  float32 [T, k]   gradient of the routing weights
 *  x        bf16 [T, H];  w_r bf16 [E, H]
 *  dlogits  float32 [T, E]   out (required)
 *  dw_r     float32 [E, H]   out, or NULL to skip
 *  dx       float32 [T, H]   out, or NULL to skip
 *  ws       moe_router_bwd_workspace_size bytes (NULL when that is 0)
 *  T >= 0, H >= 1, 1 <= k <= min(E, 32), E <= 1024.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE,
 * MOE_ERR_HIP.
 * ---------------------------------------------------------------------- */
moe_status_t moe_router_bwd_workspace_size(int64_t T, int32_t H, int32_t E,
                                           size_t* bytes);
moe_status_t moe_router_bwd(moe_ctx_t ctx, const float* logits,
                            const int32_t* topk_idx, const float* dtopk_w,
                            const void* x, const void* w_r, int64_t T,
                            int32_t H, int32_t E, int32_t k,
                            int32_t renormalize, float* dlogits, float* dw_r,
                            float* dx, void* ws, size_t ws_bytes,
                            void* stream);

/* ------------------------------------------------------------------------
 * moe_route_topk -- router top-k.
 * [PG3, practical-implications paragraph: Top-k routing; PG2, section "Why
 *  dense and MoE models differ": only a small subset of experts is active
 *  per token.]  The pages name Top-k but not the weight formula; the
 * library takes the softmax reading.
 *
 *  logits   float32 [T, E]  router logits.
 *  topk_idx int32   [T, k]  out: the k experts with the largest logits,
 *                           slot 0 the largest; equal logits go to the lower
 *                           expert id (+0 and -0 are equal).
 *  topk_w   float32 [T, k]  out: exp(l - max) normalised over the chosen k
 *                           (renormalize != 0) or over all E (== 0),
 *                           evaluated in float64, rounded to float32.
 *  1 <= k <= min(E, 32), E <= 1024, T >= 0 (T = 0 is a no-op).
 *  Logits must be finite: a NaN or infinite logit records
 *  MOE_DEVERR_LOGITS (moe_ctx_check_device_status) and leaves that token's
 *  selection unspecified; every other token is routed as above.
 * ---------------------------------------------------------------------- */
moe_status_t moe_route_topk(moe_ctx_t ctx, const float* logits, int64_t T,
                            int32_t E, int32_t k, int32_t renormalize,
                            int32_t* topk_idx, float* topk_w, void* stream);

/* ------------------------------------------------------------------------
 * moe_permute -- expert-order permutation and row gather.
 * [PG1, section "Grouped experts instead of a Python loop", and PG2, section
 *  "1) Fragmented expert kernels": the grouped GEMM gathers the tokens of
 *  every expert and takes the per-expert token counts (split_sizes); PG4,
 *  section "Using Transformers v5 features": grouped_mm runs on sorted
 *  tokens.]
 *
 * Pair p = t*k + j (token t, slot j) goes to expert e = topk_idx[t, j].
 *  split_sizes int32 [E]    out: pairs per expert.
 *  offsets     int32 [E+1]  out: exclusive prefix sum, offsets[E] = T*k.
 *  row_map     int32 [T*k]  out: destination row of pair p; rows are ordered
 *                           by expert, then by p (stable; unique).
 *  src_row     int32 [T*k]  out: inverse of row_map (src_row[row_map[p]] = p).
 *  x           bf16  [T, H] tokens.
 *  x_perm      [T*k, H]     out: x_perm[row_map[t*k+j]] = x[t]; bf16 when
 *                           out_prec = MOE_PREC_BF16, E4M3 codes (uint8) when
 *                           out_prec = MOE_PREC_MXFP8_E4M3.
 *  x_perm_scale uint8 [T*k, H/32] out (MXFP8 only, else NULL): E8M0 scales of
 *                           the row-wise blocks of 32 along H.
 *  topk_w      float32 [T, k] (nullable) routing weights;
 *  w_perm      float32 [T*k]  (nullable) out: w_perm[row_map[p]] = topk_w[p].
 *  ws          workspace of at least moe_permute_workspace_size() bytes.
 *  H % 8 == 0 (bf16) or H % 32 == 0 (MXFP8).
 * ---------------------------------------------------------------------- */
moe_status_t moe_permute_workspace_size(int64_t T, int32_t E, int32_t k,
                                        size_t* bytes);
moe_status_t moe_permute(moe_ctx_t ctx, const void* x,
                         const int32_t* topk_idx, const float* topk_w,
                         int64_t T, int32_t H, int32_t E, int32_t k,
                         moe_precision_t out_prec, void* x_perm,
                         uint8_t* x_perm_scale, float* w_perm,
                         int32_t* row_map, int32_t* src_row,
                         int32_t* split_sizes, int32_t* offsets, void* ws,
                         size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_permute_noalloc -- moe_permute without a workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 * Arguments, results and errors as moe_permute, minus ws / ws_bytes.  The
 * index build's per-block expert histograms (moe_permute_workspace_size
 * bytes) live instead in a static device array of 4 MiB that every GPU the
 * library runs on holds until the process ends; its address is looked up
 * once per device when the context is created.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).
 * Limit: moe_permute_workspace_size(T, E, k) <= 4 MiB, i.e.
 * ceil(T*k / 1024) * E <= 1048576 (e.g. E = 128 up to T*k = 8M pairs,
 * E = 1024 up to 1M); larger sizes return MOE_ERR_UNSUPPORTED and enqueue
 * nothing.  The kernels write every histogram entry before reading it, so
 * the array needs no clearing between calls; it keeps the last call's
 * contents.  All calls on one GPU share the one array: calls that overlap
 * in time on a GPU (different streams, or host threads) race and give
 * undefined results; calls ordered on one stream are safe.
 * ---------------------------------------------------------------------- */
moe_status_t moe_permute_noalloc(moe_ctx_t ctx, const void* x,
                                 const int32_t* topk_idx,
                                 const float* topk_w, int64_t T, int32_t H,
                                 int32_t E, int32_t k,
                                 moe_precision_t out_prec, void* x_perm,
                                 uint8_t* x_perm_scale, float* w_perm,
                                 int32_t* row_map, int32_t* src_row,
                                 int32_t* split_sizes, int32_t* offsets,
                                 void* stream);

/* moe_gather_rows -- the row copy of moe_permute alone, for a tensor that
 * shares an existing permutation (the upstream gradient dY -> dZ in the
 * backward pass): dst[row_map[t*k+j]] = src[t] for all t, j; pairs with
 * row_map < 0 are skipped.  src bf16 [T, H], dst bf16 [T*k, H]. */
moe_status_t moe_gather_rows(moe_ctx_t ctx, const void* src,
                             const int32_t* row_map, int64_t T, int32_t H,
                             int32_t k, void* dst, void* stream);

/* ------------------------------------------------------------------------
 * moe_unpermute -- combine back to token order.
 * [PG4, section "Sources of speedup": the combine that follows the expert
 *  compute.]
 *  y[t] = sum_{j = 0..k-1, ascending} c_j * z_perm[row_map[t*k+j]],
 *  c_j = 1 when topk_w is NULL (the weights were applied inside the grouped
 *  MLP), else topk_w[t, j].  Accumulated in float32, rounded to bf16.
 *  z_perm bf16 [T*k, H], y bf16 [T, H], H % 8 == 0.  Pairs with
 *  row_map < 0 contribute nothing.
 * ---------------------------------------------------------------------- */
moe_status_t moe_unpermute(moe_ctx_t ctx, const void* z_perm,
                           const int32_t* row_map, const float* topk_w,
                           int64_t T, int32_t H, int32_t k, void* y,
                           void* stream);

/* moe_unpermute_probs_grad -- routing-weight gradient back to token order:
 * dprobs[t, j] = dw_perm[row_map[t*k+j]] (0 where row_map < 0).
 * dw_perm float32 [T*k], dprobs float32 [T, k]. */
moe_status_t moe_unpermute_probs_grad(moe_ctx_t ctx, const float* dw_perm,
                                      const int32_t* row_map, int64_t T,
                                      int32_t k, float* dprobs, void* stream);

/* ------------------------------------------------------------------------
 * mxfp8_quantize -- MXFP8 quantisation of a bf16 tensor.
 * [PG1, section "Reducing memory and quantisation cost", and PG2, section
 *  "2) Model size and activation memory": 8-bit elements with one scale per
 *  block of 32 consecutive values; PG2, section "3) Quantisation overhead in
 *  low-precision training": 16-bit master weights are quantised.]
 * Per block v[0..31]: s = floor(log2 max|v|) - 8 clamped to [-127, 127]
 * (all-zero block: -127); scale byte = s + 127 (E8M0); code_i = OCP E4M3 of
 * v_i * 2^-s, round to nearest even, saturating at +-448, sign kept.
 *
 *  src bf16 [batch, rows, cols].
 *  ROWWISE: blocks along cols (cols % 32 == 0); codes [batch, rows, cols],
 *           scales [batch, rows, cols/32].
 *  COLWISE, seg_offsets == NULL: blocks along rows (rows % 32 == 0); output
 *           transposed: codes [batch, cols, rows], scales
 *           [batch, cols, rows/32].
 *  COLWISE, seg_offsets != NULL (batch must be 1): rows are split into
 *           n_seg segments [seg_offsets[s], seg_offsets[s+1]) (device int32,
 *           seg_offsets[n_seg] == rows); blocks restart at each segment
 *           start and the last block of a segment is zero-padded.  Segment s
 *           occupies output columns [P_s, P_s + ceil(n_s/32)*32) with
 *           P_s = sum_{s'<s} ceil(n_s'/32)*32.  codes [cols, ld],
 *           scales [cols, ld/32], ld = rows + 32*n_seg rounded up to 32
 *           (columns past the last segment are left untouched).
 *           seg_offsets not running non-decreasing from 0 to rows: nothing
 *           is written and MOE_DEVERR_OFFSETS is recorded.
 * ---------------------------------------------------------------------- */
moe_status_t mxfp8_quantize(moe_ctx_t ctx, const void* src, int64_t batch,
                            int64_t rows, int64_t cols, moe_mx_axis_t axis,
                            const int32_t* seg_offsets, int32_t n_seg,
                            uint8_t* codes, uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------
 * mxfp8_quantize_f32 -- row-wise MXFP8 quantisation of float32 values.
 * [PG1, section "Reducing memory and quantisation cost": the SwiGLU output
 *  is quantised inside the fused grouped MLP; PG2, section "2) Model size
 *  and activation memory": one scale per block of 32 consecutive values.]
 * The same rule as mxfp8_quantize ROWWISE, applied to float32 input with the
 * encoder that moe_grouped_mlp_fwd's MXFP8 gate/up epilogue runs on its
 * float32 ScaledSwiGLU output (so the epilogue's rounding can be checked
 * value by value): per block of 32, s = floor(log2 max|v|) - 8 clamped to
 * [-127, 127], scale byte s + 127, code = E4M3 of v * 2^-s (round to
 * nearest even, saturating at +-448, sign kept).  Values must be finite.
 *  src float32 [rows, cols] (cols % 32 == 0, 16-byte aligned)
 *  codes uint8 [rows, cols] (8-byte aligned), scales uint8 [rows, cols/32]
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED (cols % 32, alignment),
 * MOE_ERR_HIP.
 * ---------------------------------------------------------------------- */
moe_status_t mxfp8_quantize_f32(moe_ctx_t ctx, const float* src, int64_t rows,
                                int64_t cols, uint8_t* codes, uint8_t* scales,
                                void* stream);

/* ------------------------------------------------------------------------
 * moe_fp8_tensor_quantize -- tensor-scaled FP8 quantisation.
 * [PG1, section "Reducing memory and quantisation cost"; PG2, section "3)
 *  Quantisation overhead in low-precision training".]
 * src bf16 holds n_seg tensors of seg_elems values each (seg_elems % 8 ==
 * 0, 16-byte aligned).  Per tensor: amax = max |v|, s = amax / 448 in
 * float32 (1 when amax is 0), code = OCP E4M3 of float32(v / s), round to
 * nearest even, saturating at +-448.
 *  codes  uint8 [n_seg, seg_elems] out;  scales float32 [n_seg] out
 *  ws     moe_fp8_tensor_quantize_workspace_size bytes (the amax pass)
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED (seg_elems % 8,
 * alignment, n_seg >= 2^16), MOE_ERR_WORKSPACE, MOE_ERR_HIP.
 * ---------------------------------------------------------------------- */
moe_status_t moe_fp8_tensor_quantize_workspace_size(int64_t n_seg,
                                                    size_t* bytes);
moe_status_t moe_fp8_tensor_quantize(moe_ctx_t ctx, const void* src,
                                     int64_t n_seg, int64_t seg_elems,
                                     uint8_t* codes, float* scales, void* ws,
                                     size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_mlp_fwd -- grouped GEMM gate/up -> ScaledSwiGLU x routing
 * weight -> grouped GEMM down, over all experts in one call.
 * [PG1, sections "Grouped experts instead of a Python loop" (one grouped
 *  GEMM for all experts, split_sizes, routing weights scaled inside the
 *  grouped-MLP kernel) and "Reducing memory and quantisation cost"
 *  (GroupedLinear -> ScaledSwiGLU -> GroupedLinear fused into one op);
 *  PG2, section "3) Quantisation overhead in low-precision training".]
 * For each expert e with rows [offsets[e], offsets[e+1]) of x_perm:
 *   h1 = X_e W_gu[e]^T  (float32 accumulate), g = h1[:, :F], u = h1[:, F:]
 *   a  = w_perm * silu(g) * u        (silu(z) = z / (1 + exp(-z)))
 *   z  = a W_dn[e]^T                 -> z_perm bf16
 * Experts with no rows cost nothing.
 * MXFP8: X and W_gu are quantised along H, a and W_dn along F (E4M3 + E8M0
 * per 32, as in mxfp8_quantize ROWWISE); the GEMMs use the gfx950 scaled
 * MFMA with float32 accumulation; a is quantised from float32 in the gate/up
 * epilogue; h1_save / a_save hold the unquantised float32 values rounded to
 * bf16, and a_q_save / a_s_save (optional) A's E4M3 codes and row-major E8M0
 * scales as the down GEMM consumes them.
 * FP8 tensor-scaled (MOE_PREC_FP8_TENSOR, forward only) [PG1, section
 * "Reducing memory and quantisation cost"; PG2, section "3) Quantisation
 * overhead in low-precision training": 8-bit elements with scales from
 * 16-bit masters]: x_perm (bf16), each W_gu[e] and each W_dn[e] get one
 * float32 scale s = amax / 448 (1 if all zero) and E4M3 codes of
 * float32(v / s), as in moe_fp8_tensor_quantize; the GEMMs multiply the
 * E4M3 products by the two scales; a (bf16, over all rows) is quantised the
 * same way for the down GEMM; h1_save / a_save hold the bf16 values.
 * x_perm_scale, w_gu_s and w_dn_s must be NULL; the weights may come
 * pre-quantised (w_gu_q + w_gu_ts, w_dn_q + w_dn_ts, below).
 * Sizes: 1 <= E <= 1024; H and F multiples of 64 (bf16) or 128 (8-bit);
 * one expert's operands must stay below 4 GiB (byte offsets are 32-bit).
 * Errors: MOE_ERR_INVALID_ARG (null required pointer, bad sizes),
 * MOE_ERR_UNSUPPORTED (size limits, misaligned pointers: operands 16-byte,
 * MXFP8 scale arrays 4-byte), MOE_ERR_WORKSPACE (ws NULL or smaller than
 * moe_grouped_mlp_fwd_workspace_size), MOE_ERR_HIP.  The workspace is
 * scratch owned by the caller; its contents after the call are undefined
 * (besides tile tables and quantised operands it holds the float32 partial
 * tiles of a down GEMM whose last round of tiles is split along K, up to
 * 64 MiB).  Results are deterministic: the same inputs give the same bits.
 * offsets must run non-decreasing from 0 to rows; the device checks this
 * (it reads the per-expert counts) and otherwise records MOE_DEVERR_OFFSETS
 * and runs no GEMM tile (outputs undefined).
 * ---------------------------------------------------------------------- */
typedef struct moe_mlp_fwd_args {
  int32_t E, H, F;               /* experts, hidden, expert FFN size */
  int64_t rows;                  /* T*k = offsets[E] */
  moe_precision_t precision;
  /* x_perm: bf16 [rows, H]; in MXFP8 mode either E4M3 codes [rows, H] with
   * x_perm_scale [rows, H/32], or bf16 with x_perm_scale NULL (then
   * quantised row-wise inside the call). */
  const void* x_perm;
  const uint8_t* x_perm_scale;
  const void* w_gu;              /* bf16 [E, 2F, H]: gate rows 0..F-1, up F..2F-1 */
  const void* w_dn;              /* bf16 [E, H, F] */
  /* MXFP8 only, optional: weights already quantised row-wise along K
   * (w_gu_q [E, 2F, H] + w_gu_s [E, 2F, H/32]; w_dn_q [E, H, F] +
   * w_dn_s [E, H, F/32]).  NULL: quantised from w_gu / w_dn inside the
   * call (in the workspace). */
  const uint8_t* w_gu_q; const uint8_t* w_gu_s;
  const uint8_t* w_dn_q; const uint8_t* w_dn_s;
  const float* w_perm;           /* float32 [rows] or NULL (weight 1) */
  const int32_t* offsets;        /* int32 [E+1] on the device */
  void* z_perm;                  /* out: bf16 [rows, H] */
  void* h1_save;                 /* out, nullable: bf16 [rows, 2F] (g, u) */
  void* a_save;                  /* out, nullable: bf16 [rows, F] */
  void* ws;                      /* workspace */
  size_t ws_bytes;
  /* MXFP8 only, out, nullable: A's E4M3 codes [rows, F] (16-byte aligned)
   * and E8M0 scales [rows, F/32] (row-major), as the down GEMM reads them */
  uint8_t* a_q_save;
  uint8_t* a_s_save;
  /* FP8 tensor-scaled only, optional (with w_gu_q / w_dn_q, each pair both
   * set or both NULL): the weights already quantised, as
   * moe_fp8_tensor_quantize(w, n_seg = E) returns them: w_gu_q [E, 2F, H]
   * E4M3 codes + w_gu_ts float32 [E] scales, w_dn_q [E, H, F] + w_dn_ts
   * [E].  NULL: quantised from w_gu / w_dn inside the call.  Reuse
   * contract as for the MXFP8 codes: they must be the quantisation of this
   * call's w_gu / w_dn (not checked); a caller quantises them once per
   * weight update. */
  const float* w_gu_ts;
  const float* w_dn_ts;
} moe_mlp_fwd_args;

moe_status_t moe_grouped_mlp_fwd_workspace_size(const moe_mlp_fwd_args* args,
                                                size_t* bytes);
moe_status_t moe_grouped_mlp_fwd(moe_ctx_t ctx, const moe_mlp_fwd_args* args,
                                 void* stream);

/* ------------------------------------------------------------------------
 * moe_expert_loop_mlp_fwd -- the computation of moe_grouped_mlp_fwd (bf16)
 * done the way a per-expert Python loop does it: the baseline the grouped
 * path is measured against.
 * [PG1, section "Grouped experts instead of a Python loop": a loop over
 *  experts launches separate small kernels per expert; the grouped GEMM
 *  replaces it.]
 * The call copies offsets to the host and waits for the stream, then for
 * every expert with rows, in ascending order, launches: a gate/up GEMM
 * writing h1 = X_e W_gu[e]^T (bf16), a SwiGLU kernel writing
 * a = w_perm * silu(g) * u (float32 arithmetic on the bf16 h1, bf16 out),
 * and a down GEMM writing z = a W_dn[e]^T.  Results equal the grouped
 * path's up to the bf16 rounding of h1 before the SwiGLU.
 * args: as moe_grouped_mlp_fwd with precision MOE_PREC_BF16 (MXFP8 fields
 * ignored); h1_save / a_save nullable (then held in the workspace).
 * Errors: MOE_ERR_INVALID_ARG (null required pointer, bad sizes, offsets
 * read back not non-decreasing from 0 to rows), MOE_ERR_UNSUPPORTED (MXFP8,
 * size limits, misaligned pointers), MOE_ERR_WORKSPACE, MOE_ERR_HIP.
 * ---------------------------------------------------------------------- */
moe_status_t moe_expert_loop_mlp_fwd_workspace_size(
    const moe_mlp_fwd_args* args, size_t* bytes);
moe_status_t moe_expert_loop_mlp_fwd(moe_ctx_t ctx,
                                     const moe_mlp_fwd_args* args,
                                     void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_mlp_bwd -- the backward counterpart of moe_grouped_mlp_fwd.
 * [PG1, section "Reducing memory and quantisation cost": the fused forward
 *  op has a counterpart in the backward pass.]
 * Per expert, with s = sigmoid(g), silu(g) = g*s, a = w*silu(g)*u:
 *   dA   = dZ W_dn[e]
 *   dg   = dA * w * u * s * (1 + g*(1 - s)),   du = dA * w * silu(g)
 *   dw_perm = sum_f dA * silu(g) * u
 *   dW_dn[e] = dZ^T a,  dW_gu[e] = [dg du]^T X,  dX = [dg du] W_gu[e]
 * Experts with no rows get dW = 0.  MXFP8 mode quantises every GEMM operand
 * along that GEMM's K: dZ and dH1 = [dg du] row-wise, W_dn and W_gu along
 * their output dimension, and dZ, a, dH1, X along tokens for the weight
 * gradients (token-direction blocks restart at each expert's first row and
 * are zero-padded); dH1 is quantised from its bf16 rounding.  h1_save and
 * a_save are the forward's saves (bf16) in both modes.
 * Sizes and errors as moe_grouped_mlp_fwd; MXFP8 also needs
 * (max(H, 2F) + 256) * (rows + 128 E + 128) < 2^32 (the token-direction
 * operand copies use 32-bit byte offsets).  The workspace holds dH1 and, in
 * MXFP8 mode, every quantised operand copy (about 4 GB for T*k = 16384,
 * H = 4096, F = 14336, E = 8); its contents after the call are undefined.
 * ---------------------------------------------------------------------- */
typedef struct moe_mlp_bwd_args {
  int32_t E, H, F;
  int64_t rows;
  moe_precision_t precision;
  const void* x_perm;            /* bf16 [rows, H] */
  const void* w_gu;              /* bf16 [E, 2F, H] */
  const void* w_dn;              /* bf16 [E, H, F] */
  const float* w_perm;           /* float32 [rows] or NULL (weight 1) */
  const int32_t* offsets;        /* int32 [E+1] */
  const void* h1_save;           /* bf16 [rows, 2F] saved by the forward */
  const void* a_save;            /* bf16 [rows, F] saved by the forward */
  const void* dz_perm;           /* bf16 [rows, H] gradient of z_perm */
  void* dx_perm;                 /* out: bf16 [rows, H] */
  void* dw_gu;                   /* out: bf16 [E, 2F, H] */
  void* dw_dn;                   /* out: bf16 [E, H, F] */
  float* dw_perm;                /* out: float32 [rows] (NULL if w_perm NULL) */
  void* ws;
  size_t ws_bytes;
  /* MXFP8 only, optional (each codes/scales pair both set or both NULL):
   * the weights already quantised along the dgrad GEMMs' K, as
   * mxfp8_quantize(w, COLWISE, batch = E) returns them:
   *   w_gu_qt [E, H, 2F] codes + w_gu_st [E, H, 2F/32] scales (W_gu blocked
   *   along 2F); w_dn_qt [E, F, H] + w_dn_st [E, F, H/32] (W_dn along H).
   * NULL: quantised from w_gu / w_dn inside the call (and held in the
   * workspace).  Reuse contract: they must be the quantisation of the w_gu
   * / w_dn of this call (not checked).  Weights change only at an
   * optimizer step, so a caller quantises them once per update and passes
   * the same codes to every micro-batch's backward (and the row-wise ones,
   * w_gu_q / w_dn_q, to every forward). */
  const uint8_t* w_gu_qt; const uint8_t* w_gu_st;
  const uint8_t* w_dn_qt; const uint8_t* w_dn_st;
} moe_mlp_bwd_args;

moe_status_t moe_grouped_mlp_bwd_workspace_size(const moe_mlp_bwd_args* args,
                                                size_t* bytes);
moe_status_t moe_grouped_mlp_bwd(moe_ctx_t ctx, const moe_mlp_bwd_args* args,
                                 void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
