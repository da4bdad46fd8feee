// libmoe C ABI: argument validation, workspace sizing and kernel dispatch.
// Every call validates on the host first and enqueues nothing on failure.
#include <vector>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/moe.h"
#include "kernels.hpp"
#include "timer.hpp"

struct moe_ctx {
  int device;
  int cu_count;
  int32_t* status;  // device word: first data error
  void* perm_scratch;  // this device's static scratch of moe_permute_noalloc
  bool timing;
  moe::KernelTimer timer;
};

namespace {

thread_local std::string g_last_error;

moe_status_t fail(moe_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status_t ok() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

#define MOE_REQUIRE(cond, code, ...) \
  do {                               \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

moe_status_t check_ctx(moe_ctx_t ctx) {
  MOE_REQUIRE(ctx != nullptr, MOE_ERR_INVALID_ARG, "null context");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != ctx->device)
    return fail(MOE_ERR_INVALID_ARG,
                "context belongs to device %d but device %d is current",
                ctx->device, cur);
  return MOE_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Publishes the context's kernel timer to the launch wrappers for the
// duration of one library call.
struct TimerGuard {
  explicit TimerGuard(moe_ctx_t ctx) {
    moe::tl_timer = (ctx && ctx->timing) ? &ctx->timer : nullptr;
  }
  ~TimerGuard() { moe::tl_timer = nullptr; }
};

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    case MOE_ERR_DEVICE_CHECK: return "device-side data check failed";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status_t moe_ctx_create(int device, moe_ctx_t* out) {
  MOE_REQUIRE(out != nullptr, MOE_ERR_INVALID_ARG, "null output pointer");
  *out = nullptr;
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess) return hip_status(e, "hipGetDeviceCount");
  MOE_REQUIRE(device >= 0 && device < n, MOE_ERR_INVALID_ARG,
              "device %d out of range (%d devices)", device, n);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return hip_status(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MOE_ERR_UNSUPPORTED, "device %d is %s, libmoe needs gfx950",
                device, prop.gcnArchName);
  int prev = -1;
  (void)hipGetDevice(&prev);
  e = hipSetDevice(device);
  if (e != hipSuccess) return hip_status(e, "hipSetDevice");
  int32_t* status = nullptr;
  void* scratch = nullptr;
  e = hipMalloc(&status, sizeof(int32_t));
  if (e == hipSuccess) e = hipMemset(status, 0, sizeof(int32_t));
  const hipError_t es =
      e == hipSuccess ? moe::permute_scratch_address(device, &scratch) : e;
  if (prev >= 0) (void)hipSetDevice(prev);
  if (e != hipSuccess || es != hipSuccess) {
    if (status) (void)hipFree(status);
    return e != hipSuccess ? hip_status(e, "status word")
                           : hip_status(es, "static scratch address");
  }
  moe_ctx* c = new moe_ctx;
  c->device = device;
  c->cu_count = prop.multiProcessorCount;
  c->status = status;
  c->perm_scratch = scratch;
  c->timing = false;
  *out = c;
  return ok();
}

moe_status_t moe_ctx_destroy(moe_ctx_t ctx) {
  if (!ctx) return ok();
  (void)hipFree(ctx->status);
  delete ctx;
  return ok();
}

moe_status_t moe_ctx_check_device_status(moe_ctx_t ctx, void* stream,
                                         int32_t* host_code) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  MOE_REQUIRE(host_code != nullptr, MOE_ERR_INVALID_ARG, "null host_code");
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, ctx->status, sizeof(v),
                                hipMemcpyDeviceToHost, as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  if (e == hipSuccess && v != 0)
    e = hipMemsetAsync(ctx->status, 0, sizeof(int32_t), as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_status(e, "device status");
  *host_code = v;
  if (v != 0)
    return fail(MOE_ERR_DEVICE_CHECK, "device check code %d", (int)v);
  return ok();
}

moe_status_t moe_ctx_set_kernel_timing(moe_ctx_t ctx, int32_t enable) {
  MOE_REQUIRE(ctx != nullptr, MOE_ERR_INVALID_ARG, "null context");
  ctx->timing = enable != 0;
  return ok();
}

moe_status_t moe_ctx_reset_kernel_timing(moe_ctx_t ctx) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  ctx->timer.reset();
  return ok();
}

moe_status_t moe_ctx_kernel_time(moe_ctx_t ctx, const char* kernel,
                                 int64_t* launches, double* total_ms) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  MOE_REQUIRE(kernel && launches && total_ms, MOE_ERR_INVALID_ARG,
              "null pointer");
  return hip_status(ctx->timer.query(kernel, launches, total_ms),
                    "kernel timing events");
}

moe_status_t moe_hbm_stream_reference(moe_ctx_t ctx, const void* src,
                                      int64_t bytes, int32_t k, void* dst,
                                      void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(bytes >= 0 && k >= 1 && k <= MOE_MAX_TOPK, MOE_ERR_INVALID_ARG,
              "bad sizes");
  MOE_REQUIRE(bytes % 16 == 0, MOE_ERR_UNSUPPORTED, "bytes %% 16 != 0");
  if (bytes == 0) return ok();
  MOE_REQUIRE(src && dst, MOE_ERR_INVALID_ARG, "null pointer");
  MOE_REQUIRE(aligned16(src) && aligned16(dst), MOE_ERR_UNSUPPORTED,
              "src / dst must be 16-byte aligned");
  return hip_status(moe::launch_hbm_stream(src, bytes, k, dst, ctx->cu_count,
                                           as_stream(stream)),
                    "hbm stream reference");
}

moe_status_t moe_hbm_stream_mix(moe_ctx_t ctx, const void* src, int64_t bytes,
                                int32_t reads, int32_t writes, void* dst,
                                void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(bytes >= 0 && reads >= 0 && reads <= 2 && writes >= 0 &&
                  writes <= 2 && reads + writes >= 1,
              MOE_ERR_INVALID_ARG, "bad sizes");
  MOE_REQUIRE(bytes % 16 == 0, MOE_ERR_UNSUPPORTED, "bytes %% 16 != 0");
  if (bytes == 0) return ok();
  MOE_REQUIRE(dst && (src || reads == 0), MOE_ERR_INVALID_ARG,
              "null pointer");
  MOE_REQUIRE(aligned16(src) && aligned16(dst), MOE_ERR_UNSUPPORTED,
              "src / dst must be 16-byte aligned");
  return hip_status(moe::launch_hbm_mix(src, bytes, reads, writes, dst,
                                        ctx->cu_count, as_stream(stream)),
                    "hbm stream mix");
}

moe_status_t moe_fp8_tensor_quantize_workspace_size(int64_t n_seg,
                                                    size_t* bytes) {
  MOE_REQUIRE(bytes != nullptr && n_seg >= 0, MOE_ERR_INVALID_ARG,
              "bad arguments");
  *bytes = (size_t)n_seg * sizeof(uint32_t);
  return ok();
}

moe_status_t moe_fp8_tensor_quantize(moe_ctx_t ctx, const void* src,
                                     int64_t n_seg, int64_t seg_elems,
                                     uint8_t* codes, float* scales, void* ws,
                                     size_t ws_bytes, void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(n_seg >= 0 && seg_elems >= 0, MOE_ERR_INVALID_ARG, "bad sizes");
  MOE_REQUIRE(n_seg < 65536 && seg_elems % 8 == 0, MOE_ERR_UNSUPPORTED,
              "n_seg < 65536 and seg_elems % 8 == 0 required");
  if (n_seg == 0) return ok();
  MOE_REQUIRE(scales && (seg_elems == 0 || (src && codes)),
              MOE_ERR_INVALID_ARG, "null tensor pointer");
  MOE_REQUIRE(aligned16(src) && (reinterpret_cast<uintptr_t>(codes) & 7u) == 0,
              MOE_ERR_UNSUPPORTED, "src 16-byte and codes 8-byte aligned");
  MOE_REQUIRE(ws && ws_bytes >= (size_t)n_seg * 4, MOE_ERR_WORKSPACE,
              "fp8_tensor_quantize workspace needs %lld bytes",
              (long long)n_seg * 4);
  hipStream_t st = as_stream(stream);
  uint32_t* amax = static_cast<uint32_t*>(ws);
  hipError_t e = moe::launch_zero_u32(amax, (int)n_seg, st);
  if (e == hipSuccess) e = moe::launch_seg_amax(src, seg_elems, (int)n_seg, amax, st);
  if (e == hipSuccess)
    e = moe::launch_tensor_quant(src, seg_elems, (int)n_seg, amax, codes,
                                 scales, st);
  return hip_status(e, "fp8_tensor_quantize");
}

moe_status_t moe_router_logits(moe_ctx_t ctx, const void* x, const void* w_r,
                               const float* bias, int64_t T, int32_t H,
                               int32_t E, float* logits, void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(T >= 0 && H >= 1 && E >= 1, MOE_ERR_INVALID_ARG, "bad sizes");
  MOE_REQUIRE(E <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED, "E <= %d required",
              MOE_MAX_EXPERTS);
  MOE_REQUIRE(T < ((int64_t)1 << 62) / (H > E ? H : E), MOE_ERR_UNSUPPORTED,
              "T too large");
  MOE_REQUIRE((int64_t)T / 32 < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED,
              "T too large");
  MOE_REQUIRE(H % 8 == 0, MOE_ERR_UNSUPPORTED, "H must be a multiple of 8");
  if (T == 0) return ok();
  MOE_REQUIRE(x && w_r && logits, MOE_ERR_INVALID_ARG, "null tensor pointer");
  MOE_REQUIRE(aligned16(x) && aligned16(w_r), MOE_ERR_UNSUPPORTED,
              "x and w_r must be 16-byte aligned");
  return hip_status(moe::launch_router_logits(x, w_r, bias, T, H, E, logits,
                                              as_stream(stream)),
                    "router_logits launch");
}

moe_status_t moe_router_bwd_workspace_size(int64_t T, int32_t H, int32_t E,
                                           size_t* bytes) {
  MOE_REQUIRE(bytes != nullptr, MOE_ERR_INVALID_ARG, "null output pointer");
  MOE_REQUIRE(T >= 0 && H >= 1 && E >= 1, MOE_ERR_INVALID_ARG, "bad sizes");
  *bytes = moe::router_bwd_ws_bytes(T, H, E);
  return ok();
}

moe_status_t moe_router_bwd(moe_ctx_t ctx, const float* logits,
                            const int32_t* topk_idx, const float* dtopk_w,
                            const void* x, const void* w_r, int64_t T,
                            int32_t H, int32_t E, int32_t k,
                            int32_t renormalize, float* dlogits, float* dw_r,
                            float* dx, void* ws, size_t ws_bytes,
                            void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(T >= 0 && H >= 1 && E >= 1 && k >= 1 && k <= E,
              MOE_ERR_INVALID_ARG, "bad sizes");
  MOE_REQUIRE(E <= MOE_MAX_EXPERTS && k <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED,
              "E <= %d and k <= %d required", MOE_MAX_EXPERTS, MOE_MAX_TOPK);
  MOE_REQUIRE(T < ((int64_t)1 << 62) / (H > E ? H : E), MOE_ERR_UNSUPPORTED,
              "T too large");
  MOE_REQUIRE((T + 3) / 4 < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED,
              "T too large");
  const size_t need = moe::router_bwd_ws_bytes(T, H, E);
  if (T == 0) return ok();
  MOE_REQUIRE(logits && topk_idx && dtopk_w && dlogits, MOE_ERR_INVALID_ARG,
              "null tensor pointer");
  MOE_REQUIRE((dw_r == nullptr || x != nullptr) &&
                  (dx == nullptr || w_r != nullptr),
              MOE_ERR_INVALID_ARG, "dw_r needs x, dx needs w_r");
  MOE_REQUIRE(dw_r == nullptr || need == 0 || (ws && ws_bytes >= need),
              MOE_ERR_WORKSPACE, "router_bwd workspace needs %zu bytes", need);
  return hip_status(moe::launch_router_bwd(logits, topk_idx, dtopk_w, x, w_r,
                                           T, H, E, k, renormalize != 0,
                                           dlogits, dw_r, dx, ws,
                                           as_stream(stream)),
                    "router_bwd launch");
}

moe_status_t moe_route_topk(moe_ctx_t ctx, const float* logits, int64_t T,
                            int32_t E, int32_t k, int32_t renormalize,
                            int32_t* topk_idx, float* topk_w, void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "T < 0");
  MOE_REQUIRE(E >= 1 && k >= 1 && k <= E, MOE_ERR_INVALID_ARG,
              "need 1 <= k <= E (k=%d, E=%d)", k, E);
  MOE_REQUIRE(E <= MOE_MAX_EXPERTS && k <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED,
              "E <= %d and k <= %d required", MOE_MAX_EXPERTS, MOE_MAX_TOPK);
  MOE_REQUIRE(T <= (int64_t)INT32_MAX / 64, MOE_ERR_UNSUPPORTED, "T too large");
  if (T == 0) return ok();
  MOE_REQUIRE(logits && topk_idx && topk_w, MOE_ERR_INVALID_ARG,
              "null tensor pointer");
  return hip_status(moe::launch_route_topk(logits, T, E, k, renormalize != 0,
                                           topk_idx, topk_w, ctx->status,
                                           as_stream(stream)),
                    "route_topk launch");
}

moe_status_t moe_permute_workspace_size(int64_t T, int32_t E, int32_t k,
                                        size_t* bytes) {
  MOE_REQUIRE(bytes != nullptr, MOE_ERR_INVALID_ARG, "null output pointer");
  MOE_REQUIRE(T >= 0 && E >= 1 && k >= 1, MOE_ERR_INVALID_ARG, "bad sizes");
  *bytes = moe::permute_ws_bytes(T, E, k);
  return ok();
}

}  // extern "C"

namespace {

// moe_permute after the context check; ws holds ws_bytes of scratch.
moe_status_t permute_impl(moe_ctx_t ctx, const void* x,
                          const int32_t* topk_idx, const float* topk_w,
                          int64_t T, int32_t H, int32_t E, int32_t k,
                          moe_precision_t out_prec, void* x_perm,
                          uint8_t* x_perm_scale, float* w_perm,
                          int32_t* row_map, int32_t* src_row,
                          int32_t* split_sizes, int32_t* offsets, void* ws,
                          size_t ws_bytes, void* stream) {
  MOE_REQUIRE(T >= 0 && H >= 1 && E >= 1 && k >= 1 && k <= E,
              MOE_ERR_INVALID_ARG, "bad sizes (T=%lld H=%d E=%d k=%d)",
              (long long)T, H, E, k);
  MOE_REQUIRE(E <= MOE_MAX_EXPERTS && k <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED,
              "E <= %d and k <= %d required", MOE_MAX_EXPERTS, MOE_MAX_TOPK);
  MOE_REQUIRE(T * (int64_t)k <= (int64_t)INT32_MAX, MOE_ERR_UNSUPPORTED,
              "T*k must fit in int32");
  MOE_REQUIRE(out_prec == MOE_PREC_BF16 || out_prec == MOE_PREC_MXFP8_E4M3,
              MOE_ERR_INVALID_ARG, "bad precision");
  if (out_prec == MOE_PREC_BF16)
    MOE_REQUIRE(H % 8 == 0, MOE_ERR_UNSUPPORTED, "H %% 8 != 0");
  else
    MOE_REQUIRE(H % 32 == 0, MOE_ERR_UNSUPPORTED, "H %% 32 != 0 (MXFP8)");
  MOE_REQUIRE(split_sizes && offsets, MOE_ERR_INVALID_ARG,
              "null split_sizes/offsets");
  if (T > 0) {
    MOE_REQUIRE(x && topk_idx && x_perm && row_map && src_row,
                MOE_ERR_INVALID_ARG, "null tensor pointer");
    MOE_REQUIRE(aligned16(x) && aligned16(x_perm), MOE_ERR_UNSUPPORTED,
                "x / x_perm must be 16-byte aligned");
    if (out_prec == MOE_PREC_MXFP8_E4M3)
      MOE_REQUIRE(x_perm_scale != nullptr, MOE_ERR_INVALID_ARG,
                  "MXFP8 permute needs x_perm_scale");
    MOE_REQUIRE(w_perm == nullptr || topk_w != nullptr, MOE_ERR_INVALID_ARG,
                "w_perm requested without topk_w");
  }
  const size_t need = moe::permute_ws_bytes(T, E, k);
  MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE,
              "permute workspace needs %zu bytes", need);
  hipStream_t st = as_stream(stream);
  hipError_t e = moe::launch_permute_index(topk_idx, T, E, k, row_map, src_row,
                                           split_sizes, offsets, ws,
                                           ctx->status, st);
  if (e != hipSuccess) return hip_status(e, "permute index");
  if (out_prec == MOE_PREC_BF16)
    e = moe::launch_gather_rows(x, row_map, topk_w, T, H, k, x_perm, w_perm, st);
  else
    e = moe::launch_gather_rows_mx(x, row_map, topk_w, T, H, k,
                                   static_cast<uint8_t*>(x_perm), x_perm_scale,
                                   w_perm, st);
  return hip_status(e, "permute gather");
}

}  // namespace

extern "C" {

moe_status_t moe_permute(moe_ctx_t ctx, const void* x,
                         const int32_t* topk_idx, const float* topk_w,
                         int64_t T, int32_t H, int32_t E, int32_t k,
                         moe_precision_t out_prec, void* x_perm,
                         uint8_t* x_perm_scale, float* w_perm,
                         int32_t* row_map, int32_t* src_row,
                         int32_t* split_sizes, int32_t* offsets, void* ws,
                         size_t ws_bytes, void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  return permute_impl(ctx, x, topk_idx, topk_w, T, H, E, k, out_prec, x_perm,
                      x_perm_scale, w_perm, row_map, src_row, split_sizes,
                      offsets, ws, ws_bytes, stream);
}

moe_status_t moe_permute_noalloc(moe_ctx_t ctx, const void* x,
                                 const int32_t* topk_idx,
                                 const float* topk_w, int64_t T, int32_t H,
                                 int32_t E, int32_t k,
                                 moe_precision_t out_prec, void* x_perm,
                                 uint8_t* x_perm_scale, float* w_perm,
                                 int32_t* row_map, int32_t* src_row,
                                 int32_t* split_sizes, int32_t* offsets,
                                 void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(T >= 0 && E >= 1 && k >= 1, MOE_ERR_INVALID_ARG,
              "bad sizes (T=%lld E=%d k=%d)", (long long)T, E, k);
  const size_t need = moe::permute_ws_bytes(T, E, k);
  const size_t have = moe::permute_scratch_bytes();
  MOE_REQUIRE(need <= have, MOE_ERR_UNSUPPORTED,
              "moe_permute_noalloc: T*k = %lld pairs over E = %d experts need "
              "%zu bytes of scratch, more than the %zu of its static array "
              "(call moe_permute with a workspace)",
              (long long)(T * (int64_t)k), E, need, have);
  return permute_impl(ctx, x, topk_idx, topk_w, T, H, E, k, out_prec, x_perm,
                      x_perm_scale, w_perm, row_map, src_row, split_sizes,
                      offsets, ctx->perm_scratch, have, stream);
}

moe_status_t moe_gather_rows(moe_ctx_t ctx, const void* src,
                             const int32_t* row_map, int64_t T, int32_t H,
                             int32_t k, void* dst, void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(T >= 0 && H >= 1 && k >= 1 && k <= MOE_MAX_TOPK,
              MOE_ERR_INVALID_ARG, "bad sizes");
  MOE_REQUIRE(H % 8 == 0, MOE_ERR_UNSUPPORTED, "H %% 8 != 0");
  if (T == 0) return ok();
  MOE_REQUIRE(src && row_map && dst, MOE_ERR_INVALID_ARG, "null pointer");
  MOE_REQUIRE(aligned16(src) && aligned16(dst), MOE_ERR_UNSUPPORTED,
              "src / dst must be 16-byte aligned");
  return hip_status(moe::launch_gather_rows(src, row_map, nullptr, T, H, k,
                                            dst, nullptr, as_stream(stream)),
                    "gather rows");
}

moe_status_t moe_unpermute(moe_ctx_t ctx, const void* z_perm,
                           const int32_t* row_map, const float* topk_w,
                           int64_t T, int32_t H, int32_t k, void* y,
                           void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(T >= 0 && H >= 1 && k >= 1 && k <= MOE_MAX_TOPK,
              MOE_ERR_INVALID_ARG, "bad sizes");
  MOE_REQUIRE(H % 8 == 0, MOE_ERR_UNSUPPORTED, "H %% 8 != 0");
  if (T == 0) return ok();
  MOE_REQUIRE(z_perm && row_map && y, MOE_ERR_INVALID_ARG, "null pointer");
  MOE_REQUIRE(aligned16(z_perm) && aligned16(y), MOE_ERR_UNSUPPORTED,
              "z_perm / y must be 16-byte aligned");
  return hip_status(moe::launch_unpermute(z_perm, row_map, topk_w, T, H, k, y,
                                          as_stream(stream)),
                    "unpermute");
}

moe_status_t moe_unpermute_probs_grad(moe_ctx_t ctx, const float* dw_perm,
                                      const int32_t* row_map, int64_t T,
                                      int32_t k, float* dprobs, void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(T >= 0 && k >= 1, MOE_ERR_INVALID_ARG, "bad sizes");
  if (T == 0) return ok();
  MOE_REQUIRE(dw_perm && row_map && dprobs, MOE_ERR_INVALID_ARG,
              "null pointer");
  return hip_status(moe::launch_probs_grad(dw_perm, row_map, T, k, dprobs,
                                           as_stream(stream)),
                    "probs grad");
}

moe_status_t mxfp8_quantize(moe_ctx_t ctx, const void* src, int64_t batch,
                            int64_t rows, int64_t cols, moe_mx_axis_t axis,
                            const int32_t* seg_offsets, int32_t n_seg,
                            uint8_t* codes, uint8_t* scales, void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(batch >= 0 && rows >= 0 && cols >= 0, MOE_ERR_INVALID_ARG,
              "negative size");
  MOE_REQUIRE(axis == MOE_MX_ROWWISE || axis == MOE_MX_COLWISE,
              MOE_ERR_INVALID_ARG, "bad axis");
  if (batch * rows * cols == 0) return ok();
  MOE_REQUIRE(src && codes && scales, MOE_ERR_INVALID_ARG, "null pointer");
  MOE_REQUIRE(aligned16(src) && aligned16(codes), MOE_ERR_UNSUPPORTED,
              "src / codes must be 16-byte aligned");
  hipStream_t st = as_stream(stream);
  if (axis == MOE_MX_ROWWISE) {
    MOE_REQUIRE(seg_offsets == nullptr, MOE_ERR_INVALID_ARG,
                "segments apply to COLWISE only");
    MOE_REQUIRE(cols % 32 == 0, MOE_ERR_UNSUPPORTED, "cols %% 32 != 0");
    return hip_status(moe::launch_mx_quant_rows(src, batch * rows, cols, codes,
                                                scales, st),
                      "mxfp8 rows");
  }
  MOE_REQUIRE(cols % 8 == 0, MOE_ERR_UNSUPPORTED, "cols %% 8 != 0 (COLWISE)");
  if (seg_offsets == nullptr) {
    MOE_REQUIRE(rows % 32 == 0, MOE_ERR_UNSUPPORTED, "rows %% 32 != 0");
    MOE_REQUIRE(rows / 32 <= 0x7fffffff && batch <= 65535, MOE_ERR_UNSUPPORTED,
                "tensor too large");
    return hip_status(moe::launch_mx_quant_cols(src, batch, rows, cols, codes,
                                                scales, st),
                      "mxfp8 cols");
  }
  MOE_REQUIRE(batch == 1, MOE_ERR_INVALID_ARG, "segments need batch == 1");
  MOE_REQUIRE(n_seg >= 1 && n_seg <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED,
              "1 <= n_seg <= %d", MOE_MAX_EXPERTS);
  const int64_t ld = (rows + 32 * (int64_t)n_seg + 31) / 32 * 32;
  return hip_status(moe::launch_mx_quant_segments(src, rows, cols, seg_offsets,
                                                  n_seg, 32, ld, codes, scales,
                                                  ctx->status, st),
                    "mxfp8 segments");
}

moe_status_t mxfp8_quantize_f32(moe_ctx_t ctx, const float* src, int64_t rows,
                                int64_t cols, uint8_t* codes, uint8_t* scales,
                                void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(rows >= 0 && cols >= 0, MOE_ERR_INVALID_ARG, "negative size");
  MOE_REQUIRE(cols % 32 == 0, MOE_ERR_UNSUPPORTED, "cols %% 32 != 0");
  if (rows * cols == 0) return ok();
  MOE_REQUIRE(src && codes && scales, MOE_ERR_INVALID_ARG, "null pointer");
  MOE_REQUIRE(aligned16(src) && (reinterpret_cast<uintptr_t>(codes) & 7) == 0,
              MOE_ERR_UNSUPPORTED,
              "src must be 16-byte and codes 8-byte aligned");
  return hip_status(moe::launch_mx_quant_f32(src, rows * cols, codes, scales,
                                             as_stream(stream)),
                    "mxfp8 f32 rows");
}

namespace {

moe_status_t check_mlp_dims(int32_t E, int32_t H, int32_t F, int64_t rows,
                            moe_precision_t prec) {
  MOE_REQUIRE(E >= 1 && H >= 1 && F >= 1 && rows >= 0, MOE_ERR_INVALID_ARG,
              "bad sizes (E=%d H=%d F=%d rows=%lld)", E, H, F,
              (long long)rows);
  MOE_REQUIRE(E <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED, "E > %d",
              MOE_MAX_EXPERTS);
  MOE_REQUIRE(prec == MOE_PREC_BF16 || prec == MOE_PREC_MXFP8_E4M3 ||
                  prec == MOE_PREC_FP8_TENSOR,
              MOE_ERR_INVALID_ARG, "bad precision");
  // K steps of 64 (bf16) / 128 (8-bit) without masking; N tails are masked
  const int kq = prec == MOE_PREC_BF16 ? 64 : 128;
  MOE_REQUIRE(H % kq == 0 && F % kq == 0, MOE_ERR_UNSUPPORTED,
              "H and F must be multiples of %d", kq);
  // GEMM operands are addressed with 32-bit byte offsets inside one
  // expert's activation rows (plus a 256-row tile overhang) or weights
  const int64_t widest = (int64_t)(H > 2 * F ? H : 2 * F) * 2;
  MOE_REQUIRE(rows <= (int64_t)INT32_MAX / 2 &&
                  (rows + 256) * widest < ((int64_t)1 << 32) &&
                  (int64_t)F * 2 * H * 2 < ((int64_t)1 << 32),
              MOE_ERR_UNSUPPORTED,
              "tensor too large (an expert's operand must stay below 4 GiB)");
  return MOE_OK;
}

}  // namespace

moe_status_t moe_grouped_mlp_fwd_workspace_size(const moe_mlp_fwd_args* a,
                                                size_t* bytes) {
  MOE_REQUIRE(a && bytes, MOE_ERR_INVALID_ARG, "null pointer");
  moe_status_t s = check_mlp_dims(a->E, a->H, a->F, a->rows, a->precision);
  if (s != MOE_OK) return s;
  if (a->precision == MOE_PREC_BF16)
    *bytes = moe::mlp_fwd_bf16_ws_bytes(a->E, a->H, a->F, a->rows,
                                        a->a_save == nullptr);
  else if (a->precision == MOE_PREC_FP8_TENSOR)
    *bytes = moe::mlp_fwd_fp8t_ws_bytes(a->E, a->H, a->F, a->rows,
                                        a->a_save == nullptr,
                                        a->w_gu_q == nullptr);
  else
    *bytes = moe::mlp_fwd_mx_ws_bytes(
        a->E, a->H, a->F, a->rows, a->x_perm_scale == nullptr,
        a->w_gu_q == nullptr || a->w_dn_q == nullptr);
  return ok();
}

moe_status_t moe_grouped_mlp_fwd(moe_ctx_t ctx, const moe_mlp_fwd_args* a,
                                 void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(a != nullptr, MOE_ERR_INVALID_ARG, "null args");
  s = check_mlp_dims(a->E, a->H, a->F, a->rows, a->precision);
  if (s != MOE_OK) return s;
  MOE_REQUIRE(a->offsets != nullptr, MOE_ERR_INVALID_ARG, "null offsets");
  MOE_REQUIRE((a->x_perm && a->z_perm) || a->rows == 0, MOE_ERR_INVALID_ARG,
              "null x_perm / z_perm");
  const bool mx = a->precision == MOE_PREC_MXFP8_E4M3;
  const bool f8t = a->precision == MOE_PREC_FP8_TENSOR;
  if (f8t) {
    MOE_REQUIRE(!a->x_perm_scale && !a->w_gu_s && !a->w_dn_s,
                MOE_ERR_INVALID_ARG,
                "FP8 tensor mode takes bf16 x_perm (and float32 weight "
                "scales in w_gu_ts / w_dn_ts)");
    const bool any = a->w_gu_q || a->w_gu_ts || a->w_dn_q || a->w_dn_ts;
    MOE_REQUIRE(!any || (a->w_gu_q && a->w_gu_ts && a->w_dn_q && a->w_dn_ts),
                MOE_ERR_INVALID_ARG,
                "pre-quantised FP8 weights: all of w_gu_q, w_gu_ts, w_dn_q, "
                "w_dn_ts or none");
  } else {
    MOE_REQUIRE(!a->w_gu_ts && !a->w_dn_ts, MOE_ERR_INVALID_ARG,
                "w_gu_ts / w_dn_ts are FP8 tensor-scaled inputs");
  }
  const bool preq = (mx || f8t) && a->w_gu_q != nullptr &&
                    a->w_dn_q != nullptr;
  if (!preq)
    MOE_REQUIRE(a->w_gu && a->w_dn, MOE_ERR_INVALID_ARG, "null weights");
  if (mx && a->w_gu_q) MOE_REQUIRE(a->w_gu_s, MOE_ERR_INVALID_ARG, "w_gu_s");
  if (mx && a->w_dn_q) MOE_REQUIRE(a->w_dn_s, MOE_ERR_INVALID_ARG, "w_dn_s");
  // scale rows are read one dword (4 blocks of 32) at a time
  auto al4 = [](const void* q) {
    return (reinterpret_cast<uintptr_t>(q) & 3u) == 0;
  };
  if (mx)
    MOE_REQUIRE(al4(a->x_perm_scale) && al4(a->w_gu_s) && al4(a->w_dn_s),
                MOE_ERR_UNSUPPORTED, "MXFP8 scale arrays must be 4-byte aligned");
  MOE_REQUIRE(mx || (!a->a_q_save && !a->a_s_save), MOE_ERR_INVALID_ARG,
              "a_q_save / a_s_save are MXFP8 outputs");
  MOE_REQUIRE(aligned16(a->a_q_save), MOE_ERR_UNSUPPORTED,
              "a_q_save must be 16-byte aligned");
  MOE_REQUIRE(aligned16(a->x_perm) && aligned16(a->w_gu) &&
                  aligned16(a->w_dn) && aligned16(a->w_gu_q) &&
                  aligned16(a->w_dn_q) && aligned16(a->z_perm),
              MOE_ERR_UNSUPPORTED, "operands must be 16-byte aligned");
  size_t need = 0;
  s = moe_grouped_mlp_fwd_workspace_size(a, &need);
  if (s != MOE_OK) return s;
  MOE_REQUIRE(a->ws != nullptr && a->ws_bytes >= need, MOE_ERR_WORKSPACE,
              "grouped_mlp_fwd workspace needs %zu bytes", need);
  hipError_t e;
  if (f8t) {
    MOE_REQUIRE(aligned16(a->h1_save) && aligned16(a->a_save),
                MOE_ERR_UNSUPPORTED, "saves must be 16-byte aligned");
    e = moe::launch_mlp_fwd_fp8t(a->E, a->H, a->F, a->rows, a->x_perm,
                                 a->w_gu, a->w_dn, a->w_gu_q, a->w_gu_ts,
                                 a->w_dn_q, a->w_dn_ts, a->w_perm, a->offsets,
                                 a->z_perm, a->h1_save, a->a_save, a->ws,
                                 ctx->cu_count, ctx->status,
                                 as_stream(stream));
  } else if (!mx) {
    e = moe::launch_mlp_fwd_bf16(a->E, a->H, a->F, a->rows, a->x_perm, a->w_gu,
                                 a->w_dn, a->w_perm, a->offsets, a->z_perm,
                                 a->h1_save, a->a_save, a->ws, ctx->cu_count,
                                 ctx->status, as_stream(stream));
  } else {
    const bool xq = a->x_perm_scale != nullptr;
    e = moe::launch_mlp_fwd_mx(
        a->E, a->H, a->F, a->rows, xq ? nullptr : a->x_perm,
        xq ? static_cast<const uint8_t*>(a->x_perm) : nullptr,
        a->x_perm_scale, a->w_gu, a->w_dn, a->w_gu_q, a->w_gu_s, a->w_dn_q,
        a->w_dn_s, a->w_perm, a->offsets, a->z_perm, a->h1_save, a->a_save,
        a->a_q_save, a->a_s_save, a->ws, ctx->cu_count, ctx->status,
        as_stream(stream));
  }
  return hip_status(e, "grouped_mlp_fwd");
}

moe_status_t moe_expert_loop_mlp_fwd_workspace_size(const moe_mlp_fwd_args* a,
                                                    size_t* bytes) {
  MOE_REQUIRE(a && bytes, MOE_ERR_INVALID_ARG, "null pointer");
  MOE_REQUIRE(a->precision == MOE_PREC_BF16, MOE_ERR_UNSUPPORTED,
              "the per-expert loop is bf16 only");
  moe_status_t s = check_mlp_dims(a->E, a->H, a->F, a->rows, a->precision);
  if (s != MOE_OK) return s;
  *bytes = moe::expert_loop_fwd_ws_bytes(a->E, a->F, a->rows,
                                         a->h1_save == nullptr,
                                         a->a_save == nullptr);
  return ok();
}

moe_status_t moe_expert_loop_mlp_fwd(moe_ctx_t ctx, const moe_mlp_fwd_args* a,
                                     void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(a != nullptr, MOE_ERR_INVALID_ARG, "null args");
  size_t need = 0;
  s = moe_expert_loop_mlp_fwd_workspace_size(a, &need);
  if (s != MOE_OK) return s;
  MOE_REQUIRE(a->offsets != nullptr, MOE_ERR_INVALID_ARG, "null offsets");
  MOE_REQUIRE((a->x_perm && a->z_perm) || a->rows == 0, MOE_ERR_INVALID_ARG,
              "null x_perm / z_perm");
  MOE_REQUIRE(a->w_gu && a->w_dn, MOE_ERR_INVALID_ARG, "null weights");
  MOE_REQUIRE(aligned16(a->x_perm) && aligned16(a->w_gu) &&
                  aligned16(a->w_dn) && aligned16(a->z_perm) &&
                  aligned16(a->h1_save) && aligned16(a->a_save),
              MOE_ERR_UNSUPPORTED, "operands must be 16-byte aligned");
  MOE_REQUIRE(a->ws != nullptr && a->ws_bytes >= need, MOE_ERR_WORKSPACE,
              "expert_loop_mlp_fwd workspace needs %zu bytes", need);
  // the loop reads the per-expert row counts on the host, as a Python loop
  // over experts does: wait for the stream
  hipStream_t st = as_stream(stream);
  std::vector<int32_t> off((size_t)a->E + 1);
  hipError_t e = hipMemcpyAsync(off.data(), a->offsets,
                                off.size() * sizeof(int32_t),
                                hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_status(e, "expert_loop_mlp_fwd offsets");
  MOE_REQUIRE(off[0] == 0 && off[a->E] == a->rows, MOE_ERR_INVALID_ARG,
              "offsets must run from 0 to rows");
  for (int32_t i = 0; i < a->E; ++i)
    MOE_REQUIRE(off[i + 1] >= off[i], MOE_ERR_INVALID_ARG,
                "offsets must not decrease");
  e = moe::launch_expert_loop_fwd(a->E, a->H, a->F, a->rows, a->x_perm,
                                  a->w_gu, a->w_dn, a->w_perm, a->offsets,
                                  off.data(), a->z_perm, a->h1_save,
                                  a->a_save, a->ws, st);
  return hip_status(e, "expert_loop_mlp_fwd");
}

moe_status_t moe_grouped_mlp_bwd_workspace_size(const moe_mlp_bwd_args* a,
                                                size_t* bytes) {
  MOE_REQUIRE(a && bytes, MOE_ERR_INVALID_ARG, "null pointer");
  moe_status_t s = check_mlp_dims(a->E, a->H, a->F, a->rows, a->precision);
  if (s != MOE_OK) return s;
  MOE_REQUIRE(a->precision != MOE_PREC_FP8_TENSOR, MOE_ERR_UNSUPPORTED,
              "the FP8 tensor-scaled mode is forward only");
  if (a->precision == MOE_PREC_MXFP8_E4M3) {
    // token-direction operands [max(H, 2F)][rows + 128 E (+128)] are
    // addressed with 32-bit byte offsets
    const int64_t widest = (a->H > 2 * a->F ? a->H : 2 * (int64_t)a->F) + 256;
    const int64_t ld = a->rows + 128 * (int64_t)a->E + 128;
    MOE_REQUIRE(widest * ld < ((int64_t)1 << 32), MOE_ERR_UNSUPPORTED,
                "tensor too large for the MXFP8 weight-gradient operands");
  }
  if (a->precision == MOE_PREC_BF16)
    *bytes = moe::mlp_bwd_bf16_ws_bytes(a->E, a->H, a->F, a->rows);
  else
    *bytes = moe::mlp_bwd_mx_ws_bytes(a->E, a->H, a->F, a->rows,
                                      a->w_gu_qt == nullptr ||
                                          a->w_dn_qt == nullptr);
  return ok();
}

moe_status_t moe_grouped_mlp_bwd(moe_ctx_t ctx, const moe_mlp_bwd_args* a,
                                 void* stream) {
  moe_status_t s = check_ctx(ctx);
  if (s != MOE_OK) return s;
  TimerGuard tg(ctx);
  MOE_REQUIRE(a != nullptr, MOE_ERR_INVALID_ARG, "null args");
  s = check_mlp_dims(a->E, a->H, a->F, a->rows, a->precision);
  if (s != MOE_OK) return s;
  MOE_REQUIRE(a->precision != MOE_PREC_FP8_TENSOR, MOE_ERR_UNSUPPORTED,
              "the FP8 tensor-scaled mode is forward only");
  MOE_REQUIRE(a->offsets && a->w_gu && a->w_dn && a->dw_gu && a->dw_dn,
              MOE_ERR_INVALID_ARG, "null offsets / weights / weight grads");
  if (a->rows > 0)
    MOE_REQUIRE(a->x_perm && a->h1_save && a->a_save && a->dz_perm &&
                    a->dx_perm,
                MOE_ERR_INVALID_ARG, "null activation pointer");
  MOE_REQUIRE(a->w_perm != nullptr || a->dw_perm == nullptr ||
                  a->rows == 0,
              MOE_ERR_INVALID_ARG, "dw_perm needs w_perm");
  const bool mxb = a->precision == MOE_PREC_MXFP8_E4M3;
  MOE_REQUIRE(mxb || (!a->w_gu_qt && !a->w_gu_st && !a->w_dn_qt &&
                      !a->w_dn_st),
              MOE_ERR_INVALID_ARG, "pre-quantised weights are MXFP8 inputs");
  MOE_REQUIRE(!a->w_gu_qt == !a->w_gu_st && !a->w_dn_qt == !a->w_dn_st,
              MOE_ERR_INVALID_ARG, "codes and scales go together");
  MOE_REQUIRE(aligned16(a->w_gu_qt) && aligned16(a->w_dn_qt) &&
                  (reinterpret_cast<uintptr_t>(a->w_gu_st) & 3u) == 0 &&
                  (reinterpret_cast<uintptr_t>(a->w_dn_st) & 3u) == 0,
              MOE_ERR_UNSUPPORTED,
              "pre-quantised codes 16-byte, scales 4-byte aligned");
  size_t need = 0;
  s = moe_grouped_mlp_bwd_workspace_size(a, &need);
  if (s != MOE_OK) return s;
  MOE_REQUIRE(a->ws != nullptr && a->ws_bytes >= need, MOE_ERR_WORKSPACE,
              "grouped_mlp_bwd workspace needs %zu bytes", need);
  hipError_t e;
  if (a->precision == MOE_PREC_BF16)
    e = moe::launch_mlp_bwd_bf16(a->E, a->H, a->F, a->rows, a->x_perm, a->w_gu,
                                 a->w_dn, a->w_perm, a->offsets, a->h1_save,
                                 a->a_save, a->dz_perm, a->dx_perm, a->dw_gu,
                                 a->dw_dn, a->w_perm ? a->dw_perm : nullptr,
                                 a->ws, ctx->status, as_stream(stream));
  else
    e = moe::launch_mlp_bwd_mx(a->E, a->H, a->F, a->rows, a->x_perm, a->w_gu,
                               a->w_dn, a->w_perm, a->offsets, a->h1_save,
                               a->a_save, a->dz_perm, a->dx_perm, a->dw_gu,
                               a->dw_dn, a->w_perm ? a->dw_perm : nullptr,
                               a->w_gu_qt, a->w_gu_st, a->w_dn_qt,
                               a->w_dn_st, a->ws, ctx->status,
                               as_stream(stream));
  return hip_status(e, "grouped_mlp_bwd");
}

}  // extern "C"
