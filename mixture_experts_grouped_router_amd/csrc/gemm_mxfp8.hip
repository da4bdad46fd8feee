// MXFP8 grouped MLP (scaled-MFMA GEMMs).  Placeholder entry points until the
// scaled-MFMA kernels land: every call reports hipErrorNotSupported.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

size_t mlp_fwd_mx_ws_bytes(int, int, int, int64_t, bool, bool) { return 256; }
hipError_t launch_mlp_fwd_mx(int, int, int, int64_t, const void*,
                             const uint8_t*, const uint8_t*, const void*,
                             const void*, const uint8_t*, const uint8_t*,
                             const uint8_t*, const uint8_t*, const float*,
                             const int32_t*, void*, void*, void*, void*,
                             hipStream_t) {
  return hipErrorNotSupported;
}
size_t mlp_bwd_mx_ws_bytes(int, int, int, int64_t) { return 256; }
hipError_t launch_mlp_bwd_mx(int, int, int, int64_t, const void*, const void*,
                             const void*, const float*, const int32_t*,
                             const void*, const void*, const void*, void*,
                             void*, void*, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moe
