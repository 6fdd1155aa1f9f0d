// Host-only stand-ins for the kernel launchers and the two HIP runtime calls
// that ssd_api.cpp makes, so the C ABI's validation, size arithmetic and
// workspace carving can run under AddressSanitizer and UBSan on a machine
// without a GPU. Every launcher counts its call and returns success; nothing
// is read from or written to the (fake) device addresses.
#include <hip/hip_runtime.h>

#include "ssd_launch.hpp"

int g_launches = 0;

namespace {
hipError_t ok() {
  ++g_launches;
  return hipSuccess;
}
}  // namespace

extern "C" hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return ok(); }

namespace ssd {

hipError_t launch_quantize_bc(const Dims&, int, const void*, const void*, const float*, const float*, int8_t*,
                              int8_t*, hipStream_t) {
  return ok();
}
hipError_t launch_chunk_cumsum(const Dims&, int, const void*, const float*, float*, float*, uint8_t*, hipStream_t) {
  return ok();
}
hipError_t launch_quantize_x(const Dims&, int, const void*, const float*, int8_t*, hipStream_t) { return ok(); }
hipError_t launch_chunk_state(const Dims&, int, int, const void*, const float*, const void*, const float*,
                              const float*, const float*, const float*, void*, int8_t*, int32_t*, hipStream_t) {
  return ok();
}
hipError_t launch_state_passing(const Dims&, bool, void*, const float*, const uint8_t*, const void*, void*,
                                hipStream_t) {
  return ok();
}
hipError_t launch_chunk_bmm(const Dims&, int, bool, const void*, const void*, void*, hipStream_t) { return ok(); }
hipError_t launch_chunk_scan(const Dims&, int, int, const void*, const void*, const float*, const void*,
                             const void*, const void*, const void*, const float*, const float*, const float*,
                             const float*, const float*, void*, hipStream_t) {
  return ok();
}
hipError_t launch_forward_fused(const Dims&, int, bool, const void*, const void*, const float*, const void*,
                                const void*, const float*, const ScalePtrs&, void*, const void*, void*, void*,
                                int8_t*, int32_t*, int8_t*, int8_t*, hipStream_t) {
  return ok();
}
// the fused kernels take fp16 and bf16 inputs; the workspace stands in for
// the real carve-up with one float per (batch, head, chunk, position)
bool fused_supported(const Dims&, int dtype, bool) { return dtype != 0; }
size_t fused_workspace_bytes(const Dims& d, bool) { return (size_t)d.B * d.H * d.c * d.l * 4; }
hipError_t launch_amax_bc(const Dims&, int, const void*, const void*, float*, float*, hipStream_t) { return ok(); }
hipError_t launch_amax_xs(const Dims&, int, const void*, const float*, float*, hipStream_t) { return ok(); }
hipError_t launch_amax_states(const Dims&, const float*, float*, hipStream_t) { return ok(); }
int cu_count() { return 256; }
hipError_t launch_decode_step(const Dims&, int, bool, const void*, const void*, const float*, const void*,
                              const void*, const float*, const ScalePtrs&, void*, void*, hipStream_t) {
  return ok();
}
hipError_t launch_epilogue(const Dims&, int, const void*, const float*, float, const float*, float, void*,
                           hipStream_t) {
  return ok();
}
hipError_t launch_mean_correction(const Dims&, int, const void*, const void*, float*, hipStream_t) { return ok(); }
hipError_t launch_zero_fill(void*, size_t, hipStream_t) { return ok(); }

}  // namespace ssd
