// Fused SSD forward (placeholder: the module composition is used until the
// fused kernels land).
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

bool fused_supported(const Dims&, int, bool) { return false; }

size_t fused_workspace_bytes(const Dims&, bool) { return 0; }

hipError_t launch_forward_fused(const Dims&, int, bool, const void*, const void*, const float*,
                                const void*, const void*, const float*, const ScalePtrs&, void*,
                                void*, void*, int8_t*, int32_t*, int8_t*, int8_t*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace ssd
