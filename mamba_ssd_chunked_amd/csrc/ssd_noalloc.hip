// ssd_forward without a workspace argument: the workspace is a fixed device
// array of the library, so the call allocates nothing (for callers that cannot
// allocate device memory).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/ssd.h"

static_assert(SSD_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");

// One copy per device, held from the first launch on that device until the
// process ends. Host code never uses this name as an address (on the host it
// names a stand-in, not device memory); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of each device's copy, once looked up

// The current device's copy of scratch, looked up on its first use there.
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SSD_E_HIP;
  if (dev >= kMaxDevices) return SSD_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSD_E_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SSD_OK;
}

}  // namespace

extern "C" int ssd_forward_noalloc(const ssd_shape* shape, int path, const void* X, const void* dt,
                                   const float* A, const void* B, const void* C, const float* D,
                                   const ssd_scales* scales, void* Y, const void* initial_state,
                                   void* final_state, const ssd_taps* taps, void* stream) {
  if (!shape) return SSD_E_NULL;
  ssd_shape sh = *shape;
  size_t need = ssd_workspace_bytes(&sh, path);
  // the automatic choice falls back to the head-persistent schedule when the
  // chunk-parallel one would not fit
  if (need > SSD_NOALLOC_SCRATCH_BYTES && sh.schedule == SSD_SCHED_AUTO) {
    sh.schedule = SSD_SCHED_HEAD;
    need = ssd_workspace_bytes(&sh, path);
  }
  if (need > SSD_NOALLOC_SCRATCH_BYTES) return SSD_E_TOO_LARGE;
  void* ws = nullptr;
  const int rc = scratch_of_current_device(&ws);
  if (rc != SSD_OK) return rc;
  return ssd_forward(&sh, path, X, dt, A, B, C, D, scales, Y, initial_state, final_state, ws,
                     SSD_NOALLOC_SCRATCH_BYTES, taps, stream);
}
