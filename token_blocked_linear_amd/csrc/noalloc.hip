// The forward for callers that cannot allocate device memory (code under HIP graph capture,
// serving loops that must not call hipMalloc, harnesses that forbid it): mhla_forward_noalloc
// runs mhla_forward with its workspace in a fixed device array of this library instead of a
// caller-owned buffer.  Nothing here allocates: the array is part of the library's code object,
// which the HIP runtime places on a device when the library's device code is loaded there, and
// each device keeps its own copy until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mhla.h"

namespace {

static_assert(MHLA_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch array keeps the workspace's alignment");

// The workspace of mhla_forward_noalloc.  In host code `scratch` names a host-side stand-in, not
// the device array: host code uses only the per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[MHLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` per device (null: not looked up)

// The device address of the current device's copy of `scratch`, looked up once per device (with
// that device current) and kept.
mhla_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MHLA_ERR_HIP;
  if (dev >= kMaxDevices) return MHLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MHLA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MHLA_OK;
}

}  // namespace

extern "C" mhla_status mhla_forward_noalloc(mhla_handle h, const void* q, const void* k, const void* v,
                                            const float* mc, void* o, void* stream) {
  if (!h) return MHLA_ERR_INVALID_ARG;
  try {
    size_t need = 0;
    mhla_status st = mhla_workspace_size(h, &need);
    if (st != MHLA_OK) return st;
    if (need > (size_t)MHLA_NOALLOC_SCRATCH_BYTES) return MHLA_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st != MHLA_OK) return st;
    return mhla_forward(h, q, k, v, mc, o, ws, (size_t)MHLA_NOALLOC_SCRATCH_BYTES, stream);
  } catch (...) {
    return MHLA_ERR_INTERNAL;
  }
}
