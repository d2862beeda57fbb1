// sana_linattn_fwd_noalloc: the forward pass with its workspace in a static
// device array, for callers that cannot allocate device memory.
//
// `scratch` below exists once per GPU the library runs on and lives until the
// process ends. In host code its name is only a host-side stand-in, never a
// device address: the address of a device's copy comes from
// hipGetSymbolAddress, asked once per device with that device current, and
// only that address is handed to the kernels.

#include <hip/hip_runtime.h>

#include <mutex>

#include "linattn_internal.h"
#include "sana_linattn.h"

namespace sana {
namespace {

constexpr size_t kScratchBytes = SANA_LINATTN_SCRATCH_BYTES;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// The current device's copy of `scratch` (looked up on the first call on that
// device, then kept).
hipError_t scratch_workspace(void** workspace, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_status[dev] == hipSuccess ? p : nullptr;
  });
  if (g_status[dev] != hipSuccess) return g_status[dev];
  *workspace = g_scratch[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

}  // namespace
}  // namespace sana

extern "C" sana_status_t sana_linattn_fwd_noalloc(const void* q, const void* k, const void* v,
                                                  void* out, int64_t B, int64_t N, int64_t H,
                                                  int64_t d, float eps, sana_dtype_t dtype,
                                                  hipStream_t stream) {
  // the size limit first: a host-side check, like every other argument check
  size_t need = 0;
  const sana_status_t s = sana_linattn_workspace_size(B, N, H, d, dtype, &need);
  if (s != SANA_OK) return s;
  if (need > sana::kScratchBytes) return SANA_ERR_WORKSPACE;
  return sana::forward_from_source(q, k, v, out, B, N, H, d, eps, dtype,
                                   sana::scratch_workspace, stream);
}
