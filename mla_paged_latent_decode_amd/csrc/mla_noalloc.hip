// The built-in scratch of mla_decode_noalloc (include/mla.h): the stage-1
// partials and per-sequence records that mla_decode keeps in the caller's
// workspace live here instead, in a file-scope device array of a fixed size,
// so that the call needs no allocation at all.  Each device the library runs
// on holds its own copy of the array until the process ends; host code never
// uses the array's name as an address, only the device address looked up for
// the current device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla_internal.h"

namespace mla {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];
}  // namespace

int noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  // looked up once per device, with that device current
  std::call_once(g_once[dev], [dev] {
    g_err[dev] = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_err[dev] != hipSuccess) return (int)g_err[dev];
  *ptr = g_ptr[dev];
  return 0;
}

}  // namespace mla
