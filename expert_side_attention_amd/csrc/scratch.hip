// Fixed device scratch for the forward entry point that allocates nothing.
//
// The array lives in the library's code object: every device the library
// runs on holds its own copy, from the first use on that device until the
// process ends.  In host code `scratch` names a host-side stand-in, not
// device memory, so the device address is looked up once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace afd {
namespace {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_addr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t static_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // first call on this device (with it current): look the address up
  std::call_once(g_once[dev], [dev] {
    g_err[dev] = hipGetSymbolAddress(&g_addr[dev], HIP_SYMBOL(scratch));
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_addr[dev];
  return hipSuccess;
}

}  // namespace afd
