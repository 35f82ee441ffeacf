// Scratch of the allocation-free streaming step (gdn_step_noalloc): a
// file-scope device array stands in for the caller's workspace.  It is part of
// the library's code object, so every device the library runs on holds its
// own copy, at its own address, until the process ends.  In host code the
// array's name is only a stand-in for that address: the device address is
// taken once per device with hipGetSymbolAddress and only that pointer is
// handed to kernels.
#include <mutex>

#include "gdn_internal.h"

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace gdn {

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with device `dev` current
    addr[dev] = err[dev] == hipSuccess ? p : nullptr;
  });
  if (err[dev] != hipSuccess) return err[dev];
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace gdn
