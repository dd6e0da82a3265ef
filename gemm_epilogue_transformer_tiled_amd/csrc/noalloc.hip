// Static device scratch for gemm_epilogue_run_noalloc, the entry point that allocates nothing.
//
// The array below lives in the library's code object: every GPU the library runs on holds its
// own copy, at its own address, from the moment the code object is loaded on that device until
// the process ends.  Host code never passes the array's name to a kernel (on the host that
// name is only a stand-in, not a device address); it looks up the device address once per
// device with hipGetSymbolAddress and uses that pointer everywhere.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gemm_epilogue.h"
#include "ge_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[GE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

namespace ge {

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // once per device, with that device current (it is: hipGetDevice above names it)
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace ge
