// noalloc.hip -- the device scratch of the allocation-free forward call (sol_attn_fwd_noalloc).
//
// One file-scope array per GPU serves as that call's workspace: the code object reserves it when
// the library's kernels are loaded on a device, and it stays until the process ends.  Host code
// never uses the array's name as an address (on the host it is only a stand-in symbol); the
// device address of each GPU's copy is looked up once per device with hipGetSymbolAddress, with
// that device current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace solattn {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = p;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace solattn
