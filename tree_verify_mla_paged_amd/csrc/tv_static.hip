// Device-resident scratch for tv_verify_attn_static: the workspace of a call
// (visibility words, split partial outputs and LSEs, dispatch order) taken
// from a file-scope device array instead of a caller allocation, for callers
// that cannot allocate device memory.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, from the moment the code object is loaded until the process ends.
// In host code the array's name is only a host-side handle: its device address
// is looked up once per device (hipGetSymbolAddress, with that device current)
// and that address is what the kernels receive.  Every call on a GPU shares
// the array, so calls that overlap on one GPU race; a call overwrites every
// byte it later reads, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "treeverify.h"
#include "tv_kernels.h"

namespace tv {

static __device__ __align__(256) uint8_t scratch[TV_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
}  // namespace

hipError_t static_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    // the current device's copy; two threads racing here both store the same
    // address
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace tv
