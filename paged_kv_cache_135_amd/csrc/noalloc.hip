// Scratch memory of the allocation-free decode entry point
// (paged_attention_decode_noalloc): one file-scope device array, which every
// GPU the library runs on holds from module load until the process ends.
//
// In host code the array's name is only a host-side stand-in; the array's
// device address on the current GPU comes from hipGetSymbolAddress, taken once
// per device (each GPU has its own copy at its own address) and kept here.
// Only that address is ever handed to a kernel.
#include <atomic>

#include "pkv_internal.h"

namespace pkv {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_for_current_device(void** ptr) {
  static std::atomic<void*> addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // first call on this device, with this device current
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);  // host threads store the same value
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace pkv
