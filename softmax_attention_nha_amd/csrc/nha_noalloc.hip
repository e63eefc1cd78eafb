// nha_noalloc.hip -- the scratch array of the allocation-free forward
// (nha_fwd_noalloc in include/nha.h), for callers that cannot allocate device
// memory: code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy from module load until the process ends.  On the host
// its name is only a stand-in, never a device address, so host code uses the
// address hipGetSymbolAddress returns for the current device (looked up once
// per device, with that device current) wherever it needs the array: as the
// forward's workspace pointer.
#include <mutex>

#include "nha_internal.h"

namespace nha {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
std::mutex scratch_mu;
void* scratch_addr[64];  // per device: the array's device address, once looked up
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_addr[dev] = p;
  }
  *ptr = scratch_addr[dev];
  return hipSuccess;
}

}  // namespace nha
