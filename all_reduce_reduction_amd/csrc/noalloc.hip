// noalloc.hip -- the fixed device scratch of sim_allreduce_noalloc.
//
// Callers that cannot allocate device memory while they run (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc)
// use an all-reduce entry point whose only scratch -- the fp32 partial slots
// of the 16-bit ring -- is this file-scope array instead of a buffer the
// library allocates.  The code object carries the array, so each device the
// library is loaded on holds its own copy, at its own address, from module
// load until the process ends.
//
// In host code the array's name is only a host-side stand-in for the
// symbol, never a device address: the address is looked up once per device
// (noalloc_setup, called by sim_init with that device current) and every
// later use goes through noalloc_scratch().
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "simar.h"

namespace {
__device__ __align__(256) unsigned char scratch[SIM_NOALLOC_SCRATCH_BYTES];
void* g_scratch_ptr[simar::kMaxDevices];
}  // namespace

namespace simar {

int noalloc_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return SIM_ERR_INVALID_ARG;
  if (g_scratch_ptr[device]) return SIM_OK;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();
    return SIM_ERR_HIP;
  }
  g_scratch_ptr[device] = ptr;
  return SIM_OK;
}

void* noalloc_scratch(int device) {
  return (device >= 0 && device < kMaxDevices) ? g_scratch_ptr[device] : nullptr;
}

}  // namespace simar
