// launch.h -- how every kernel of the library is enqueued.
//
// The by-address launch (hipLaunchKernelGGL / hipLaunchKernel) looks the
// kernel up from its host stub on every call.  Here the kernel's function
// handle on the library's device is looked up once (hipGetFuncBySymbol) and
// each launch goes straight to hipModuleLaunchKernel with it: about 0.2 us
// less host time per launch on MI355X (2.1 instead of 2.3 us for a kernel
// with a 32-byte argument block), which is most of a small all-reduce's
// cost.  launch<K>() returns the launch's own status; on failure the
// runtime's last-error state is cleared, as the by-address form's callers
// did with hipGetLastError.
//
// The arguments are converted to the kernel's own parameter types (taken
// from K's signature), so each pointer handed to the runtime addresses an
// object of exactly the size the kernel's argument layout expects.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace simar {

template <auto K>
struct Kernel;

template <class... P, void (*K)(P...)>
struct Kernel<K> {
  static hipError_t launch(dim3 grid, dim3 block, hipStream_t s, const P&... a) {
    static hipFunction_t fn[kMaxDevices];  // per device, filled on first use
    const int d = g_launch_device;
    if (d < 0 || d >= kMaxDevices) return hipErrorInvalidDevice;
    hipFunction_t f = __atomic_load_n(&fn[d], __ATOMIC_ACQUIRE);
    if (!f) {
      // the handle for the current device, which the library has made its
      // own device before any launch
      const hipError_t e = hipGetFuncBySymbol(&f, reinterpret_cast<const void*>(K));
      if (e != hipSuccess) {
        (void)hipGetLastError();
        return e;
      }
      __atomic_store_n(&fn[d], f, __ATOMIC_RELEASE);
    }
    void* args[] = {const_cast<void*>(static_cast<const void*>(&a))...};
    const hipError_t e =
        hipModuleLaunchKernel(f, grid.x, grid.y, grid.z, block.x, block.y, block.z, 0, s, args, nullptr);
    if (e != hipSuccess) (void)hipGetLastError();
    return e;
  }
};

template <auto K, class... A>
hipError_t launch(dim3 grid, dim3 block, hipStream_t s, const A&... a) {
  return Kernel<K>::launch(grid, block, s, a...);
}

}  // namespace simar
