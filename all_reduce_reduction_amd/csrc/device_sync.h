// device_sync.h -- signal / wait between workgroups of one launch, and the
// device-scope accesses the data behind a signal is moved with (gfx950).
//
// After the MemoryChannel put / signal / wait of "MSCCL++ ..." (section 4):
// a producer writes its data, waits until its own stores have completed,
// meets its workgroup at a barrier, and only then stores a counter; a
// consumer's lane 0 polls the counter, the workgroup meets at a barrier, and
// only then are the data loaded.  Counters hold (epoch << 32 | count) with a
// per-call epoch, so a value left by an earlier call always compares lower
// than anything this call waits for (monotonic expected values).  Each XCD
// has its own L2 and a CU's own cache is coherent only for its own waves, so
// the data are moved with device-scope (sc1) buffer accesses and the
// counters with agent-scope atomics: both reach the memory side's coherence
// point without flushing or invalidating any cache.
#pragma once

#include "device_common.h"

namespace simar {
namespace {

__device__ __forceinline__ unsigned long long tag(unsigned epoch, unsigned long long count) {
  return ((unsigned long long)epoch << 32) | count;
}

// Device-scope (sc1) accesses through a buffer resource over one region
// (offsets are bytes; out-of-range offsets are dropped by the hardware
// bounds check of the resource).
constexpr int kSC1 = 16;  // cache-policy bit: coherent at device scope
// cache policy of the device-scope loads and stores (the build may add the
// nontemporal bit, 2, to either)
#ifndef SIMAR_FIFO_LOAD_AUX
#define SIMAR_FIFO_LOAD_AUX 16
#endif
#ifndef SIMAR_FIFO_STORE_AUX
#define SIMAR_FIFO_STORE_AUX 16
#endif
constexpr int kLd = SIMAR_FIFO_LOAD_AUX;
constexpr int kSt = SIMAR_FIFO_STORE_AUX;
static_assert((kLd & kSC1) != 0 && (kSt & kSC1) != 0, "data behind a signal must move at device scope");
__device__ __forceinline__ __amdgpu_buffer_rsrc_t fifo_rsrc(uint32_t* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
// a buffer resource over `bytes` bytes of an output buffer from byte `at`
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(void* base, int64_t at, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((char*)base + at, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// thread 0 polls *p until it reaches `want` (or the spin limit); the whole
// workgroup learns the outcome through *flag_lds.  Returns false on
// timeout.  Each call site owns its flag word: a lane reads the flag after
// this barrier and before the end-of-step barrier, and the flag is only
// rewritten (by the same call site) after that end-of-step barrier.
__device__ __forceinline__ bool wait_geq(unsigned long long* p, unsigned long long want,
                                         unsigned long long spin_limit, int* flag_lds) {
  if (threadIdx.x == 0) {
    unsigned long long v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned long long spins = 0;
    bool ok = true;
    while (v < want) {
      if (++spins > spin_limit) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *flag_lds = ok ? 1 : 0;
  }
  __syncthreads();
  return *flag_lds != 0;
}

// Lanes 0 .. n-1 of the workgroup each poll one counter, all at once, until
// it reaches `want` (or the spin limit): one poll round trip for n
// producers instead of n in a row.  The workgroup learns the outcome through
// *flag_lds; true when every counter got there.  `counter(k)` gives lane k's
// counter.  The same reuse rule as wait_geq applies to *flag_lds.
template <class Counter>
__device__ __forceinline__ bool wait_all_geq(int n, Counter counter, unsigned long long want,
                                             unsigned long long spin_limit, int* flag_lds) {
  if (threadIdx.x == 0) *flag_lds = 1;
  __syncthreads();
  if ((int)threadIdx.x < n) {
    unsigned long long* p = counter((int)threadIdx.x);
    unsigned long long v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned long long spins = 0;
    while (v < want) {
      if (++spins > spin_limit) {
        *flag_lds = 0;  // any failing lane clears it; nobody sets it back
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  return *flag_lds != 0;
}

}  // namespace
}  // namespace simar
