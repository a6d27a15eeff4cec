// k_streams.hip -- k independent streaming copies in one launch (gfx950):
// the measured bandwidth ceiling of the one-shot's memory access pattern.
//
// The fused one-shot moves 2 p S bytes through p input streams and p output
// streams at once.  Whether it is at the HBM roofline of that access
// pattern can only be told against a kernel that moves the same streams
// with no arithmetic in between, on the same GPU, in the same run: k = p
// copies here have exactly the one-shot's stream count, k = 1 is a plain
// copy.  Each lane moves 16-byte vectors with the same streaming
// (nontemporal) loads and stores, the same split of every address into a
// workgroup-uniform base in scalar registers plus one 32-bit lane offset,
// and the same grid-stride walk over spans of kBlock vectors as the fold
// kernel; copy q of a span issues all k loads before any store.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "launch.h"

namespace simar {

template <int K>
__global__ void __launch_bounds__(kBlock) k_copy_streams(CopyStreamsArgs a) {
  constexpr int MAXK = K ? K : SIM_MAX_RANKS;
  const int k = K ? K : a.k;
  const void* sp[MAXK];
  void* dp[MAXK];
#pragma unroll
  for (int q = 0; q < MAXK; q++) {
    sp[q] = (q < k) ? a.src[q] : nullptr;
    dp[q] = (q < k) ? a.dst[q] : nullptr;
  }
  const int tid = threadIdx.x;
  const int64_t nvec = a.nvec;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  auto span_body = [&](int64_t base, auto guard) {
    constexpr bool GUARD = decltype(guard)::value;
    if (GUARD && base + tid >= nvec) return;
    const int64_t sbyte = base * 16;
    const uint32_t lane = lane_offset((uint32_t)tid * 16u);
    u32x4 w[MAXK];
#pragma unroll
    for (int q = 0; q < MAXK; q++)
      if (q < k) w[q] = ld16u(sp[q], sbyte, lane);
#pragma unroll
    for (int q = 0; q < MAXK; q++)
      if (q < k) st16u(dp[q], sbyte, lane, w[q]);
  };
  int64_t base = (int64_t)blockIdx.x * kBlock;
  for (; base + kBlock <= nvec; base += stride) span_body(base, std::false_type());
  if (base < nvec) span_body(base, std::true_type());
}

hipError_t launch_copy_streams(const CopyStreamsArgs& a, int workgroups, hipStream_t s) {
  const dim3 grid((unsigned)workgroups), block(kBlock);
  switch (a.k) {
    case 1: return launch<k_copy_streams<1>>(grid, block, s, a);
    case 2: return launch<k_copy_streams<2>>(grid, block, s, a);
    case 4: return launch<k_copy_streams<4>>(grid, block, s, a);
    case 8: return launch<k_copy_streams<8>>(grid, block, s, a);
    default: return launch<k_copy_streams<0>>(grid, block, s, a);
  }
}

}  // namespace simar
