// k_ll.hip -- one-shot all-reduce through LL packets (gfx950).
//
// The LL protocol ("MSCCL++ ...", section 4.2 "LL (Low-Latency)
// Protocol"; "Inside NCCL all-reduce", section "Three ways to move a
// byte"): data travel in 8-byte words that carry 4 bytes of payload and a
// 4-byte flag written by the same store instruction, so a reader that sees
// the flag also sees the data beside it -- no fence and no separate
// semaphore.  The flag differs on every transfer round (here a per-call
// epoch, never 0) so a stale packet from an earlier call never matches.
//
// One launch, persistent grid (every workgroup resident at once):
//   produce: rank q's data word k is stored as the packet
//            {low 32 bits = data, high 32 bits = epoch} to ll[q][k] with a
//            64-bit agent-scope atomic store (one instruction; agent scope
//            makes it visible to the other XCDs' L2s); the p words of an
//            index are loaded together before their packets are stored;
//   consume: each workgroup then takes a tile produced by ANOTHER
//            workgroup (tile t + shift), polls the p packets of every word
//            with 64-bit agent-scope atomic loads until each carries the
//            expected flag, folds the payloads in the all-pairs order
//            (owner first, then ascending) and writes every rank's output.
// Every workgroup produces before it consumes and all workgroups are
// co-resident (the host caps the grid at the occupancy limit), so every
// poll is answered.  A lane issues its p polls together and re-polls only
// the packets still missing, at most spin_limit rounds; on expiry it
// records SIM_ERR_TIMEOUT in the device error word and raises its
// workgroup's give-up flag, and from then on every lane of the workgroup
// skips its remaining waits and writes (the outputs are undefined after a
// timeout anyway): a workgroup that holds many words -- a small grid under a
// workgroup budget -- gives up after one spin limit, not one per word.  The
// kernel exits normally.
#include "device_common.h"
#include "kernels.h"
#include "launch.h"

namespace simar {

template <int DT, int OP>
__global__ void __launch_bounds__(kBlock) k_ll(LLArgs a) {
  typedef typename Ty<DT>::A A;
  typedef Op<DT, OP> O;
  constexpr int E = Ty<DT>::E;
  constexpr int EPW = 4 / E;  // elements per 32-bit word
  const int p = a.p;
  const unsigned long long flag = (unsigned long long)a.epoch << 32;
  const int64_t nwords = a.nwords;

  // ---- produce ----------------------------------------------------------------
  // The p words of one index are loaded together, then packed and stored:
  // one load round trip per word index, not one per rank.
  for (int64_t t = blockIdx.x; t < a.ntiles; t += gridDim.x) {
    const int64_t kend = min(nwords, (t + 1) * a.tile_words);
    for (int64_t k = t * a.tile_words + threadIdx.x; k < kend; k += kBlock) {
      const bool whole = (EPW == 1 || (k + 1) * EPW <= a.n);  // else the odd 16-bit tail: a lone element
      uint32_t w[SIM_MAX_RANKS];
#pragma unroll
      for (int q = 0; q < SIM_MAX_RANKS; q++)
        if (q < p) w[q] = whole ? ((const uint32_t*)a.x[q])[k] : ((const uint16_t*)a.x[q])[k * EPW];
#pragma unroll
      for (int q = 0; q < SIM_MAX_RANKS; q++)
        if (q < p)
          __hip_atomic_store(a.ll + q * a.ll_stride + k, flag | w[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- consume ----------------------------------------------------------------
  // give-up flag of the workgroup: set (to 1 only) by any lane whose wait
  // expired, read by every lane before each word; a lane that reads it late
  // spends at most one more wait
  __shared__ int give_up;
  if (threadIdx.x == 0) give_up = 0;
  __syncthreads();
  for (int64_t t = blockIdx.x; t < a.ntiles; t += gridDim.x) {
    const int64_t tile = (t + a.shift) % a.ntiles;
    const int64_t kend = min(nwords, (tile + 1) * a.tile_words);
    for (int64_t k = tile * a.tile_words + threadIdx.x; k < kend; k += kBlock) {
      if (__hip_atomic_load(&give_up, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) break;
      // issue the p polls back to back (one memory round trip when every
      // packet is already there), then re-poll only the packets still missing
      unsigned long long pk[SIM_MAX_RANKS];
#pragma unroll
      for (int q = 0; q < SIM_MAX_RANKS; q++)
        if (q < p)
          pk[q] = __hip_atomic_load(a.ll + q * a.ll_stride + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bool ok = true;
      for (unsigned long long round = 0;; round++) {
        bool all = true;
#pragma unroll
        for (int q = 0; q < SIM_MAX_RANKS; q++)
          if (q < p && (unsigned)(pk[q] >> 32) != a.wait_epoch) all = false;
        if (all) break;
        if (round >= a.spin_limit) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int q = 0; q < SIM_MAX_RANKS; q++)
          if (q < p && (unsigned)(pk[q] >> 32) != a.wait_epoch)
            pk[q] = __hip_atomic_load(a.ll + q * a.ll_stride + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (!ok) {
        __hip_atomic_store(a.err, (int)SIM_ERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&give_up, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        break;
      }
      uint32_t d[SIM_MAX_RANKS];
#pragma unroll
      for (int q = 0; q < SIM_MAX_RANKS; q++) d[q] = (q < p) ? (uint32_t)pk[q] : 0u;
      uint32_t outw = 0;
#pragma unroll
      for (int e = 0; e < EPW; e++) {
        const int64_t i = k * EPW + e;
        if (i >= a.n) break;
        int j = 0;  // owner of element i: the last chunk whose start is <= i
#pragma unroll
        for (int c = 1; c < SIM_MAX_RANKS; c++)
          if (c < p && a.lo[c] <= i) j = c;
        A acc = 0;
#pragma unroll
        for (int q = 0; q < SIM_MAX_RANKS; q++)
          if (q < p && q == j) acc = O::pre(widen_bits<DT>(d[q] >> (16 * e)), a.inv_p);
#pragma unroll
        for (int q = 0; q < SIM_MAX_RANKS; q++)
          if (q < p && q != j) acc = O::comb(acc, O::pre(widen_bits<DT>(d[q] >> (16 * e)), a.inv_p));
        acc = O::post(acc, p);
        outw |= narrow_bits<DT>(acc) << (16 * e);
      }
      if (EPW == 1 || (k + 1) * EPW <= a.n) {
        for (int r = 0; r < p; r++) ((uint32_t*)a.y[r])[k] = outw;
      } else {
        for (int r = 0; r < p; r++) ((uint16_t*)a.y[r])[k * EPW] = (uint16_t)outw;
      }
    }
  }
}

template <int DT>
static hipError_t ll_by_op(int op, const LLArgs& a, int grid, hipStream_t s) {
  const dim3 g(grid), b(kBlock);
  switch (op) {
    case SIM_SUM: return launch<k_ll<DT, SIM_SUM>>(g, b, s, a);
    case SIM_PROD: return launch<k_ll<DT, SIM_PROD>>(g, b, s, a);
    case SIM_MIN: return launch<k_ll<DT, SIM_MIN>>(g, b, s, a);
    case SIM_MAX: return launch<k_ll<DT, SIM_MAX>>(g, b, s, a);
    case SIM_AVG: return launch<k_ll<DT, SIM_AVG>>(g, b, s, a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_ll(int dtype, int op, const LLArgs& a, int grid, hipStream_t s) {
  switch (dtype) {
    case SIM_INT32: return ll_by_op<SIM_INT32>(op, a, grid, s);
    case SIM_FP32: return ll_by_op<SIM_FP32>(op, a, grid, s);
    case SIM_FP16: return ll_by_op<SIM_FP16>(op, a, grid, s);
    case SIM_BF16: return ll_by_op<SIM_BF16>(op, a, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int DT, int OP>
static int occ() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void*)k_ll<DT, OP>, kBlock, 0) != hipSuccess)
    return 1;
  return nb > 0 ? nb : 1;
}

template <int DT>
static int occ_by_op(int op) {
  switch (op) {
    case SIM_SUM: return occ<DT, SIM_SUM>();
    case SIM_PROD: return occ<DT, SIM_PROD>();
    case SIM_MIN: return occ<DT, SIM_MIN>();
    case SIM_MAX: return occ<DT, SIM_MAX>();
    default: return occ<DT, SIM_AVG>();
  }
}

int ll_blocks_per_cu(int dtype, int op) {
  switch (dtype) {
    case SIM_INT32: return occ_by_op<SIM_INT32>(op);
    case SIM_FP32: return occ_by_op<SIM_FP32>(op);
    case SIM_FP16: return occ_by_op<SIM_FP16>(op);
    default: return occ_by_op<SIM_BF16>(op);
  }
}

}  // namespace simar
