// k_ring_ll.hip -- the single-launch ring with LL packets (gfx950), the
// protocol the single-launch ring uses for small messages.
//
// The ring ("Inside NCCL all-reduce", section "The ring, exactly as the
// kernel runs it") with NCCL's LL protocol choice for small sizes (same
// page, section "Three ways to move a byte"; "MSCCL++ ...", section 4.2):
// every value that crosses from rank r to rank r + 1 travels as an 8-byte
// packet whose upper half is the call's epoch, written by one store, so
// the receiver polls the packet itself.  The FIFO path pays three memory
// round trips per step (its slot stores completing, then the counter
// becoming visible, then the slot loads); here a step costs the packet's
// trip alone, at twice the bytes of a 32-bit payload, which only pays where
// the ring is latency-bound.
//
// Workgroup (rank r, channel ch) walks its channel's slice of every chunk
// through the 2p - 1 steps of rank r:
//   k = 0            send the scaled own value of chunk r - 1;
//   k = 1 .. p - 2   receive a partial, fold the own value into it, send;
//   k = p - 1        receive the partial of chunk r (its owner), fold the
//                    own value, post-process: the finished value is written
//                    to Y[r] and sent on (storage bits);
//   k = p .. 2p - 2  receive a finished element, write it to Y[r], send it
//                    on (all but the last).
// The fold order is the ring's: chunk c starts at rank c + 1 and each rank
// folds its own value into the accumulator.  A thread handles the same
// slice offset of every chunk, so in place (Y[r] == X[r]) the read of
// X[r][i] always precedes the write of Y[r][i] in that thread's program.
// Send k goes to ll[(r+1) * ll_stride + k * maxchunk + offset in chunk]:
// each (send, element) has its own packet within a call, and the epoch
// differs from call to call, so no packet is reused or stale.  Polls are
// bounded by spin_limit; on expiry the workgroup records SIM_ERR_TIMEOUT
// and leaves (its successors then expire too), so a missing partner ends
// in an error, never a hang.
#include "device_common.h"
#include "kernels.h"
#include "launch.h"

namespace simar {

template <int DT, int OP>
__global__ void __launch_bounds__(kBlock) k_ring_ll(RingLLArgs a) {
  typedef typename Ty<DT>::A A;
  typedef Op<DT, OP> O;
  const int p = a.p;
  const int r = (int)(blockIdx.x / (unsigned)a.Cg);
  const int ch = (int)(blockIdx.x % (unsigned)a.Cg);
  if (ch >= a.C) return;                // grid padding
  if (a.withhold && r == 0) return;     // test hook: a partner that never shows up
  const int C = a.C;
  const int tid = threadIdx.x;
  const float inv_p = a.inv_p;
  const unsigned long long flag = (unsigned long long)a.epoch << 32;
  const unsigned wait_epoch = a.wait_epoch;
  const void* const xr = a.x[r];
  void* const yr = a.y[r];
  unsigned long long* const in_q = a.ll + (int64_t)r * a.ll_stride;                   // packets for me
  unsigned long long* const out_q = a.ll + (int64_t)((r + 1) % p) * a.ll_stride;    // for my successor

  for (int k = 0; k <= 2 * p - 2; k++) {
    int c = (k <= p - 1) ? r - 1 - k : r - (k - p + 1);
    c = ((c % p) + p) % p;
    const int64_t clo = a.lo[c], clen = a.lo[c + 1] - clo;
    const int64_t s_lo = clen * ch / C, s_hi = clen * (ch + 1) / C;  // offsets in the chunk
    for (int64_t o = s_lo + tid; o < s_hi; o += kBlock) {
      const int64_t i = clo + o;
      uint32_t in_bits = 0;
      if (k >= 1) {  // receive send k - 1 of my predecessor
        unsigned long long* const src = in_q + (int64_t)(k - 1) * a.maxchunk + o;
        unsigned long long pk = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (unsigned long long spins = 0; (unsigned)(pk >> 32) != wait_epoch; spins++) {
          if (spins >= a.spin_limit) {
            __hip_atomic_store(a.err, (int)SIM_ERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
          }
          __builtin_amdgcn_s_sleep(1);
          pk = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        in_bits = (uint32_t)pk;
      }
      uint32_t out_bits;
      if (k <= p - 1) {  // reduce-scatter half
        const A own = O::pre(load_elem<DT>(xr, i), inv_p);
        A v = (k == 0) ? own : O::comb(__builtin_bit_cast(A, in_bits), own);
        if (k == p - 1) {  // the owner: finished
          v = O::post(v, p);
          store_elem<DT>(yr, i, v);
          out_bits = narrow_bits<DT>(v);
        } else {
          out_bits = __builtin_bit_cast(uint32_t, v);
        }
      } else {  // all-gather half: a finished element in storage bits
        if constexpr (Ty<DT>::E == 4) ((uint32_t*)yr)[i] = in_bits;
        else ((uint16_t*)yr)[i] = (uint16_t)in_bits;
        out_bits = in_bits;
      }
      if (k <= 2 * p - 3)
        __hip_atomic_store(out_q + (int64_t)k * a.maxchunk + o, flag | out_bits, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int DT>
static hipError_t by_op(int op, const RingLLArgs& a, hipStream_t s) {
  const dim3 g((unsigned)(a.p * a.Cg)), b(kBlock);
  switch (op) {
    case SIM_SUM: return launch<k_ring_ll<DT, SIM_SUM>>(g, b, s, a);
    case SIM_PROD: return launch<k_ring_ll<DT, SIM_PROD>>(g, b, s, a);
    case SIM_MIN: return launch<k_ring_ll<DT, SIM_MIN>>(g, b, s, a);
    case SIM_MAX: return launch<k_ring_ll<DT, SIM_MAX>>(g, b, s, a);
    case SIM_AVG: return launch<k_ring_ll<DT, SIM_AVG>>(g, b, s, a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_ring_ll(int dtype, int op, const RingLLArgs& a, hipStream_t s) {
  if (a.p < 2 || a.p > SIM_MAX_RANKS || a.C < 1 || a.Cg < a.C || a.maxchunk < 0 ||
      (int64_t)(2 * a.p - 2) * a.maxchunk > a.ll_stride)
    return hipErrorInvalidValue;
  switch (dtype) {
    case SIM_INT32: return by_op<SIM_INT32>(op, a, s);
    case SIM_FP32: return by_op<SIM_FP32>(op, a, s);
    case SIM_FP16: return by_op<SIM_FP16>(op, a, s);
    case SIM_BF16: return by_op<SIM_BF16>(op, a, s);
  }
  return hipErrorInvalidValue;
}

// Workgroups of the (dtype, op) instantiation that fit on one CU at once.
template <int DT, int OP>
static int occ() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void*)k_ring_ll<DT, OP>, kBlock, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 1;
  }
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

int ring_ll_blocks_per_cu(int dtype, int op) {
  switch (dtype) {
    case SIM_INT32: return occ_by_op<SIM_INT32>(op);
    case SIM_FP32: return occ_by_op<SIM_FP32>(op);
    case SIM_FP16: return occ_by_op<SIM_FP16>(op);
    default: return occ_by_op<SIM_BF16>(op);
  }
}

}  // namespace simar
