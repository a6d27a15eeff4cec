// k_sched.hip -- one fold step of the tree, recursive-exchange and 2PH
// schedules (gfx950).
//
// Each transfer folds one chunk over an ordered list of ranks' current
// values: a tree parent adds its children's subtree totals to its own
// element ("Inside NCCL all-reduce", section "The double binary tree": a
// parent reduces its children's incoming data against its own contribution
// in registers as it streams through); a recursive-exchange group folds its
// members ("Demystifying NVSHMEM", Fig. 7); a 2PH rank folds its node's
// elements or the node partials across nodes ("MSCCL++ ...", section "The
// Collective Algorithm Library", item 4).  The members of an exchange group
// all end with the same value, so the group is one transfer whose result is
// stored to every member from the same registers -- on one HBM the group's
// operands are read once instead of once per member.
//
// Operands are either inputs (widened and avg-scaled as they are read) or
// accumulator-typed partials left by an earlier step (fp32 for 16-bit
// types, so each element is rounded to 16 bits once, at the post-processed
// final write).  Up to four operands' 16-byte loads are issued together
// before they are folded, in order.
//
// Layout: 1-D grid of tiles * nx workgroups; workgroup b runs tile b / nx of
// transfer b mod nx (the transfers in flight together cover different
// chunks).  The transfer is uniform over the workgroup, so its operand list
// lives in scalar registers.  Ragged chunk edges run element by element.
#include "device_common.h"
#include "kernels.h"
#include "launch.h"

namespace simar {

template <int DT, int OP>
__device__ __forceinline__ void sched_operand(const SchedArgs& a, const SchedXfer& x, int k, int64_t i0,
                                              typename Ty<DT>::A* out) {
  typedef Op<DT, OP> O;
  constexpr int V = epv<DT>();
  constexpr int E = Ty<DT>::E;
  const int q = (int)((x.order >> (4 * k)) & 15u);
  if ((x.from_part >> k) & 1u) {
    load_part<DT>(a.part[q], i0, out);  // already scaled when it was first read
  } else {
    unpack<DT>(ld16(a.x[q], i0 * E), out);
#pragma unroll
    for (int e = 0; e < V; e++) out[e] = O::pre(out[e], a.inv_p);
  }
}

template <int DT, int OP>
__global__ void __launch_bounds__(kBlock) k_sched_fold(SchedArgs a) {
  typedef typename Ty<DT>::A A;
  typedef Op<DT, OP> O;
  constexpr int V = epv<DT>();
  const unsigned xi = blockIdx.x % (unsigned)a.nx;
  const int64_t tile = blockIdx.x / (unsigned)a.nx;
  const SchedXfer& x = a.xf[xi];
  const int64_t lo = x.lo, hi = x.hi;
  const int nsrc = x.nsrc;
  const int p = a.p;
  int64_t head = (int64_t)((V - (lo % V)) % V);
  if (head > hi - lo) head = hi - lo;
  const int64_t vbeg = lo + head;
  const int64_t nvec = (hi - vbeg) / V;
  const int64_t tail_beg = vbeg + nvec * V;
  const int64_t nscalar = head + (hi - tail_beg);
  const int tid = threadIdx.x;
  const int64_t stride = (int64_t)a.tiles * kBlock;

  for (int64_t v = tile * kBlock + tid; v < nvec; v += stride) {
    const int64_t i0 = vbeg + v * V;
    A acc[V];
    for (int k0 = 0; k0 < nsrc; k0 += 4) {
      A t[4][V];
#pragma unroll
      for (int b = 0; b < 4; b++)
        if (k0 + b < nsrc) sched_operand<DT, OP>(a, x, k0 + b, i0, t[b]);
#pragma unroll
      for (int b = 0; b < 4; b++) {
        if (k0 + b >= nsrc) break;
        if (k0 + b == 0) {
#pragma unroll
          for (int e = 0; e < V; e++) acc[e] = t[b][e];
        } else {
#pragma unroll
          for (int e = 0; e < V; e++) acc[e] = O::comb(acc[e], t[b][e]);
        }
      }
    }
    if (x.final_) {
#pragma unroll
      for (int e = 0; e < V; e++) acc[e] = O::post(acc[e], p);
      const u32x4 out = pack<DT>(acc);
      for (uint32_t m = x.dmask; m; m &= m - 1) st16(a.y[__builtin_ctz(m)], i0 * Ty<DT>::E, out);
    } else {
      for (uint32_t m = x.dmask; m; m &= m - 1) store_part<DT>(a.part[__builtin_ctz(m)], i0, acc);
    }
  }

  // ragged edges, element by element
  for (int64_t s = tile * kBlock + tid; s < nscalar; s += stride) {
    const int64_t i = (s < head) ? lo + s : tail_beg + (s - head);
    A acc = A(0);
    for (int k = 0; k < nsrc; k++) {
      const int q = (int)((x.order >> (4 * k)) & 15u);
      const A v = ((x.from_part >> k) & 1u) ? ((const A*)a.part[q])[part_pos<DT>(i)] : O::pre(load_elem<DT>(a.x[q], i), a.inv_p);
      acc = (k == 0) ? v : O::comb(acc, v);
    }
    if (x.final_) {
      acc = O::post(acc, p);
      for (uint32_t m = x.dmask; m; m &= m - 1) store_elem<DT>(a.y[__builtin_ctz(m)], i, acc);
    } else {
      for (uint32_t m = x.dmask; m; m &= m - 1) ((A*)a.part[__builtin_ctz(m)])[part_pos<DT>(i)] = acc;
    }
  }
}

template <int DT, int OP>
static hipError_t go(const SchedArgs& a, hipStream_t s) {
  return launch<k_sched_fold<DT, OP>>(dim3((unsigned)a.tiles * (unsigned)a.nx), dim3(kBlock), s, a);
}

template <int DT>
static hipError_t by_op(int op, const SchedArgs& a, hipStream_t s) {
  switch (op) {
    case SIM_SUM: return go<DT, SIM_SUM>(a, s);
    case SIM_PROD: return go<DT, SIM_PROD>(a, s);
    case SIM_MIN: return go<DT, SIM_MIN>(a, s);
    case SIM_MAX: return go<DT, SIM_MAX>(a, s);
    case SIM_AVG: return go<DT, SIM_AVG>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sched_fold(int dtype, int op, const SchedArgs& a, hipStream_t s) {
  if (a.nx < 1 || a.nx > kSchedMaxXfers || a.tiles < 1) return hipErrorInvalidValue;
  switch (dtype) {
    case SIM_INT32: return by_op<SIM_INT32>(op, a, s);
    case SIM_FP32: return by_op<SIM_FP32>(op, a, s);
    case SIM_FP16: return by_op<SIM_FP16>(op, a, s);
    case SIM_BF16: return by_op<SIM_BF16>(op, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace simar
