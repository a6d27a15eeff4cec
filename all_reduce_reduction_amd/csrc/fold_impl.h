// fold_impl.h -- the gather-fold kernel template and its launchers, included
// by the translation units that instantiate it (k_fold*.hip).
//
// One-shot ("MSCCL++ ...", section "The Collective Algorithm Library":
// in 1PA every rank reads every rank's data and reduces it in one phase;
// its multi-peer reduction reads all peers at the same time instead of one
// by one): each lane issues the 16-byte loads of all p ranks for its
// vector back to back, folds them in VGPRs in the all-pairs order (owner of
// the chunk first, then the other ranks ascending -- the order of the
// scratch slots in the all-pairs program of "MSCCL, in depth ...", section
// "Writing an algorithm in MSCCLang"), and stores the one result to every
// rank's output from the same registers (T-CCL, section III-C1: load once,
// store to several peers).  Each input byte is read once and each output
// byte written once: 2 p S bytes, the floor for p ranks in one HBM.
//
// All-pairs step 1 / direct reduce-scatter is the same fold with only the
// owner's output written (owner-only mode).
//
// Layout: a 1-D grid of tiles * p workgroups; workgroup b folds chunk
// j = b mod p, tile b / p.  The chunk is uniform over a workgroup, so the
// fold order is too and the operand pointers are chosen once, in scalar
// registers.  Neighbouring workgroups -- the ones in flight together --
// work on different chunks: at any moment the 2p streams of the chunk being
// folded are spread over p regions of every buffer instead of one, which
// measured ~13% faster on MI355X than running the chunks one after another
// (the same offset in p buffers tends to land on the same HBM channels).
// A workgroup walks its chunk in spans of kBlock * U vectors; a ragged
// chunk edge (a vector that would straddle two chunks, or a misaligned
// operand) is done element by element so every element keeps its own
// chunk's order.
//
// The one-shot and all-pairs step 1 also run from a small argument block
// whose rank pointers sit in device memory (FoldTabArgs; it computes the
// standard chunk bounds and writes outputs unshifted, so the direct
// reduce-scatter keeps the full form); both argument forms are read through
// the accessors below, and every pointer is loaded once, before the first
// store.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "fold.h"
#include "launch.h"

namespace simar {

namespace {
// rank pointers, chunk bounds, vector eligibility and output shift of chunk j
__device__ __forceinline__ const void* x_of(const FoldArgs& a, int q) { return a.x[q]; }
__device__ __forceinline__ void* y_of(const FoldArgs& a, int r) { return a.y[r]; }
__device__ __forceinline__ int64_t lo_of(const FoldArgs& a, int j, int) { return a.lo[j]; }
__device__ __forceinline__ bool vec_of(const FoldArgs& a, int j) { return (a.vec_ok >> j) & 1u; }
__device__ __forceinline__ int64_t shift_of(const FoldArgs& a, int j) { return a.out_shift[j]; }

__device__ __forceinline__ const void* x_of(const FoldTabArgs& a, int q) { return a.set->x[q]; }
__device__ __forceinline__ void* y_of(const FoldTabArgs& a, int r) { return a.set->y[r]; }
// floor(j n / p): n < 2^46 and j <= 16, so j n cannot overflow
__device__ __forceinline__ int64_t lo_of(const FoldTabArgs& a, int j, int p) { return (int64_t)j * a.n / p; }
__device__ __forceinline__ bool vec_of(const FoldTabArgs&, int) { return true; }  // every pointer is 16-byte aligned
__device__ __forceinline__ int64_t shift_of(const FoldTabArgs&, int) { return 0; }
}  // namespace

template <int DT, int OP, int P, int PMAX, bool ALL_OUT, int U, class Args>
__global__ void __launch_bounds__(kBlock) k_fold(Args a) {
  typedef typename Ty<DT>::A A;
  typedef Op<DT, OP> O;
  constexpr int V = epv<DT>();
  constexpr int E = Ty<DT>::E;
  constexpr int MAXP = P ? P : PMAX;
  const int p = P ? P : a.p;
  const int j = (int)(blockIdx.x % (unsigned)p);
  const int64_t tile = blockIdx.x / (unsigned)p;
  const int64_t lo = lo_of(a, j, p), hi = lo_of(a, j + 1, p);
  const float inv_p = a.inv_p;

  // operand k of the fold: rank j for k == 0, then the ranks != j ascending
  const void* xp[MAXP];
#pragma unroll
  for (int k = 0; k < MAXP; k++) {
    const int q = (k == 0) ? j : (k <= j ? k - 1 : k);
    xp[k] = (k < p) ? x_of(a, q) : nullptr;
  }
  // outputs: every rank's (one-shot) or the owner's
  void* yp[ALL_OUT ? MAXP : 1];
#pragma unroll
  for (int r = 0; r < (ALL_OUT ? MAXP : 1); r++) yp[r] = (r < p) ? y_of(a, ALL_OUT ? r : j) : nullptr;

  const bool vec = vec_of(a, j);
  int64_t head = vec ? (int64_t)((V - (lo % V)) % V) : (hi - lo);
  if (head > hi - lo) head = hi - lo;
  const int64_t vbeg = lo + head;
  const int64_t nvec = (hi - vbeg) / V;
  const int64_t tail_beg = vbeg + nvec * V;
  const int64_t nscalar = head + (hi - tail_beg);
  const int tid = threadIdx.x;
  const int64_t span = (int64_t)kBlock * U;
  const int64_t stride = (int64_t)a.tiles * span;
  const int64_t oshift = ALL_OUT ? 0 : shift_of(a, j);
  void* const yj = yp[0];

  // One span: U vectors per lane, each folded from p operands and stored to
  // the output(s).  GUARD: the span may run past nvec (the last one only).
  auto span_body = [&](int64_t base, auto guard) {
    constexpr bool GUARD = decltype(guard)::value;
    // this span's first byte in every buffer (uniform) and the lane's 16-byte
    // slot within it (one 32-bit VGPR for all 2p accesses)
    const int64_t sbyte = (vbeg + base * V) * E;
    const uint32_t lane = lane_offset((uint32_t)tid * 16u);
    u32x4 L[U][MAXP];
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (!GUARD || base + u * kBlock + tid < nvec) {
#pragma unroll
        for (int k = 0; k < MAXP; k++)
          if (k < p) L[u][k] = ld16u(xp[k], sbyte + (int64_t)u * kBlock * 16, lane);
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (!GUARD || base + u * kBlock + tid < nvec) {
        A acc[V], t[V];
        unpack<DT>(L[u][0], acc);
#pragma unroll
        for (int e = 0; e < V; e++) acc[e] = O::pre(acc[e], inv_p);
#pragma unroll
        for (int k = 1; k < MAXP; k++) {
          if (k < p) {
            unpack<DT>(L[u][k], t);
#pragma unroll
            for (int e = 0; e < V; e++) acc[e] = O::comb(acc[e], O::pre(t[e], inv_p));
          }
        }
#pragma unroll
        for (int e = 0; e < V; e++) acc[e] = O::post(acc[e], p);
        const u32x4 out = pack<DT>(acc);
        const int64_t ub = sbyte + (int64_t)u * kBlock * 16;
        if constexpr (ALL_OUT) {
#pragma unroll
          for (int r = 0; r < MAXP; r++)
            if (r < p) st16u(yp[r], ub, lane, out);
        } else {
          st16u(yj, ub - oshift * E, lane, out);
        }
      }
    }
  };
  // Whole spans run unguarded: a span's loads, fold and stores are then one
  // straight-line block, and the compiler's wait counting needs no
  // conservative wait (for stores still in flight) before the next span's
  // loads, which an exec-masked load block followed by a separately masked
  // fold block had forced.  The one partial span, if any, is guarded.
  int64_t base = tile * span;
  for (; base + span <= nvec; base += stride) span_body(base, std::false_type());
  if (base < nvec) span_body(base, std::true_type());

  // ragged edges, element by element
  for (int64_t s = tile * kBlock + tid; s < nscalar; s += (int64_t)a.tiles * kBlock) {
    const int64_t i = (s < head) ? lo + s : tail_beg + (s - head);
    A acc = O::pre(load_elem<DT>(xp[0], i), inv_p);
#pragma unroll
    for (int k = 1; k < MAXP; k++)
      if (k < p) acc = O::comb(acc, O::pre(load_elem<DT>(xp[k], i), inv_p));
    acc = O::post(acc, p);
    if constexpr (ALL_OUT) {
#pragma unroll
      for (int r = 0; r < MAXP; r++)
        if (r < p) store_elem<DT>(yp[r], i, acc);
    } else {
      store_elem<DT>(yj, i - oshift, acc);
    }
  }
}

// The launchers of one (P, PMAX) pair, for every dtype, op and output mode;
// U = 2 and U = 4 only where the rank count is a compile-time constant of 8
// or less (with p up to 16 unknown, a second vector per lane would hold
// 2 * 16 * 4 more VGPRs).  U = 4 keeps 4 p loads in flight per lane (128
// VGPRs at p = 8): it is for launches with fewer workgroups than CUs (a
// workgroup budget), where each workgroup has a CU to itself and the fold
// runs at what one workgroup keeps in flight.
template <int DT, int OP, int P, int PMAX, bool ALL_OUT, int U, class Args>
static hipError_t go(const Args& a, hipStream_t s) {
  return launch<k_fold<DT, OP, P, PMAX, ALL_OUT, U, Args>>(dim3((unsigned)a.tiles * (unsigned)a.p), dim3(kBlock), s,
                                                           a);
}

template <int DT, int OP, int P, int PMAX, class Args>
static hipError_t by_shape(bool all_out, int unroll, const Args& a, hipStream_t s) {
  if constexpr (P > 0 && P <= 8) {
    if (unroll == 2)
      return all_out ? go<DT, OP, P, PMAX, true, 2>(a, s) : go<DT, OP, P, PMAX, false, 2>(a, s);
    if (unroll == 4)
      return all_out ? go<DT, OP, P, PMAX, true, 4>(a, s) : go<DT, OP, P, PMAX, false, 4>(a, s);
  }
  return all_out ? go<DT, OP, P, PMAX, true, 1>(a, s) : go<DT, OP, P, PMAX, false, 1>(a, s);
}

template <int DT, int P, int PMAX, class Args>
static hipError_t by_op(int op, bool all_out, int unroll, const Args& a, hipStream_t s) {
  switch (op) {
    case SIM_SUM: return by_shape<DT, SIM_SUM, P, PMAX>(all_out, unroll, a, s);
    case SIM_PROD: return by_shape<DT, SIM_PROD, P, PMAX>(all_out, unroll, a, s);
    case SIM_MIN: return by_shape<DT, SIM_MIN, P, PMAX>(all_out, unroll, a, s);
    case SIM_MAX: return by_shape<DT, SIM_MAX, P, PMAX>(all_out, unroll, a, s);
    case SIM_AVG: return by_shape<DT, SIM_AVG, P, PMAX>(all_out, unroll, a, s);
  }
  return hipErrorInvalidValue;
}

template <int P, int PMAX, class Args>
hipError_t fold_dispatch(int dtype, int op, bool all_out, int unroll, const Args& a, hipStream_t s) {
  switch (dtype) {
    case SIM_INT32: return by_op<SIM_INT32, P, PMAX>(op, all_out, unroll, a, s);
    case SIM_FP32: return by_op<SIM_FP32, P, PMAX>(op, all_out, unroll, a, s);
    case SIM_FP16: return by_op<SIM_FP16, P, PMAX>(op, all_out, unroll, a, s);
    case SIM_BF16: return by_op<SIM_BF16, P, PMAX>(op, all_out, unroll, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace simar

// one (P, PMAX) pair's launchers, for both argument forms
#define SIMAR_FOLD_INSTANTIATE(P, PMAX)                                                                    \
  template hipError_t simar::fold_dispatch<P, PMAX, simar::FoldArgs>(int, int, bool, int,                  \
                                                                     const simar::FoldArgs&, hipStream_t); \
  template hipError_t simar::fold_dispatch<P, PMAX, simar::FoldTabArgs>(int, int, bool, int,               \
                                                                        const simar::FoldTabArgs&, hipStream_t);
