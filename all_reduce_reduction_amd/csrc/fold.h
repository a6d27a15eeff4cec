// fold.h -- the gather-fold launchers of one rank-count form.
//
// The fold kernel (fold_impl.h) is compiled once per rank-count form: P the
// rank count as a compile-time constant (2, 4, 8 or 16: every loop over the
// ranks unrolls into straight-line loads, folds and stores), or P = 0 with
// the count read at run time and bounded by PMAX (8 or 16).  A run-time
// count costs a scalar branch around every load, fold step and store and
// keeps the condition masks and 2 * PMAX pointers live across the loop.
// Each form is instantiated in its own translation unit (k_fold.hip,
// k_fold_p2p4.hip, k_fold_p16.hip), so the library's objects build in
// parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace simar {

// Enqueue the fold for one (P, PMAX) form.  unroll 2 (two 16-byte vectors
// per lane per pass) exists for P = 2, 4 and 8; any other value runs 1.
template <int P, int PMAX, class Args>
hipError_t fold_dispatch(int dtype, int op, bool all_out, int unroll, const Args& a, hipStream_t s);

#define SIMAR_FOLD_EXTERN(P, PMAX)                                                                       \
  extern template hipError_t fold_dispatch<P, PMAX, FoldArgs>(int, int, bool, int, const FoldArgs&,     \
                                                              hipStream_t);                             \
  extern template hipError_t fold_dispatch<P, PMAX, FoldTabArgs>(int, int, bool, int, const FoldTabArgs&, \
                                                                 hipStream_t);
SIMAR_FOLD_EXTERN(2, 2)
SIMAR_FOLD_EXTERN(4, 4)
SIMAR_FOLD_EXTERN(8, 8)
SIMAR_FOLD_EXTERN(16, 16)
SIMAR_FOLD_EXTERN(0, 8)
SIMAR_FOLD_EXTERN(0, 16)
#undef SIMAR_FOLD_EXTERN

}  // namespace simar
