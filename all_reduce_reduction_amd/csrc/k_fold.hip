// k_fold.hip -- the gather-fold kernel for gfx950 (the fused one-shot
// all-reduce, all-pairs step 1 and the direct reduce-scatter; the kernel
// itself is in fold_impl.h): the launchers by rank count, and the forms for
// p = 8 and for a run-time p of at most 8.
#include "fold_impl.h"

namespace simar {

// the rank-count form for p: a compile-time constant where one exists
template <class Args>
static hipError_t by_rank_count(int dtype, int op, int p, bool all_out, const Args& a, int unroll, hipStream_t s) {
  switch (p) {
    case 2: return fold_dispatch<2, 2>(dtype, op, all_out, unroll, a, s);
    case 4: return fold_dispatch<4, 4>(dtype, op, all_out, unroll, a, s);
    case 8: return fold_dispatch<8, 8>(dtype, op, all_out, unroll, a, s);
    case 16: return fold_dispatch<16, 16>(dtype, op, all_out, unroll, a, s);
  }
  if (p < 2 || p > SIM_MAX_RANKS) return hipErrorInvalidValue;
  return p < 8 ? fold_dispatch<0, 8>(dtype, op, all_out, 1, a, s) : fold_dispatch<0, 16>(dtype, op, all_out, 1, a, s);
}

hipError_t launch_fold(int dtype, int op, int p, bool all_out, const FoldArgs& a, int unroll, hipStream_t s) {
  return by_rank_count(dtype, op, p, all_out, a, unroll, s);
}

hipError_t launch_fold_tab(int dtype, int op, int p, bool all_out, const FoldTabArgs& a, int unroll, hipStream_t s) {
  return by_rank_count(dtype, op, p, all_out, a, unroll, s);
}

}  // namespace simar

SIMAR_FOLD_INSTANTIATE(8, 8)
SIMAR_FOLD_INSTANTIATE(0, 8)
