// k_fold_p16.hip -- the gather-fold kernel (fold_impl.h) for p = 16 as a
// compile-time constant and for a run-time p of 9 to 15.
#include "fold_impl.h"

SIMAR_FOLD_INSTANTIATE(16, 16)
SIMAR_FOLD_INSTANTIATE(0, 16)
