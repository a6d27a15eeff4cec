// k_fold_p2p4.hip -- the gather-fold kernel (fold_impl.h) for p = 2 and
// p = 4 as compile-time constants.
#include "fold_impl.h"

SIMAR_FOLD_INSTANTIATE(2, 2)
SIMAR_FOLD_INSTANTIATE(4, 4)
