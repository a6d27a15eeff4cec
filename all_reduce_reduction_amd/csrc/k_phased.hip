// k_phased.hip -- the phased fold (phased_impl.h) with every rank's output
// written: the one-shot all-reduce for large messages; and the launchers of
// both output modes and layouts (the owner-only mode is instantiated in
// k_phased_owner.hip, the one-shot's whole-buffer layout in
// k_phased_whole.hip).
#include "phased_impl.h"

namespace simar {

template hipError_t phased_launch<true, false>(int, int, int, const PhasedArgs&, hipStream_t);
template int phased_occupancy<true, false>(int, int, int);
extern template hipError_t phased_launch<false, false>(int, int, int, const PhasedArgs&, hipStream_t);
extern template int phased_occupancy<false, false>(int, int, int);
extern template hipError_t phased_launch<true, true>(int, int, int, const PhasedArgs&, hipStream_t);
extern template int phased_occupancy<true, true>(int, int, int);

// all_out with a.gblk > 0: the one-shot in the whole-buffer layout
hipError_t launch_fold_phased(int dtype, int op, int p, bool all_out, const PhasedArgs& a, hipStream_t s) {
  if (!all_out) return phased_launch<false, false>(dtype, op, p, a, s);
  return a.gblk > 0 ? phased_launch<true, true>(dtype, op, p, a, s) : phased_launch<true, false>(dtype, op, p, a, s);
}

int fold_phased_blocks_per_cu(int dtype, int op, int p, bool all_out, bool whole) {
  if (!all_out) return phased_occupancy<false, false>(dtype, op, p);
  return whole ? phased_occupancy<true, true>(dtype, op, p) : phased_occupancy<true, false>(dtype, op, p);
}

int fold_phased_vecs_per_lane(int p) {
  switch (p) {
    case 2: return PhasedShape<2>::K;
    case 4: return PhasedShape<4>::K;
    case 8: return PhasedShape<8>::K;
    case 16: return PhasedShape<16>::K;
  }
  return 0;
}

}  // namespace simar
