// k_phased_whole.hip -- the phased one-shot (phased_impl.h) in the
// whole-buffer layout: the grid takes the whole buffer's blocks in turn
// (instantiated on its own so the build compiles it beside k_phased.hip).
#include "phased_impl.h"

namespace simar {

template hipError_t phased_launch<true, true>(int, int, int, const PhasedArgs&, hipStream_t);
template int phased_occupancy<true, true>(int, int, int);

}  // namespace simar
