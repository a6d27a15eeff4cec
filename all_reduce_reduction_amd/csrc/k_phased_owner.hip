// k_phased_owner.hip -- the phased fold (phased_impl.h) with only the owner's
// output written: all-pairs step 1 and the direct reduce-scatter for large
// messages.
#include "phased_impl.h"

namespace simar {

template hipError_t phased_launch<false, false>(int, int, int, const PhasedArgs&, hipStream_t);
template int phased_occupancy<false, false>(int, int, int);

}  // namespace simar
