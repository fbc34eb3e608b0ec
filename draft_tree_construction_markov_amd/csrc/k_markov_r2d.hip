// k_markov_r2d.hip -- fused Markov kernel instantiations for rank 32,
// L rows read directly.
#include "k_markov_impl.h"

namespace pct {
hipError_t launch_mfma_r2d(const K1Plan& pl, const K1Args& a,
                          hipStream_t s) {
  return launch_mfma_rank<2, false>(pl, a, s);
}
}  // namespace pct
