// k_markov_r8d.hip -- fused Markov kernel instantiations for rank 128,
// L rows read directly.
#include "k_markov_impl.h"

namespace pct {
hipError_t launch_mfma_r8d(const K1Plan& pl, const K1Args& a,
                          hipStream_t s) {
  return launch_mfma_rank<8, false>(pl, a, s);
}
}  // namespace pct
