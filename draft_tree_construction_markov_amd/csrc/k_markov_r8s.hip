// k_markov_r8s.hip -- fused Markov kernel instantiations for rank 128,
// L rows staged through LDS.
#include "k_markov_impl.h"

namespace pct {
hipError_t launch_mfma_r8s(const K1Plan& pl, const K1Args& a,
                          hipStream_t s) {
  return launch_mfma_rank<8, true>(pl, a, s);
}
}  // namespace pct
