// k_markov_r2.hip -- fused Markov kernel instantiations for rank 32.
#include "k_markov_impl.h"

namespace pct {
hipError_t launch_mfma_r2(const K1Plan& pl, const K1Args& a, hipStream_t s) {
  return launch_mfma_rank<2>(pl, a, s);
}
}  // namespace pct
