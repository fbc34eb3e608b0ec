// k_markov_r4.hip -- fused Markov kernel instantiations for rank 64.
#include "k_markov_impl.h"

namespace pct {
hipError_t launch_mfma_r4(const K1Plan& pl, const K1Args& a, hipStream_t s) {
  return launch_mfma_rank<4>(pl, a, s);
}
}  // namespace pct
