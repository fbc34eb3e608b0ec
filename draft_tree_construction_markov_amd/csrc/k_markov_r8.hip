// k_markov_r8.hip -- fused Markov kernel instantiations for rank 128.
#include "k_markov_impl.h"

namespace pct {
hipError_t launch_mfma_r8(const K1Plan& pl, const K1Args& a, hipStream_t s) {
  return launch_mfma_rank<8>(pl, a, s);
}
}  // namespace pct
