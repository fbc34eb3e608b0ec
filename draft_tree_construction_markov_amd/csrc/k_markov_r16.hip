// k_markov_r16.hip -- fused Markov kernel instantiations for rank 256.
#include "k_markov_impl.h"

namespace pct {
hipError_t launch_mfma_r16(const K1Plan& pl, const K1Args& a, hipStream_t s) {
  return launch_mfma_rank<16>(pl, a, s);
}
}  // namespace pct
