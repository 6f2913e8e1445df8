// Butterfly kernel instantiations: IN mode (rows bucketed by expert).
#include "butterfly_impl.hpp"

namespace bmoe {

hipError_t launch_bfly_in(const BflyArgs& a, int act, int log2n, hipStream_t s) {
  if (act == ACT_BF16) return launch_bfly_width<BFLY_IN, ACT_BF16, false, 6>(a, log2n, s);
  return launch_bfly_width<BFLY_IN, ACT_F32, false, 6>(a, log2n, s);
}

}  // namespace bmoe
