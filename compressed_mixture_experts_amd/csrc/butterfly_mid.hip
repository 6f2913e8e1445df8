// Butterfly kernel instantiations: MID mode (rows bucketed by expert).
#include "butterfly_impl.hpp"

namespace bmoe {

hipError_t launch_bfly_mid(const BflyArgs& a, int act, int log2n, hipStream_t s) {
  if (act == ACT_BF16) return launch_bfly_width<BFLY_MID, ACT_BF16, false, 6>(a, log2n, s);
  return launch_bfly_width<BFLY_MID, ACT_F32, false, 6>(a, log2n, s);
}

}  // namespace bmoe
