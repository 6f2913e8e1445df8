// Butterfly kernel instantiations: test hook (one angle set for all rows).
#include "butterfly_impl.hpp"

namespace bmoe {

hipError_t launch_bfly_dbg(const BflyArgs& a, int act, int log2n, hipStream_t s) {
  if (act == ACT_BF16)
    return a.transpose ? launch_bfly_width<BFLY_DBG, ACT_BF16, true, 3>(a, log2n, s)
                       : launch_bfly_width<BFLY_DBG, ACT_BF16, false, 3>(a, log2n, s);
  return a.transpose ? launch_bfly_width<BFLY_DBG, ACT_F32, true, 3>(a, log2n, s)
                     : launch_bfly_width<BFLY_DBG, ACT_F32, false, 3>(a, log2n, s);
}

}  // namespace bmoe
