// Butterfly kernel instantiations: ROT mode (bucket rows to bucket rows, each
// expert's B or B^T; the training forward keeps every rotation's output).
#include "butterfly_impl.hpp"

namespace bmoe {

hipError_t launch_bfly_rot(const BflyArgs& a, int act, int log2n, bool transpose, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (act == ACT_BF16)
    return transpose ? launch_bfly_width<BFLY_ROT, ACT_BF16, true, 6>(a, log2n, s)
                     : launch_bfly_width<BFLY_ROT, ACT_BF16, false, 6>(a, log2n, s);
  return transpose ? launch_bfly_width<BFLY_ROT, ACT_F32, true, 6>(a, log2n, s)
                   : launch_bfly_width<BFLY_ROT, ACT_F32, false, 6>(a, log2n, s);
}

}  // namespace bmoe
