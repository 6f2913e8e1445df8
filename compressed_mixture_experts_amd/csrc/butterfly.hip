// Butterfly launch dispatch by mode (kernels in butterfly_impl.hpp, one
// translation unit per mode).
#include "butterfly_impl.hpp"

namespace bmoe {

hipError_t launch_butterfly(const BflyArgs& a, int mode, int act, int log2n, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  switch (mode) {
    case BFLY_IN: return launch_bfly_in(a, act, log2n, s);
    case BFLY_MID: return launch_bfly_mid(a, act, log2n, s);
    default: return launch_bfly_out(a, act, log2n, s);
  }
}

}  // namespace bmoe
