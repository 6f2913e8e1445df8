// Derivative of the FFN experts' activation (ButterflyViT,
// gist.science/pt/paper/2603.06746, §2: a GELU between the FFN's two
// rotated substrate products), with the same erf as the forward passes:
//     dh = da * GELU'(h),   GELU'(h) = Phi(h) + h phi(h)
//        = (1 + erf(h / sqrt 2)) / 2 + h exp(-h^2 / 2) / sqrt(2 pi).
// Elementwise over 8-element groups (16-byte vectors for bf16), grid-stride.
#include "butterfly_impl.hpp"

namespace bmoe {

template <int A>
__global__ __launch_bounds__(256) void gelu_bwd_kernel(const void* h, const void* da, void* dh, size_t groups) {
  for (size_t q = size_t(blockIdx.x) * 256 + threadIdx.x; q < groups; q += size_t(gridDim.x) * 256) {
    float hv[8], dv[8], out[8];
    load8<A>(h, 8 * q, hv);
    load8<A>(da, 8 * q, dv);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = hv[j];
      // exp(-x^2 / 2) = exp2(-x^2 / (2 ln 2))
      const float g = 0.5f * (1.0f + erf_as(x * 0.70710678118654752f)) +
                      x * 0.39894228040143268f * __builtin_amdgcn_exp2f(-0.72134752044448170f * x * x);
      out[j] = dv[j] * g;
    }
    store8<A>(dh, 8 * q, out);
  }
}

hipError_t launch_gelu_bwd(const void* h, const void* da, void* dh, size_t n, int act, hipStream_t s) {
  const size_t groups = n / 8;
  if (groups == 0) return hipSuccess;
  size_t blocks = (groups + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (act == ACT_BF16) hipLaunchKernelGGL(gelu_bwd_kernel<ACT_BF16>, dim3(unsigned(blocks)), dim3(256), 0, s, h, da, dh, groups);
  else hipLaunchKernelGGL(gelu_bwd_kernel<ACT_F32>, dim3(unsigned(blocks)), dim3(256), 0, s, h, da, dh, groups);
  return hipGetLastError();
}

}  // namespace bmoe
