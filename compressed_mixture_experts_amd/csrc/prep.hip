// Weight preparation for the expert kernels: re-encodings of the
// shared ternary substrate and of each expert's rotations that depend on the
// weights only (ButterflyMoE, gist.science/zh/paper/2601.13563, technical
// summary §2.1-§2.2: the substrate is ternary, every expert rotates with its
// own Givens angles).  Done once per weight set (bmoe_prepare) or per call.
//
// Grid: PR_FS workgroups per expert (matrix-core square layers), else enough
// workgroups to cover the words.  Every workgroup unpacks a grid-stride share
// of the 2-bit words of one or two substrates; for the matrix-core kernel each builds a share of
// its expert's rotation block factors (mfma_factors.hpp).
#include "mfma_factors.hpp"

namespace bmoe {

constexpr int PR_THREADS = 512;
constexpr int PR_FS = 4;  // workgroups per expert

template <int LF>
__global__ __launch_bounds__(PR_THREADS) void prep_kernel(PrepArgs a) {
  constexpr int CS = LF > 0 ? LF * (1 << (LF - 1)) : 1;
  __shared__ float2 s_cs[2][CS];
  const int tid = threadIdx.x;
  // substrate: 16 weights per word, column 2j+h of the word's 16: nonzero bit
  // 16h+j, sign bit 16h+8+j.  Bytes: +1 -> 0x3F, -1 -> 0xBF, 0 -> 0 (bf16 high
  // byte of +-0.5); paired 2-bit code (pair2_to_fp4): column c < 8 at bits
  // 4c+1 (nonzero) and 4c+3 (sign), column 8+c at bits 4c and 4c+2
  const int nw = a.w_words + a.w_words1;
  for (int i = blockIdx.x * PR_THREADS + tid; i < nw; i += gridDim.x * PR_THREADS) {
    const bool s1 = i >= a.w_words;
    const int w = s1 ? i - a.w_words : i;
    const bool fp4 = s1 || a.w_fp4;
    const uint32_t P = s1 ? a.w_packed1[w] : a.w_packed[w];
    unsigned char* out = s1 ? a.w_out1 : a.w_out;
    if (fp4) {
      uint32_t o = 0u;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int j = c >> 1, h = c & 1;
        const uint32_t nz = (P >> (16 * h + j)) & 1u, sg = nz & (P >> (16 * h + 8 + j));
        const int at = c < 8 ? 4 * c + 1 : 4 * (c - 8);
        o |= (nz << at) | (sg << (at + 2));
      }
      reinterpret_cast<uint32_t*>(out)[w] = o;
    } else {
      uint32_t code[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int j = c >> 1, h = c & 1;
        const uint32_t nz = (P >> (16 * h + j)) & 1u, sg = (P >> (16 * h + 8 + j)) & 1u;
        code[c] = nz * (0x3Fu | (sg << 7));
      }
      uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int c = 0; c < 16; ++c) o[c >> 2] |= code[c] << (8 * (c & 3));
      reinterpret_cast<uint4*>(out)[w] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  if constexpr (LF > 0) {
    const int e = blockIdx.x / PR_FS, z = blockIdx.x % PR_FS;
    const size_t angs = size_t(LF) * (1 << (LF - 1));
    mf_fill_cs<LF>(s_cs[0], a.theta + size_t(e) * angs, tid, PR_THREADS);
    mf_fill_cs<LF>(s_cs[1], a.phi + size_t(e) * angs, tid, PR_THREADS);
    __syncthreads();
    unsigned char* fe = a.fac + size_t(e) * MfCfg<LF>::per_expert;
    for (int job = z * PR_THREADS + tid; job < mf_factor_jobs<LF>(); job += PR_FS * PR_THREADS)
      mf_factor_job<LF>(job, s_cs[0], s_cs[1], fe);
  }
}

hipError_t launch_prep(const PrepArgs& a, hipStream_t s) {
  const int64_t nw = int64_t(a.w_words) + a.w_words1;
  const int grid = a.fac_log2n ? a.n_experts * PR_FS : int((nw + PR_THREADS - 1) / PR_THREADS < 8192 ? (nw + PR_THREADS - 1) / PR_THREADS : 8192);
  if (grid <= 0) return hipSuccess;
  switch (a.fac_log2n) {
    case 8: hipLaunchKernelGGL(prep_kernel<8>, dim3(grid), dim3(PR_THREADS), 0, s, a); break;
    case 9: hipLaunchKernelGGL(prep_kernel<9>, dim3(grid), dim3(PR_THREADS), 0, s, a); break;
    default: hipLaunchKernelGGL(prep_kernel<0>, dim3(grid), dim3(PR_THREADS), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace bmoe
