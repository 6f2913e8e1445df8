// Backward of the gated combine y_t = sum_j g_{t,j} o_{t,j} (ButterflyMoE,
// gist.science/nl/paper/2601.13563, §2 "Gated Routing": the top-k experts'
// outputs weighted by the gating network; gist.science/zh/paper/2601.13563,
// technical summary §2.1).  For routed slot s = t*k + j held at bucket
// position q (the router's bucket order):
//     d_rows[q] = g_s * dy[t]              (gradient at the expert's output)
//     d_gate[s] = dy[t] . o[q]             (when the expert outputs are given)
// A wave per bucket position, 16-byte vectors (8 bf16 or 4 fp32 per lane),
// fp32 dot products.  Every slot is written once: the result does not depend
// on scheduling.
#include "common.hpp"

namespace bmoe {

struct CombBwdArgs {
  const void* dy;        // [T][d]
  const int32_t* slots;  // [R] flat slot of each bucket position
  const float* gate;     // [R] by flat slot
  const void* o;         // [R][d] by bucket position, or null
  void* d_rows;          // [R][d]
  float* d_gate;         // [R] by flat slot, or null
  int32_t R, k, d;
};

template <int A>
__global__ __launch_bounds__(256) void combine_bwd_kernel(CombBwdArgs a) {
  constexpr int V = A == ACT_BF16 ? 8 : 4;  // elements per 16-byte vector
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (q >= a.R) return;
  const int s = min(max(a.slots[q], 0), a.R - 1);
  const int t = s / a.k;
  const float g = a.gate[s];
  float dot = 0.f;
  for (int i = lane * V; i < a.d; i += 64 * V) {
    float v[8], w[8];
    const size_t di = size_t(t) * a.d + i, oi = size_t(q) * a.d + i;
    if constexpr (A == ACT_BF16) {
      load8<A>(a.dy, di, v);
      if (a.o) load8<A>(a.o, oi, w);
    } else {
      const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(a.dy) + di);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      if (a.o) {
        const float4 y = *reinterpret_cast<const float4*>(static_cast<const float*>(a.o) + oi);
        w[0] = y.x; w[1] = y.y; w[2] = y.z; w[3] = y.w;
      }
    }
    if (a.o) {
#pragma unroll
      for (int j = 0; j < V; ++j) dot = fmaf(v[j], w[j], dot);
    }
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] *= g;
    if constexpr (A == ACT_BF16) {
      store8<A>(a.d_rows, oi, v);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.d_rows) + oi) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
  if (a.o) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (lane == 0) a.d_gate[s] = dot;
  }
}

hipError_t launch_combine_bwd(const void* dy, const int32_t* slots, const float* gate, const void* o, void* d_rows,
                              float* d_gate, int R, int k, int d, int act, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  const CombBwdArgs a{dy, slots, gate, o, d_rows, d_gate, R, k, d};
  const dim3 grid((R + 3) / 4);
  if (act == ACT_BF16) hipLaunchKernelGGL(combine_bwd_kernel<ACT_BF16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(combine_bwd_kernel<ACT_F32>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bmoe
