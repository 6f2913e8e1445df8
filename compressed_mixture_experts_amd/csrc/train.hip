// Helpers of the layer's training path (ButterflyMoE, gist.science/nl/paper/2601.13563,
// §2 "Drie Fasen van de Methode": the experts' rotation angles and the latent
// substrate are trained end to end, the ternary substrate through a
// straight-through estimator).  They move rows between token order and the
// bucketed order of the routed rows, transpose the packed substrate code for
// the backward product, and apply GELU and a cast elementwise.  All of them
// are bandwidth-bound passes in 16-byte vectors.
#include "butterfly_impl.hpp"

namespace bmoe {

constexpr int TR_THREADS = 256;

static int grid_for(size_t items) {
  const size_t g = (items + TR_THREADS - 1) / TR_THREADS;
  return int(g < 16384 ? g : 16384);
}

// qpos[perm[q]] = q: the bucket position of every routed slot
__global__ __launch_bounds__(TR_THREADS) void invert_perm_kernel(const int32_t* __restrict__ perm,
                                                                 int32_t* __restrict__ qpos, int R) {
  for (int q = blockIdx.x * TR_THREADS + threadIdx.x; q < R; q += gridDim.x * TR_THREADS) qpos[perm[q]] = q;
}

hipError_t launch_invert_perm(const int32_t* perm, int32_t* qpos, int R, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(invert_perm_kernel, dim3(grid_for(size_t(R))), dim3(TR_THREADS), 0, s, perm, qpos, R);
  return hipGetLastError();
}

// out[q] = x[perm[q] / k]: token rows in bucket order (width d, 8 elements per chunk)
template <int ACT>
__global__ __launch_bounds__(TR_THREADS) void gather_rows_kernel(const void* x, const int32_t* __restrict__ perm,
                                                                 void* out, int R, int d, int k) {
  const size_t cpr = size_t(d) >> 3, chunks = size_t(R) * cpr;
  for (size_t c = size_t(blockIdx.x) * TR_THREADS + threadIdx.x; c < chunks; c += size_t(gridDim.x) * TR_THREADS) {
    const size_t q = c / cpr, col = (c - q * cpr) << 3;
    const size_t t = size_t(perm[q] / k);
    float v[8];
    load8<ACT>(x, t * d + col, v);
    store8<ACT>(out, q * d + col, v);
  }
}

hipError_t launch_gather_rows(const void* x, const int32_t* perm, void* out, int R, int d, int k, int act,
                              hipStream_t s) {
  if (R <= 0) return hipSuccess;
  const int g = grid_for(size_t(R) * (d >> 3));
  if (act == ACT_BF16)
    hipLaunchKernelGGL(gather_rows_kernel<ACT_BF16>, dim3(g), dim3(TR_THREADS), 0, s, x, perm, out, R, d, k);
  else
    hipLaunchKernelGGL(gather_rows_kernel<ACT_F32>, dim3(g), dim3(TR_THREADS), 0, s, x, perm, out, R, d, k);
  return hipGetLastError();
}

// out[t] = base[t] + sum_j term_j, j = 0 .. k-1 in slot order, fp32 sums:
// term_j = gate[t k + j] * rows[qpos[t k + j]] rounded to the activation
// dtype (the per-slot row of the forward) when gate is given, else the row
// itself; base optional (fp32).  out in the activation dtype or fp32.
template <int ACT, bool OUT_F32>
__global__ __launch_bounds__(TR_THREADS) void token_sum_kernel(const void* rows, const int32_t* __restrict__ qpos,
                                                               const float* __restrict__ gate,
                                                               const float* __restrict__ base, void* out, int T,
                                                               int d, int k) {
  const size_t cpr = size_t(d) >> 3, chunks = size_t(T) * cpr;
  for (size_t c = size_t(blockIdx.x) * TR_THREADS + threadIdx.x; c < chunks; c += size_t(gridDim.x) * TR_THREADS) {
    const size_t t = c / cpr, col = (c - t * cpr) << 3;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (base) load8<ACT_F32>(base, t * d + col, acc);
    for (int j = 0; j < k; ++j) {
      const size_t s = t * k + j;
      float v[8];
      load8<ACT>(rows, size_t(qpos[s]) * d + col, v);
      if (gate) {
        const float g = gate[s];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = g * v[i];
          v[i] = ACT == ACT_BF16 ? float(__bf16(p)) : p;
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if constexpr (OUT_F32) store8<ACT_F32>(out, t * d + col, acc);
    else store8<ACT>(out, t * d + col, acc);
  }
}

hipError_t launch_token_sum(const void* rows, const int32_t* qpos, const float* gate, const float* base, void* out,
                            bool out_f32, int T, int d, int k, int act, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int g = grid_for(size_t(T) * (d >> 3));
  if (act == ACT_BF16) {
    if (out_f32)
      hipLaunchKernelGGL((token_sum_kernel<ACT_BF16, true>), dim3(g), dim3(TR_THREADS), 0, s, rows, qpos, gate, base,
                         out, T, d, k);
    else
      hipLaunchKernelGGL((token_sum_kernel<ACT_BF16, false>), dim3(g), dim3(TR_THREADS), 0, s, rows, qpos, gate,
                         base, out, T, d, k);
  } else {
    hipLaunchKernelGGL((token_sum_kernel<ACT_F32, true>), dim3(g), dim3(TR_THREADS), 0, s, rows, qpos, gate, base,
                       out, T, d, k);
  }
  return hipGetLastError();
}

// W^T in the packed 2-bit format (include/bmoe.h: column 2j+h of a 16-column
// word has its nonzero bit at 16h+j and its sign bit at 16h+8+j) from W
// [rows][cols]: output word (i, w) holds W[16w + c][i], c < 16.
__global__ __launch_bounds__(TR_THREADS) void transpose_packed_kernel(const uint32_t* __restrict__ w,
                                                                      uint32_t* __restrict__ wt, int rows, int cols) {
  const int wpr_in = cols >> 4, wpr_out = rows >> 4;
  const size_t words = size_t(cols) * wpr_out;
  for (size_t o = size_t(blockIdx.x) * TR_THREADS + threadIdx.x; o < words; o += size_t(gridDim.x) * TR_THREADS) {
    const int i = int(o / wpr_out), wo = int(o % wpr_out);
    const int jin = (i & 15) >> 1, hin = i & 1;
    uint32_t r = 0u;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint32_t src = w[size_t(16 * wo + c) * wpr_in + (i >> 4)];
      const uint32_t nz = (src >> (16 * hin + jin)) & 1u, sg = (src >> (16 * hin + 8 + jin)) & 1u;
      const int j = c >> 1, h = c & 1;
      r |= (nz << (16 * h + j)) | (sg << (16 * h + 8 + j));
    }
    wt[o] = r;
  }
}

hipError_t launch_transpose_packed(const uint32_t* w, uint32_t* wt, int rows, int cols, hipStream_t s) {
  const size_t words = size_t(rows) * cols / 16;
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_packed_kernel, dim3(grid_for(words)), dim3(TR_THREADS), 0, s, w, wt, rows, cols);
  return hipGetLastError();
}

// a = GELU(h) = h (1 + erf(h / sqrt 2)) / 2, the forward kernels' gelu_erf,
// 8 elements per thread step
template <int ACT>
__global__ __launch_bounds__(TR_THREADS) void gelu_fwd_kernel(const void* h, void* a, size_t n) {
  for (size_t c = size_t(blockIdx.x) * TR_THREADS + threadIdx.x; c < (n >> 3); c += size_t(gridDim.x) * TR_THREADS) {
    float v[8];
    load8<ACT>(h, c << 3, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = gelu_erf(v[i]);
    store8<ACT>(a, c << 3, v);
  }
}

hipError_t launch_gelu_fwd(const void* h, void* a, size_t n, int act, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int g = grid_for(n >> 3);
  if (act == ACT_BF16) hipLaunchKernelGGL(gelu_fwd_kernel<ACT_BF16>, dim3(g), dim3(TR_THREADS), 0, s, h, a, n);
  else hipLaunchKernelGGL(gelu_fwd_kernel<ACT_F32>, dim3(g), dim3(TR_THREADS), 0, s, h, a, n);
  return hipGetLastError();
}

// bf16 copy (round to nearest even) of fp32 rows, for the bf16 substrate-gradient product
__global__ __launch_bounds__(TR_THREADS) void cast_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out,
                                                               size_t n) {
  for (size_t c = size_t(blockIdx.x) * TR_THREADS + threadIdx.x; c < (n >> 3); c += size_t(gridDim.x) * TR_THREADS) {
    float v[8];
    load8<ACT_F32>(in, c << 3, v);
    store8<ACT_BF16>(out, c << 3, v);
  }
}

hipError_t launch_cast_bf16(const float* in, uint16_t* out, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid_for(n >> 3)), dim3(TR_THREADS), 0, s, in, out, n);
  return hipGetLastError();
}

// zero fill (a kernel rather than hipMemsetAsync, so that a captured graph of
// the call replays it like every other step)
__global__ __launch_bounds__(TR_THREADS) void zero_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * TR_THREADS + threadIdx.x; i < n; i += size_t(gridDim.x) * TR_THREADS) p[i] = 0u;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n)), dim3(TR_THREADS), 0, s, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace bmoe
