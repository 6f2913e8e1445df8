// Shared ternary substrate product Z = alpha * U * W^T (ButterflyMoE,
// gist.science/zh/paper/2601.13563, technical summary §2.2: one ternary
// {-1, 0, +1} substrate shared by every expert; §2.1: the rotated input is
// multiplied by that substrate).  Because the substrate is shared, the rows
// of all experts form one dense contraction: M = routed rows, N = d_out,
// K = d_in.
//
// bf16 path: the 2-bit substrate tile is unpacked once per workgroup into exact
// bf16 +-1/0 in LDS and contracted on MFMA (v_mfma_f32_16x16x32_bf16, fp32
// accumulation).  The MFMA "A" operand is the substrate (rows n) and "B" the
// activations (columns m), so each lane ends with four consecutive output
// columns of one row and stores them as one 8-byte write.
// fp32 path: a plain fp32 FMA loop (small layers and tests).
#include "common.hpp"

namespace bmoe {

constexpr int GM_THREADS = 256;
constexpr int GT_N = 128;     // substrate rows per workgroup tile
constexpr int GT_M = 128;     // activation rows per workgroup tile
constexpr int GBK = 64;       // K per stage
constexpr int GLDK = GBK + 8; // padded LDS row (bf16 elements): conflict-free fragment reads

// Blocks are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of logical tiles so tiles sharing an activation row-block
// share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

__global__ __launch_bounds__(GM_THREADS) void gemm_bf16_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* sW = smem;                       // [2][GT_N][GLDK]
  uint16_t* sU = smem + 2 * GT_N * GLDK;     // [2][GT_M][GLDK]

  const int ntn = (a.N + GT_N - 1) / GT_N;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tn = logical % ntn, tm = logical / ntn;
  const int n0 = tn * GT_N, m0 = tm * GT_M;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int K = a.K, KW = a.K >> 4;
  const uint16_t* A = reinterpret_cast<const uint16_t*>(a.a);

  uint4 ureg[4];
  uint32_t wreg[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + GM_THREADS * i;
      const int row = c >> 3, ch = c & 7;
      const int m = m0 + row;
      ureg[i] = (m < a.M) ? *reinterpret_cast<const uint4*>(A + size_t(m) * K + k0 + 8 * ch)
                          : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int w = tid + GM_THREADS * i;
      const int row = w >> 2, kw = w & 3;
      const int n = n0 + row;
      wreg[i] = (n < a.N) ? a.w[size_t(n) * KW + (k0 >> 4) + kw] : 0u;
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* su = sU + buf * GT_M * GLDK;
    uint16_t* sw = sW + buf * GT_N * GLDK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + GM_THREADS * i;
      const int row = c >> 3, ch = c & 7;
      *reinterpret_cast<uint4*>(su + row * GLDK + 8 * ch) = ureg[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int w = tid + GM_THREADS * i;
      const int row = w >> 2, kw = w & 3;
      const uint32_t P = wreg[i];
      uint4 lo, hi;
      lo.x = ternary_pair_bf16(P, 0); lo.y = ternary_pair_bf16(P, 1);
      lo.z = ternary_pair_bf16(P, 2); lo.w = ternary_pair_bf16(P, 3);
      hi.x = ternary_pair_bf16(P, 4); hi.y = ternary_pair_bf16(P, 5);
      hi.z = ternary_pair_bf16(P, 6); hi.w = ternary_pair_bf16(P, 7);
      uint4* dst = reinterpret_cast<uint4*>(sw + row * GLDK + 16 * kw);
      dst[0] = lo;
      dst[1] = hi;
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  const int nk = K / GBK;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * GBK);
    const uint16_t* sw = sW + buf * GT_N * GLDK;
    const uint16_t* su = sU + buf * GT_M * GLDK;
#pragma unroll
    for (int kk = 0; kk < GBK; kk += 32) {
      bf16x8_t wf[4], uf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        wf[i] = *reinterpret_cast<const bf16x8_t*>(sw + (wn * 64 + 16 * i + (lane & 15)) * GLDK + kk + 8 * (lane >> 4));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        uf[j] = *reinterpret_cast<const bf16x8_t*>(su + (wm * 64 + 16 * j + (lane & 15)) * GLDK + kk + 8 * (lane >> 4));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i], uf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  uint16_t* Z = reinterpret_cast<uint16_t*>(a.z);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + wn * 64 + 16 * i + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 64 + 16 * j + (lane & 15);
      if (m < a.M && n < a.N) {
        uint2 o;
        o.x = pack_bf16x2(a.alpha * acc[i][j][0], a.alpha * acc[i][j][1]);
        o.y = pack_bf16x2(a.alpha * acc[i][j][2], a.alpha * acc[i][j][3]);
        *reinterpret_cast<uint2*>(Z + size_t(m) * a.N + n) = o;
      }
    }
  }
}

// fp32: one output per thread, sequential FMA over K.
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  const size_t id = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (id >= size_t(a.M) * a.N) return;
  const int m = int(id / a.N), n = int(id - size_t(m) * a.N);
  const float* A = reinterpret_cast<const float*>(a.a) + size_t(m) * a.K;
  const uint32_t* W = a.w + size_t(n) * (a.K >> 4);
  float s = 0.f;
  for (int kw = 0; kw < (a.K >> 4); ++kw) {
    const uint32_t P = W[kw];
#pragma unroll
    for (int c = 0; c < 16; ++c) s = fmaf(A[16 * kw + c], ternary_value(P, c), s);
  }
  reinterpret_cast<float*>(a.z)[size_t(m) * a.N + n] = a.alpha * s;
}

hipError_t launch_gemm(const GemmArgs& a, int act, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (act == ACT_BF16) {
    const int ntn = (a.N + GT_N - 1) / GT_N, ntm = (a.M + GT_M - 1) / GT_M;
    const size_t lds = size_t(2) * (GT_N + GT_M) * GLDK * sizeof(uint16_t);
    static int attr_done[64] = {0};
    int dev = 0;
    hipGetDevice(&dev);
    if (dev < 64 && !attr_done[dev]) {
      hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
      if (e != hipSuccess) return e;
      attr_done[dev] = 1;
    }
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3(ntn * ntm), dim3(GM_THREADS), lds, s, a);
  } else {
    const size_t total = size_t(a.M) * a.N;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// y[t] = sum_j Y[t*k + j] in slot order (fp32 sum, one rounding).
template <int ACT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const size_t chunks = size_t(a.T) * (a.d >> 3);
  for (size_t c = size_t(blockIdx.x) * 256 + threadIdx.x; c < chunks; c += size_t(gridDim.x) * 256) {
    const size_t t = c / (a.d >> 3);
    const size_t col = (c - t * (a.d >> 3)) << 3;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < a.k; ++j) {
      float v[8];
      load8<ACT>(a.yp, (t * a.k + j) * a.d + col, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += v[q];
    }
    store8<ACT>(a.y, t * a.d + col, acc);
  }
}

hipError_t launch_combine(const CombineArgs& a, int act, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const size_t chunks = size_t(a.T) * (a.d >> 3);
  size_t grid = (chunks + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (act == ACT_BF16)
    hipLaunchKernelGGL(combine_kernel<ACT_BF16>, dim3(unsigned(grid)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<ACT_F32>, dim3(unsigned(grid)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bmoe
