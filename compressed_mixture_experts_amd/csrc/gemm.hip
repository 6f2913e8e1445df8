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
#include <type_traits>

namespace bmoe {

constexpr int GM_THREADS = 256;
constexpr int GBK = 64;       // K per pipeline step
constexpr int GLDK = GBK + 8; // padded LDS row (bf16 elements): conflict-free fragment reads


// Workgroup tile: TN substrate rows (output columns) x TM activation rows,
// four waves in a 2 x 2 arrangement.  NS register sets keep the global loads
// of the next NS K-steps in flight (NS >= K/64 issues every load of the tile
// at once); two LDS buffers, one barrier per step.
template <int TM, int TN, int NS>
__global__ __launch_bounds__(GM_THREADS) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int WN = TN / 2, WM = TM / 2;            // wave tile
  constexpr int NI = WN / 16, MJ = WM / 16;          // MFMA blocks per wave
  constexpr int UCH = TM * (GBK / 8);                // 16-byte chunks of the U tile per step
  constexpr int UPT = UCH / GM_THREADS;
  constexpr int WWD = TN * (GBK / 16);               // packed words of the W tile per step
  constexpr int WPT = WWD / GM_THREADS;
  static_assert(UPT >= 1 && WPT >= 1, "tile too small");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* sW = smem;                       // [2][TN][GLDK]
  uint16_t* sU = smem + 2 * TN * GLDK;       // [2][TM][GLDK]

  const int ntn = (a.N + TN - 1) / TN;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tn = logical % ntn, tm = logical / ntn;
  const int n0 = tn * TN, m0 = tm * TM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int K = a.K, KW = a.K >> 4;
  const uint16_t* A = reinterpret_cast<const uint16_t*>(a.a);

  uint4 ureg[NS][UPT];
  uint32_t wreg[NS][WPT];
  // (all set indices below are compile-time constants after unrolling)
  auto gload = [&](int k0, uint4 (&ur)[UPT], uint32_t (&wr)[WPT]) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int c = tid + GM_THREADS * i;
      const int row = c >> 3, ch = c & 7;
      const int m = m0 + row;
      ur[i] = (m < a.M) ? *reinterpret_cast<const uint4*>(A + size_t(m) * K + k0 + 8 * ch)
                        : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int w = tid + GM_THREADS * i;
      const int row = w >> 2, kw = w & 3;
      const int n = n0 + row;
      wr[i] = (n < a.N) ? a.w[size_t(n) * KW + (k0 >> 4) + kw] : 0u;
    }
  };
  auto lstore = [&](int buf, const uint4 (&ur)[UPT], const uint32_t (&wr)[WPT]) {
    uint16_t* su = sU + buf * TM * GLDK;
    uint16_t* sw = sW + buf * TN * GLDK;
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int c = tid + GM_THREADS * i;
      const int row = c >> 3, ch = c & 7;
      *reinterpret_cast<uint4*>(su + row * GLDK + 8 * ch) = ur[i];
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int w = tid + GM_THREADS * i;
      const int row = w >> 2, kw = w & 3;
      const uint32_t P = wr[i];
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

  f32x4_t acc[NI][MJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = K / GBK;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < nk) gload(s * GBK, ureg[s], wreg[s]);

  for (int kb = 0; kb < nk; kb += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int kt = kb + s;
      if (kt < nk) {
        const int buf = kt & 1;
        lstore(buf, ureg[s], wreg[s]);
        __syncthreads();
        if (kt + NS < nk) gload((kt + NS) * GBK, ureg[s], wreg[s]);  // refill this set
        const uint16_t* sw = sW + buf * TN * GLDK;
        const uint16_t* su = sU + buf * TM * GLDK;
#pragma unroll
        for (int kk = 0; kk < GBK; kk += 32) {
          bf16x8_t wf[NI], uf[MJ];
#pragma unroll
          for (int i = 0; i < NI; ++i)
            wf[i] = *reinterpret_cast<const bf16x8_t*>(sw + (wn * WN + 16 * i + (lane & 15)) * GLDK + kk + 8 * (lane >> 4));
#pragma unroll
          for (int j = 0; j < MJ; ++j)
            uf[j] = *reinterpret_cast<const bf16x8_t*>(su + (wm * WM + 16 * j + (lane & 15)) * GLDK + kk + 8 * (lane >> 4));
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < MJ; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i], uf[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  uint16_t* Z = reinterpret_cast<uint16_t*>(a.z);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int n = n0 + wn * WN + 16 * i + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      const int m = m0 + wm * WM + 16 * j + (lane & 15);
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

template <int TM, int TN, int NS>
static hipError_t launch_gemm_tile(const GemmArgs& a, hipStream_t s) {
  const int ntn = (a.N + TN - 1) / TN, ntm = (a.M + TM - 1) / TM;
  const size_t lds = size_t(2) * (TN + TM) * GLDK * sizeof(uint16_t);
  const hipError_t e = allow_dynamic_lds((const void*)gemm_bf16_kernel<TM, TN, NS>, lds);
  if (e != hipSuccess) return e;
  auto kern = gemm_bf16_kernel<TM, TN, NS>;
  hipLaunchKernelGGL(kern, dim3(ntn * ntm), dim3(GM_THREADS), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, int act, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (act == ACT_BF16) {
    // 128-row tiles once they give every CU two workgroups, 64-row tiles below
    const long tiles128 = long((a.M + 127) / 128) * ((a.N + 127) / 128);
    if (tiles128 >= 512) return launch_gemm_tile<128, 128, 1>(a, s);
    if (a.K <= 8 * GBK) return launch_gemm_tile<64, 128, 8>(a, s);
    return launch_gemm_tile<64, 128, 2>(a, s);
  }
  const size_t total = size_t(a.M) * a.N;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, s, a);
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
