// Shared ternary substrate product Z = alpha * U * W^T for wide layers, with the
// substrate pre-encoded as fp4 e2m1 (ButterflyMoE, gist.science/zh/paper/2601.13563,
// technical summary §2.1-§2.2: one ternary substrate shared by every expert, so
// all routed rows form one dense contraction: M = rows, N = d_out, K = d_in).
//
// Workgroup tile: 128 rows x TN output columns, four waves; wave w owns output
// columns [w TN/4, (w+1) TN/4) for all 128 rows, so no two waves read the same
// substrate rows.  Its substrate fragments come straight from global memory
// (16 bytes = 32 fp4 weights per lane per 128-wide K step; four lanes fill a
// 64-byte half line of a row) and become exact bf16 +-1/0 with one
// v_cvt_scalef32_pk_bf16_fp4 per two weights.  The activation tile (128 rows x
// 128 K, bf16) goes through two LDS buffers and is read by all four waves.
// In a K step, lanes 16g .. 16g+15 supply contraction indices 32g .. 32g+31 of
// the step (8 per MFMA); the activation operand follows the same order.
// Accumulators (up to 256 per lane) live in AGPRs; one workgroup per CU.
//
// Tile order: groups of 4 row tiles sweep all column tiles, so a substrate
// slice is reused by 4 row tiles and an activation tile by every column tile
// while both sit in one XCD's L2 (contiguous logical tiles per XCD).
#include "common.hpp"

namespace bmoe {

constexpr int GF_THREADS = 256;
constexpr int GF_TM = 128;
constexpr int GF_KS = 128;          // K per step
constexpr int GF_UST = GF_KS + 8;   // LDS row stride (bf16)
constexpr int GF_GRP = 4;           // row tiles per group

__device__ __forceinline__ uint32_t gf_u4get(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

__device__ __forceinline__ uint4 gf_fp4x8_to_bf16(uint32_t w) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
  return r;
}

template <int TN>
__global__ __launch_bounds__(GF_THREADS, 1) void gemm_fp4_kernel(GemmFp4Args a) {
  constexpr int WN = TN / 4;                  // output columns per wave
  constexpr int OB = WN / 16;                 // 16-column blocks per wave
  constexpr int MB = GF_TM / 16;              // 16-row blocks
  constexpr int UCH = GF_TM * GF_KS / 8;      // 16-byte chunks of an activation tile
  constexpr int UPT = UCH / GF_THREADS;       // per thread (8)
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];  // [2][GF_TM][GF_UST]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int ntn = a.N / TN, ntm = (a.M + GF_TM - 1) / GF_TM;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = logical / (GF_GRP * ntn), r = logical % (GF_GRP * ntn);
  const int tn = r / GF_GRP, tm = grp * GF_GRP + r % GF_GRP;
  if (tm >= ntm) return;
  const int m0 = tm * GF_TM, n0 = tn * TN + wave * WN;
  const int K = a.K, nk = K / GF_KS;
  const uint16_t* U = reinterpret_cast<const uint16_t*>(a.a);
  // this lane's substrate rows n0 + 16 i + l16, bytes 16 g .. 16 g + 15 of each 64-byte step
  const unsigned char* wrow = a.w + size_t(n0 + l16) * (K / 2) + 16 * g;

  auto load_w = [&](int kt, uint4 (&w)[OB]) {
#pragma unroll
    for (int i = 0; i < OB; ++i)
      w[i] = *reinterpret_cast<const uint4*>(wrow + size_t(16 * i) * (K / 2) + 64 * kt);
  };
  auto load_u = [&](int kt, uint4 (&u)[UPT]) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int c = j * GF_THREADS + tid;
      const int row = c / (GF_KS / 8), ch = c % (GF_KS / 8);
      const int m = m0 + row;
      u[j] = m < a.M ? *reinterpret_cast<const uint4*>(U + size_t(m) * K + kt * GF_KS + 8 * ch)
                     : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_u = [&](int buf, const uint4 (&u)[UPT]) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int c = j * GF_THREADS + tid;
      const int row = c / (GF_KS / 8), ch = c % (GF_KS / 8);
      *reinterpret_cast<uint4*>(smem + (buf * GF_TM + row) * GF_UST + 8 * ch) = u[j];
    }
  };

  f32x4_t acc[OB][MB];
#pragma unroll
  for (int i = 0; i < OB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 W0[OB], W1[OB], Ur[UPT];
  load_u(0, Ur);
  load_w(0, W0);
  if (nk > 1) load_w(1, W1);
  store_u(0, Ur);
  if (nk > 1) load_u(1, Ur);
  __syncthreads();

  // one K step: MFMAs on LDS buffer `buf` with substrate set Wc; then publish
  // the next activation tile and refill Wc with step kt + 2
  auto step = [&](int kt, uint4 (&Wc)[OB]) {
    const int buf = kt & 1;
    const uint16_t* su = smem + buf * GF_TM * GF_UST + l16 * GF_UST + 32 * g;
#pragma unroll 1
    for (int s = 0; s < 4; ++s) {
      bf16x8_t uf[MB];
#pragma unroll
      for (int j = 0; j < MB; ++j)
        uf[j] = *reinterpret_cast<const bf16x8_t*>(su + 16 * j * GF_UST + 8 * s);
#pragma unroll
      for (int i = 0; i < OB; ++i) {
        const bf16x8_t wf = __builtin_bit_cast(bf16x8_t, gf_fp4x8_to_bf16(gf_u4get(Wc[i], s)));
#pragma unroll
        for (int j = 0; j < MB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, uf[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 2 < nk) load_w(kt + 2, Wc);
    if (kt + 1 < nk) {
      store_u(buf ^ 1, Ur);
      if (kt + 2 < nk) load_u(kt + 2, Ur);
    }
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, W0);
    if (kt + 1 < nk) step(kt + 1, W1);
  }

  uint16_t* Z = reinterpret_cast<uint16_t*>(a.z);
#pragma unroll
  for (int i = 0; i < OB; ++i) {
    const int n = n0 + 16 * i + 4 * g;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int m = m0 + 16 * j + l16;
      if (m < a.M) {
        uint2 o;
        o.x = pack_bf16x2(a.alpha * acc[i][j][0], a.alpha * acc[i][j][1]);
        o.y = pack_bf16x2(a.alpha * acc[i][j][2], a.alpha * acc[i][j][3]);
        *reinterpret_cast<uint2*>(Z + size_t(m) * a.N + n) = o;
      }
    }
  }
}

template <int TN>
static hipError_t launch_gemm_fp4_tn(const GemmFp4Args& a, hipStream_t s) {
  const int ntn = a.N / TN, ntm = (a.M + GF_TM - 1) / GF_TM;
  const int ngrp = (ntm + GF_GRP - 1) / GF_GRP;
  const size_t lds = size_t(2) * GF_TM * GF_UST * sizeof(uint16_t);
  static int attr_done[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (lds > 64 * 1024 && (dev < 0 || dev >= 64 || !attr_done[dev])) {
    e = hipFuncSetAttribute((const void*)gemm_fp4_kernel<TN>, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_done[dev] = 1;
  }
  hipLaunchKernelGGL(gemm_fp4_kernel<TN>, dim3(ngrp * GF_GRP * ntn), dim3(GF_THREADS), lds, s, a);
  return hipGetLastError();
}

bool gemm_fp4_supported(int N, int K) { return N % 256 == 0 && K % GF_KS == 0; }

hipError_t launch_gemm_fp4(const GemmFp4Args& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (!gemm_fp4_supported(a.N, a.K)) return hipErrorInvalidValue;
  if (a.N % 512 == 0) return launch_gemm_fp4_tn<512>(a, s);
  return launch_gemm_fp4_tn<256>(a, s);
}

}  // namespace bmoe
