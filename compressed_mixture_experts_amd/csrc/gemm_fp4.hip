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
// the step (8 per MFMA); the activation operand follows the same order.  The
// loads of step k+1 are issued before the products of step k.
// TN = 256: 64 columns per wave, 128 accumulators per lane, two workgroups
// per CU (LDS 64 KiB each), so one workgroup's products cover the other's
// load waits.
//
// Tile order: groups of 4 row tiles sweep all column tiles, so a substrate
// slice is reused by 4 row tiles and an activation tile by every column tile
// while both sit in one XCD's L2 (contiguous logical tiles per XCD).
#include "common.hpp"

namespace bmoe {

constexpr int GF_THREADS = 256;
constexpr int GF_TM = 128;
constexpr int GF_KS = 128;          // K per step
constexpr int GF_GRP = 4;           // row tiles per group
constexpr int GF_TILE = GF_TM * GF_KS;  // bf16 elements of one activation tile

typedef __attribute__((address_space(3))) void gf_lds_t;
typedef __attribute__((address_space(1))) const void gf_glob_t;

__device__ __forceinline__ uint4 gf_fp4x8_to_bf16(uint32_t w) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
  return r;
}

// Activation tile in LDS: 128 rows of 128 bf16 (256 bytes, no padding); the
// 16-byte chunk ch of row r sits at position ch ^ (r & 15) of the row, so the
// 16 rows one MFMA operand read touches hit 16 different bank groups.  The
// tile is filled by direct global->LDS loads: one 16-byte load per lane, each
// wave-wide load filling 4 consecutive rows.
template <int TN>
__global__ __launch_bounds__(GF_THREADS, 2) void gemm_fp4_kernel(GemmFp4Args a) {
  constexpr int WN = TN / 4;                  // output columns per wave
  constexpr int OB = WN / 16;                 // 16-column blocks per wave
  constexpr int MB = GF_TM / 16;              // 16-row blocks
  constexpr int DPW = GF_TM / 4 / 4;          // direct loads per wave per tile (4 rows each)
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];  // [2][GF_TM][GF_KS]

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
  // this lane's source of direct load j: row 4 (DPW wave + j) + lane / 16 (clamped to
  // M - 1: rows past M are never stored), chunk (lane % 16) ^ (row % 16)
  auto usrc = [&](int j) {
    const int row = 4 * (DPW * wave + j) + (lane >> 4);
    const int ch = (lane & 15) ^ (row & 15);
    return U + size_t(min(m0 + row, a.M - 1)) * K + 8 * ch;
  };

  auto load_w = [&](int kt, uint4 (&w)[OB]) {
#pragma unroll
    for (int i = 0; i < OB; ++i)
      w[i] = *reinterpret_cast<const uint4*>(wrow + size_t(16 * i) * (K / 2) + 64 * kt);
  };
  auto load_u = [&](int kt, int buf) {
#pragma unroll
    for (int j = 0; j < DPW; ++j)
      __builtin_amdgcn_global_load_lds((gf_glob_t*)(usrc(j) + kt * GF_KS),
                                       (gf_lds_t*)(smem + buf * GF_TILE + (4 * (DPW * wave + j)) * GF_KS),
                                       16, 0, 0);
  };

  f32x4_t acc[OB][MB];
#pragma unroll
  for (int i = 0; i < OB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // operand reads: row 16 jb + l16, chunk 4 g + s at position (4 g + s) ^ l16
  auto load_uf = [&](const uint16_t* ub, int s, bf16x8_t (&uf)[MB]) {
    const int p = (4 * g + s) ^ l16;
#pragma unroll
    for (int j = 0; j < MB; ++j)
      uf[j] = *reinterpret_cast<const bf16x8_t*>(ub + (16 * j + l16) * GF_KS + 8 * p);
  };
  // products of one sub-step with dword 0 of each substrate fragment, which
  // then rotates so that the next sub-step's dword is dword 0 (the sub-step
  // loop stays rolled, which bounds the live operand registers)
  auto substep = [&](const bf16x8_t (&uf)[MB], uint4 (&Wc)[OB]) {
#pragma unroll
    for (int i = 0; i < OB; ++i) {
      const bf16x8_t wf = __builtin_bit_cast(bf16x8_t, gf_fp4x8_to_bf16(Wc[i].x));
      Wc[i] = make_uint4(Wc[i].y, Wc[i].z, Wc[i].w, Wc[i].x);
#pragma unroll
      for (int j = 0; j < MB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, uf[j], acc[i][j], 0, 0, 0);
    }
  };
  // step kt: start the loads of step kt + 1 (activation tile into the other LDS
  // buffer, substrate fragments into Wn), multiply buffer kt & 1 with Wc, then
  // wait for the loads and for every wave.  The operand fragments of sub-step
  // s + 1 are read while sub-step s multiplies (the read past sub-step 3 is of
  // chunk 4 g + 4 ^ l16 < 16 of the same rows, unused).
  auto step = [&](int kt, uint4 (&Wc)[OB], uint4 (&Wn)[OB]) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      load_u(kt + 1, buf ^ 1);
      load_w(kt + 1, Wn);
    }
    const uint16_t* ub = smem + buf * GF_TILE;
    bf16x8_t ua[MB], ubf[MB];
    load_uf(ub, 0, ua);
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      load_uf(ub, 2 * h + 1, ubf);
      substep(ua, Wc);
      load_uf(ub, (2 * h + 2) & 3, ua);
      substep(ubf, Wc);
    }
    __syncthreads();  // waits for this wave's loads, then for every wave
  };

  uint4 W0[OB], W1[OB];
  load_u(0, 0);
  load_w(0, W0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, W0, W1);
    if (kt + 1 < nk) step(kt + 1, W1, W0);
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
  const size_t lds = size_t(2) * GF_TILE * sizeof(uint16_t);
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
  return launch_gemm_fp4_tn<256>(a, s);
}

}  // namespace bmoe
