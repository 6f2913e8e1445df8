// Gradient of the latent substrate weights (ButterflyMoE,
// gist.science/nl/paper/2601.13563, §2 "Drie Fasen": the ternary substrate is
// trained through a straight-through estimator; gist.science/zh/paper/2601.13563,
// technical summary §2.2).  The estimator passes the gradient of the product
// Z = alpha U W^T through the quantiser unchanged, and the substrate is shared
// by every expert, so one contraction over all routed rows gives it:
//     dW[o][i] = alpha * sum_r dZ[r][o] U[r][i]      (M = d_out, N = d_in, K = rows)
//
// bf16 rows on MFMA (16x16x32, fp32 accumulation).  Both operands are stored
// with K (the row) outermost while a fragment needs 8 consecutive K per lane,
// so each 64-row step goes through LDS with K innermost: a thread loads an
// 8 x 8 block (8 rows of 8 consecutive columns, eight 16-byte loads),
// transposes it in registers and writes 8 columns of 8 rows as 16-byte runs;
// the fragments are then 16-byte LDS reads.  Lane l of a wave takes row block
// l % 8 and column block l / 8 (+ 8 per earlier wave of its operand), so the
// 16 lanes of an LDS write phase cover all banks.  Workgroup tile: T x T
// outputs with T = 128 (four waves of 64 x 64) or, where the tiles still fill
// the GPU, T = 256 (eight waves of 128 x 64, one workgroup per CU: twice the
// products per loaded byte, the loads being the limit); the next step's loads
// are in flight while the current step multiplies, two LDS buffers.  Few output tiles
// (small d) split K: each split writes an fp32 partial tile and a second
// kernel adds the splits in order (deterministic), times alpha.
#include "common.hpp"

namespace bmoe {

constexpr int SG_KT = 64;   // rows per step (two MFMA K)
constexpr int SG_RS = 72;   // LDS row stride in bf16: 64 rows + 8 (144 bytes)

struct SgradArgs {
  const uint16_t* dz;  // [R][M] bf16
  const uint16_t* u;   // [R][N] bf16
  float* out;          // [M][N]
  float* part;         // [nsplit][M][N] when nsplit > 1
  float alpha;
  int32_t R, M, N, kchunk, nsplit;
};

template <int T>
__global__ __launch_bounds__(2 * T, T == 128 ? 2 : 1) void sgrad_kernel(SgradArgs a) {
  constexpr int NW = 2 * T / 64;      // waves
  constexpr int WM = T / 2;           // rows (of dW) per wave: two waves along M
  constexpr int IM = WM / 16;         // 16-row blocks per wave
  __shared__ __attribute__((aligned(16))) uint16_t sm[2][2][T * SG_RS];  // [buffer][dZ, U][col][row]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int tM = a.M / T, tN = a.N / T, tiles = tM * tN;
  const int tile = blockIdx.x % tiles, split = blockIdx.x / tiles;
  const int m0 = (tile % tM) * T, n0 = (tile / tM) * T;
  const int k0 = split * a.kchunk, k1 = min(a.R, k0 + a.kchunk);
  const int wm = wave & 1, wn = wave >> 1;  // wave's 64 columns: wn of T / 64
  // loader: operand op (first half of the waves dZ, second U), row block rb,
  // column block cb
  const int op = wave / (NW / 2), rb = lane & 7, cb = (lane >> 3) + 8 * (wave % (NW / 2));
  const uint16_t* src = op ? a.u : a.dz;
  const int ld = op ? a.N : a.M, c0 = (op ? n0 : m0) + 8 * cb;
  uint4 blk[8];

  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = kb + 8 * rb + i;
      blk[i] = r < k1 ? *reinterpret_cast<const uint4*>(src + size_t(r) * ld + c0) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  // column c of the block (rows 0..7) as four words of two rows each
  auto lstore = [&](int buf) {
    uint16_t* base = sm[buf][op] + (8 * cb) * SG_RS + 8 * rb;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint4& x0 = blk[2 * p];
        const uint4& x1 = blk[2 * p + 1];
        const uint32_t v0 = (c >> 1) == 0 ? x0.x : (c >> 1) == 1 ? x0.y : (c >> 1) == 2 ? x0.z : x0.w;
        const uint32_t v1 = (c >> 1) == 0 ? x1.x : (c >> 1) == 1 ? x1.y : (c >> 1) == 2 ? x1.z : x1.w;
        w[p] = (c & 1) ? ((v0 >> 16) | (v1 & 0xFFFF0000u)) : ((v0 & 0xFFFFu) | (v1 << 16));
      }
      *reinterpret_cast<uint4*>(base + c * SG_RS) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };

  f32x4_t acc[IM][4];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (k0 < k1) {
    gload(k0);
    lstore(0);
  }
  __syncthreads();
  int buf = 0;
  for (int kb = k0; kb < k1; kb += SG_KT) {
    const bool more = kb + SG_KT < k1;
    if (more) gload(kb + SG_KT);
    const uint16_t* A = sm[buf][0];
    const uint16_t* B = sm[buf][1];
#pragma unroll
    for (int ks = 0; ks < SG_KT / 32; ++ks) {
      bf16x8_t fa[IM], fb[4];
#pragma unroll
      for (int i = 0; i < IM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8_t*>(A + (wm * WM + 16 * i + l16) * SG_RS + 32 * ks + 8 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fb[i] = *reinterpret_cast<const bf16x8_t*>(B + (wn * 64 + 16 * i + l16) * SG_RS + 32 * ks + 8 * g);
#pragma unroll
      for (int i = 0; i < IM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (more) lstore(buf ^ 1);  // its last readers finished before the previous barrier
    __syncthreads();
    buf ^= 1;
  }

  // acc[i][j][v] = C[m0 + WM wm + 16 i + 4 g + v][n0 + 64 wn + 16 j + l16]
  float* dst = a.nsplit > 1 ? a.part + size_t(split) * a.M * a.N : a.out;
  const float sc = a.nsplit > 1 ? 1.f : a.alpha;
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int o = m0 + WM * wm + 16 * i + 4 * g + v, n = n0 + 64 * wn + 16 * j + l16;
        dst[size_t(o) * a.N + n] = sc * acc[i][j][v];
      }
}

// out = alpha * sum over the splits in order (4 outputs per thread)
__global__ __launch_bounds__(256) void sgrad_reduce_kernel(SgradArgs a) {
  const size_t MN = size_t(a.M) * a.N, q = (size_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (q >= MN) return;
  float4 s = *reinterpret_cast<const float4*>(a.part + q);
  for (int k = 1; k < a.nsplit; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(a.part + size_t(k) * MN + q);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  *reinterpret_cast<float4*>(a.out + q) = make_float4(a.alpha * s.x, a.alpha * s.y, a.alpha * s.z, a.alpha * s.w);
}

__global__ __launch_bounds__(256) void sgrad_zero_kernel(float* out, size_t n) {
  const size_t q = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (q < n) out[q] = 0.f;
}

bool sgrad_shape_ok(int M, int N) { return M % 128 == 0 && N % 128 == 0 && M > 0 && N > 0; }

// output tile edge: 256 where those tiles number at least 256 (one workgroup
// per CU), else 128
static int sgrad_tile(int M, int N) {
  return (M % 256 == 0 && N % 256 == 0 && (M / 256) * (N / 256) >= 256) ? 256 : 128;
}

// splits of K: none when the output tiles alone fill the chip (>= 256),
// else enough for about 512 workgroups with at least 512 rows each
int sgrad_splits(int M, int N, int R, int* kchunk) {
  const int T = sgrad_tile(M, N), tiles = (M / T) * (N / T);
  int ns = 1;
  if (tiles < 256) {
    ns = (512 + tiles - 1) / tiles;
    const int kmax = (R + 511) / 512;
    ns = ns < kmax ? ns : kmax;
    ns = ns < 1 ? 1 : ns;
  }
  int kc = (R + ns - 1) / ns;
  kc = (kc + SG_KT - 1) / SG_KT * SG_KT;
  if (kc < SG_KT) kc = SG_KT;
  ns = (R + kc - 1) / kc;
  if (ns < 1) ns = 1;
  if (kchunk) *kchunk = kc;
  return ns;
}

size_t sgrad_workspace(int M, int N, int R) {
  if (R <= 0) return 0;
  const int ns = sgrad_splits(M, N, R, nullptr);
  return ns > 1 ? size_t(ns) * M * N * sizeof(float) : 0;
}

hipError_t launch_sgrad(const void* dz, const void* u, float alpha, float* out, float* part, int R, int M, int N,
                        hipStream_t s) {
  const size_t MN = size_t(M) * N;
  if (R <= 0) {
    hipLaunchKernelGGL(sgrad_zero_kernel, dim3((MN + 255) / 256), dim3(256), 0, s, out, MN);
    return hipGetLastError();
  }
  SgradArgs a{static_cast<const uint16_t*>(dz), static_cast<const uint16_t*>(u), out, part, alpha, R, M, N, 0, 0};
  a.nsplit = sgrad_splits(M, N, R, &a.kchunk);
  const int T = sgrad_tile(M, N), tiles = (M / T) * (N / T);
  if (T == 256) {
    hipLaunchKernelGGL(sgrad_kernel<256>, dim3(tiles * a.nsplit), dim3(512), 0, s, a);
  } else {
    hipLaunchKernelGGL(sgrad_kernel<128>, dim3(tiles * a.nsplit), dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(sgrad_reduce_kernel, dim3((MN / 4 + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bmoe
