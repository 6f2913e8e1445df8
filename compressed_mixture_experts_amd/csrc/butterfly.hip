// Butterfly rotations of token rows (ButterflyMoE, gist.science/zh/paper/2601.13563,
// technical summary §2.2: each expert's rotations are hierarchical Givens
// rotations and permutations; §2.1: inference rotates the input, multiplies by
// the ternary substrate, rotates the output, without materialising the expert).
//
// One workgroup owns a tile of rows that all belong to one expert (rows are
// bucketed by expert beforehand), so the expert's angles are read and turned
// into (cos, sin) once per tile and reused for every row of the tile.
//
// The tile lives in LDS as fp32.  The log2(n) stages are applied in passes of up
// to three consecutive stages: in a pass every thread holds the 2^m elements
// of one closed group (indices that differ only in the pass's stage bits) in
// registers, applies the m stages there and writes the group back, so each
// stage costs no LDS traffic of its own.  Rows are padded by 8 floats every 64
// so that the strided groups of the middle passes hit distinct LDS banks.
//
// Modes:
//   DBG  rows in -> rows out, one shared angle set (test hook)
//   IN   gather x[token of bucket row q] -> B(theta_e)^T -> U[q]
//   MID  H[q] -> B(phi_up,e) -> GELU -> B(theta_dn,e)^T -> A[q] (in place)
//   OUT  Z[q] -> B(phi_e) -> * gate -> Y[slot of q]
#include "common.hpp"

namespace bmoe {

constexpr int BF_THREADS = 256;
constexpr float kInv2Pi = 0.15915494309189535f;

__device__ __forceinline__ int pidx(int i) { return i + ((i >> 6) << 3); }

__device__ __forceinline__ float gelu_erf(float h) {
  return h * 0.5f * (1.0f + erff(h * 0.70710678118654752f));
}

// cos and sin of an angle in radians with the hardware transcendental unit
// (v_sin_f32 / v_cos_f32 take the angle in revolutions).
__device__ __forceinline__ void sincos_rev(float a, float& c, float& s) {
  const float r = a * kInv2Pi;
  s = __builtin_amdgcn_sinf(r);
  c = __builtin_amdgcn_cosf(r);
}

int bfly_rows_per_tile(int log2n) {
  // fp32 tile with 1/8 padding: about 72 KiB up to n = 1024 (two workgroups
  // per CU), about 144 KiB above (one workgroup per CU).
  const int n = 1 << log2n;
  const int budget_floats = (log2n <= 10 ? 18432 : 36864);
  int rt = budget_floats / (n + (n >> 3));
  if (rt > 32) rt = 32;
  if (rt < 1) rt = 1;
  // power of two
  int p = 1;
  while (p * 2 <= rt) p *= 2;
  return p;
}

// One pass of M stages s0 .. s0+M-1 over rows [0, nr) of the tile.
template <int M, bool TRANS, bool POST_GELU>
__device__ __forceinline__ void bfly_pass(float* __restrict__ tile, int stride, int n, int s0,
                                          int nr, const float* __restrict__ ang) {
  constexpr int E = 1 << M;
  constexpr int P = E / 2;
  const int half = n >> 1;
  const int G = n >> M;
  const int tid = threadIdx.x;
  int g0, gstep, r0, rstep;
  if (G >= BF_THREADS) {
    g0 = tid; gstep = BF_THREADS; r0 = 0; rstep = 1;
  } else {
    g0 = tid & (G - 1); gstep = G; r0 = tid / G; rstep = BF_THREADS / G;
  }
  for (int g = g0; g < G; g += gstep) {
    const int lowmask = (1 << s0) - 1;
    const int base = (g & lowmask) | ((g >> s0) << (s0 + M));
    float cs[M][P], sn[M][P];
#pragma unroll
    for (int k = 0; k < M; ++k) {
      const int s = s0 + k;
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int e = ((q >> k) << (k + 1)) | (q & ((1 << k) - 1));
        const int i = base + (e << s0);
        const int p = ((i >> (s + 1)) << s) | (i & ((1 << s) - 1));
        sincos_rev(ang[s * half + p], cs[k][q], sn[k][q]);
      }
    }
    int addr[E];
#pragma unroll
    for (int e = 0; e < E; ++e) addr[e] = pidx(base + (e << s0));
    for (int r = r0; r < nr; r += rstep) {
      float* row = tile + r * stride;
      float v[E];
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = row[addr[e]];
      if constexpr (!TRANS) {
#pragma unroll
        for (int k = 0; k < M; ++k) {
#pragma unroll
          for (int q = 0; q < P; ++q) {
            const int e = ((q >> k) << (k + 1)) | (q & ((1 << k) - 1));
            const int f = e + (1 << k);
            const float a = v[e], b = v[f], c = cs[k][q], s = sn[k][q];
            v[e] = c * a - s * b;
            v[f] = s * a + c * b;
          }
        }
      } else {
#pragma unroll
        for (int k = M - 1; k >= 0; --k) {
#pragma unroll
          for (int q = 0; q < P; ++q) {
            const int e = ((q >> k) << (k + 1)) | (q & ((1 << k) - 1));
            const int f = e + (1 << k);
            const float a = v[e], b = v[f], c = cs[k][q], s = sn[k][q];
            v[e] = c * a + s * b;
            v[f] = c * b - s * a;
          }
        }
      }
      if constexpr (POST_GELU) {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = gelu_erf(v[e]);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) row[addr[e]] = v[e];
    }
  }
}

template <bool TRANS, bool POST_GELU>
__device__ __forceinline__ void bfly_pass_m(int m, float* tile, int stride, int n, int s0, int nr,
                                            const float* ang) {
  if (m == 3) bfly_pass<3, TRANS, POST_GELU>(tile, stride, n, s0, nr, ang);
  else if (m == 2) bfly_pass<2, TRANS, POST_GELU>(tile, stride, n, s0, nr, ang);
  else bfly_pass<1, TRANS, POST_GELU>(tile, stride, n, s0, nr, ang);
}

// All L stages of one butterfly over the tile; passes of three stages.
// Forward (B v): stage 0 first.  Transposed (B^T v): stage L-1 first.
template <bool TRANS>
__device__ void bfly_all(float* tile, int stride, int L, int nr, const float* ang, bool post_gelu) {
  const int n = 1 << L;
  const int np = (L + 2) / 3;
  for (int t = 0; t < np; ++t) {
    const int P = TRANS ? (np - 1 - t) : t;
    const int s0 = 3 * P;
    const int m = (L - s0) < 3 ? (L - s0) : 3;
    const bool last = (t == np - 1);
    if (post_gelu && last) bfly_pass_m<TRANS, true>(m, tile, stride, n, s0, nr, ang);
    else bfly_pass_m<TRANS, false>(m, tile, stride, n, s0, nr, ang);
    __syncthreads();
  }
}

// Exclusive scan over the 256 threads of the block; `total` gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_tmp[w] = x;
  __syncthreads();
  int pre = 0;
  for (int i = 0; i < w; ++i) pre += s_tmp[i];
  total = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
  return pre + x - v;
}

template <int MODE, int ACT, bool DBG_TRANS>
__global__ __launch_bounds__(BF_THREADS) void bfly_kernel(BflyArgs a, int L, int RT) {
  extern __shared__ float tile[];
  __shared__ int s_info[3];
  __shared__ int s_tmp[4];
  const int n = 1 << L;
  const int stride = n + (n >> 3);
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const size_t angs = size_t(L) * (n >> 1);

  int e, r0, nr;
  if constexpr (MODE == BFLY_DBG) {
    e = 0;
    r0 = t * RT;
    nr = min(RT, a.rows - r0);
    if (nr <= 0) return;
  } else {
    if (tid == 0) s_info[0] = -1;
    int nt = 0, cnt = 0, off = 0;
    if (tid < a.n_experts) {
      off = a.offsets[tid];
      cnt = a.offsets[tid + 1] - off;
      nt = (cnt + RT - 1) / RT;
    }
    int total;
    const int excl = block_excl_scan(nt, s_tmp, total);
    if (tid < a.n_experts && t >= excl && t < excl + nt) {
      const int j = t - excl;
      s_info[0] = tid;
      s_info[1] = off + j * RT;
      s_info[2] = min(RT, cnt - j * RT);
    }
    __syncthreads();
    e = s_info[0];
    if (e < 0) return;
    r0 = s_info[1];
    nr = s_info[2];
  }

  // ---- prologue: rows -> fp32 tile
  const int cpr = n >> 3;  // 8-element chunks per row
  for (int c = tid; c < nr * cpr; c += BF_THREADS) {
    const int r = c / cpr;
    const int col = (c - r * cpr) << 3;
    const int q = r0 + r;
    size_t src;
    if constexpr (MODE == BFLY_IN) {
      const int slot = a.perm[q];
      src = size_t(slot / a.top_k) * n + col;
    } else {
      src = size_t(q) * n + col;
    }
    float v[8];
    load8<ACT>(a.in, src, v);
    float* dst = tile + r * stride + pidx(col);
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = v[j];
  }
  __syncthreads();

  // ---- rotations
  if constexpr (MODE == BFLY_DBG) {
    bfly_all<DBG_TRANS>(tile, stride, L, nr, a.ang0, false);
  } else if constexpr (MODE == BFLY_IN) {
    bfly_all<true>(tile, stride, L, nr, a.ang0 + size_t(e) * angs, false);
  } else if constexpr (MODE == BFLY_MID) {
    bfly_all<false>(tile, stride, L, nr, a.ang0 + size_t(e) * angs, a.gelu != 0);
    bfly_all<true>(tile, stride, L, nr, a.ang1 + size_t(e) * angs, false);
  } else {
    bfly_all<false>(tile, stride, L, nr, a.ang0 + size_t(e) * angs, false);
  }

  // ---- epilogue: fp32 tile -> rows
  for (int c = tid; c < nr * cpr; c += BF_THREADS) {
    const int r = c / cpr;
    const int col = (c - r * cpr) << 3;
    const int q = r0 + r;
    const float* srcp = tile + r * stride + pidx(col);
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = srcp[j];
    size_t dst;
    if constexpr (MODE == BFLY_OUT) {
      const int slot = a.perm[q];
      const float g = a.gate[slot];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] *= g;
      dst = size_t(slot) * n + col;
    } else {
      dst = size_t(q) * n + col;
    }
    store8<ACT>(a.out, dst, v);
  }
}

template <int MODE, int ACT, bool TR>
static hipError_t launch_one(const BflyArgs& a, int log2n, hipStream_t s) {
  const int n = 1 << log2n;
  const int RT = bfly_rows_per_tile(log2n);
  const size_t lds = size_t(RT) * (n + (n >> 3)) * sizeof(float);
  int grid = (a.rows + RT - 1) / RT;
  if (MODE != BFLY_DBG) grid += a.n_experts;
  if (grid == 0) return hipSuccess;
  auto k = bfly_kernel<MODE, ACT, TR>;
  static int attr_done[64] = {0};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64 || !attr_done[dev]) {
    err = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                              int(size_t(36864) * sizeof(float)));
    if (err != hipSuccess) return err;
    if (dev >= 0 && dev < 64) attr_done[dev] = 1;
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(BF_THREADS), lds, s, a, log2n, RT);
  return hipGetLastError();
}

hipError_t launch_butterfly(const BflyArgs& a, int mode, int act, int log2n, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
#define BMOE_BF(MODE, TR)                                                        \
  return act == ACT_BF16 ? launch_one<MODE, ACT_BF16, TR>(a, log2n, s)           \
                         : launch_one<MODE, ACT_F32, TR>(a, log2n, s)
  switch (mode) {
    case BFLY_DBG:
      if (a.transpose) { BMOE_BF(BFLY_DBG, true); }
      BMOE_BF(BFLY_DBG, false);
    case BFLY_IN: BMOE_BF(BFLY_IN, false);
    case BFLY_MID: BMOE_BF(BFLY_MID, false);
    default: BMOE_BF(BFLY_OUT, false);
  }
#undef BMOE_BF
}

}  // namespace bmoe
