// Gradients through the experts' butterfly rotations (ButterflyMoE,
// gist.science/zh/paper/2601.13563, technical summary §2.2: each expert's
// learnable parameters are the angles of its hierarchical Givens rotations).
//
// Rows are bucketed by expert (rows offsets[e] .. offsets[e+1]-1 belong to
// expert e).  For y_r = B(ang_e) x_r (or B(ang_e)^T x_r) and a given dy_r the
// pass returns dx_r and, per expert, the angle gradients summed over its rows.
//
// Every stage is a rotation, so its input follows from its output by the
// inverse rotation, and the derivative of a rotated pair by its angle is a
// quarter turn of the pair's output: for (a', b') = (c a - s b, s a + c b)
//     d a'/dt = -b',   d b'/dt = a'
// (for the transposed stage, (c a + s b, -s a + c b): d a'/dt = b', d b'/dt = -a').
// So one workgroup holds a tile of one expert's rows in LDS (fp32), runs the
// forward stages on them, then walks the stages back: each thread owns whole
// pairs of the stage, and for every row of the tile adds the pair's angle
// gradient (dy_a d a'/dt + dy_b d b'/dt), turns the pair's gradient back
// through the stage and the pair's values back to the stage input.  The
// tile's angle gradients go to a per-tile partial row, which a second kernel
// sums per expert in tile order (deterministic).
//
// Tiles: RT = min(64, 16384 / n) rows, so the two fp32 tiles fit 128 KiB of
// LDS; expert e's tiles are tile indices floor(off_e / RT) + e + j, j <
// ceil(cnt_e / RT) (at most one unused index between two experts), so the
// grid and the partial buffer have ceil(R / RT) + N entries.
#include "common.hpp"

namespace bmoe {

constexpr int BB_THREADS = 256;

int bfly_bwd_tile_rows(int log2n) {
  const int n = 1 << log2n;
  const int rt = 16384 / n;
  return rt > 64 ? 64 : rt;
}

struct BflyBwdArgs {
  const void* x;          // [R][n] rows, bucketed by expert
  const void* dy;         // [R][n]
  void* dx;               // [R][n]
  const float* ang;       // [N][L][n/2]
  const int32_t* offsets; // [N+1]
  float* part;            // [n_tiles][L][n/2] per-tile angle gradients
  float* dang;            // [N][L][n/2]
  int32_t rows, n_experts, transpose, rt, n_tiles;
};

// lower index of pair p in stage s
__device__ __forceinline__ int pair_lo(int p, int s) { return ((p >> s) << (s + 1)) | (p & ((1 << s) - 1)); }

template <int ACT>
__global__ __launch_bounds__(BB_THREADS) void bfly_bwd_kernel(BflyBwdArgs a, int L) {
  extern __shared__ __attribute__((aligned(16))) float tile[];  // V [RT][n], then G [RT][n]
  __shared__ int s_info[3];
  const int n = 1 << L, half = n >> 1, tid = threadIdx.x, RT = a.rt;
  float* V = tile;
  float* G = tile + size_t(RT) * n;

  // ---- which expert and rows this tile holds
  if (tid == 0) s_info[0] = -1;
  __syncthreads();
  for (int e = tid; e < a.n_experts; e += BB_THREADS) {
    const int off = min(max(a.offsets[e], 0), a.rows);
    const int cnt = min(max(a.offsets[e + 1], off), a.rows) - off;
    const int base = off / RT + e, nt = (cnt + RT - 1) / RT;
    const int b = blockIdx.x;
    if (b >= base && b < base + nt) {
      s_info[0] = e;
      s_info[1] = off + (b - base) * RT;
      s_info[2] = min(RT, cnt - (b - base) * RT);
    }
  }
  __syncthreads();
  const int e = s_info[0];
  if (e < 0) return;
  const int r0 = s_info[1], nr = s_info[2];
  const float* ang = a.ang + size_t(e) * L * half;

  // ---- rows -> LDS
  for (int q = tid; q < nr * n; q += BB_THREADS) {
    const size_t gi = size_t(r0) * n + q;
    V[q] = load1<ACT>(a.x, gi);
    G[q] = load1<ACT>(a.dy, gi);
  }
  __syncthreads();

  const bool tr = a.transpose != 0;
  // ---- forward stages: B applies stage 0 first, B^T stage L-1 first
  for (int k = 0; k < L; ++k) {
    const int s = tr ? L - 1 - k : k;
    for (int p = tid; p < half; p += BB_THREADS) {
      const int i = pair_lo(p, s), j = i + (1 << s);
      float sn, c;
      sincosf(ang[s * half + p], &sn, &c);
      for (int r = 0; r < nr; ++r) {
        const float x0 = V[r * n + i], x1 = V[r * n + j];
        V[r * n + i] = tr ? c * x0 + sn * x1 : c * x0 - sn * x1;
        V[r * n + j] = tr ? -sn * x0 + c * x1 : sn * x0 + c * x1;
      }
    }
    __syncthreads();
  }

  // ---- backward: stages in the reverse order of application
  float* part = a.part + size_t(blockIdx.x) * L * half;
  for (int k = L - 1; k >= 0; --k) {
    const int s = tr ? L - 1 - k : k;
    for (int p = tid; p < half; p += BB_THREADS) {
      const int i = pair_lo(p, s), j = i + (1 << s);
      float sn, c;
      sincosf(ang[s * half + p], &sn, &c);
      float acc = 0.f;
      for (int r = 0; r < nr; ++r) {
        const float o0 = V[r * n + i], o1 = V[r * n + j];  // stage outputs
        const float g0 = G[r * n + i], g1 = G[r * n + j];  // their gradients
        if (!tr) {
          acc += g1 * o0 - g0 * o1;
          G[r * n + i] = c * g0 + sn * g1;   // through S^T
          G[r * n + j] = -sn * g0 + c * g1;
          V[r * n + i] = c * o0 + sn * o1;   // stage input
          V[r * n + j] = -sn * o0 + c * o1;
        } else {
          acc += g0 * o1 - g1 * o0;
          G[r * n + i] = c * g0 - sn * g1;   // through S
          G[r * n + j] = sn * g0 + c * g1;
          V[r * n + i] = c * o0 - sn * o1;
          V[r * n + j] = sn * o0 + c * o1;
        }
      }
      part[s * half + p] = acc;
    }
    __syncthreads();
  }

  // ---- input gradients
  for (int q = tid; q < nr * n; q += BB_THREADS) {
    const size_t gi = size_t(r0) * n + q;
    if constexpr (ACT == ACT_BF16) {
      reinterpret_cast<uint16_t*>(a.dx)[gi] = uint16_t(pack_bf16x2(G[q], 0.f) & 0xFFFFu);
    } else {
      reinterpret_cast<float*>(a.dx)[gi] = G[q];
    }
  }
}

// dang[e] = sum over e's tiles, in tile order, of their partial rows (zero
// for an expert without rows).  Grid: (ceil(L n/2 / 256), N).
__global__ __launch_bounds__(BB_THREADS) void bfly_bwd_reduce_kernel(BflyBwdArgs a, int L) {
  const int half = 1 << (L - 1), LH = L * half, RT = a.rt;
  const int e = blockIdx.y, q = blockIdx.x * BB_THREADS + threadIdx.x;
  if (q >= LH) return;
  int nt = 0, base = 0;
  if (a.rows > 0) {
    const int off = min(max(a.offsets[e], 0), a.rows);
    const int cnt = min(max(a.offsets[e + 1], off), a.rows) - off;
    base = off / RT + e;
    nt = (cnt + RT - 1) / RT;
  }
  float s = 0.f;
  for (int j = 0; j < nt; ++j) s += a.part[size_t(base + j) * LH + q];
  a.dang[size_t(e) * LH + q] = s;
}

size_t bfly_bwd_workspace(int log2n, int n_experts, int rows) {
  const int rt = bfly_bwd_tile_rows(log2n);
  const size_t tiles = rows > 0 ? size_t((rows + rt - 1) / rt + n_experts) : 0;
  return tiles * size_t(log2n) * (size_t(1) << (log2n - 1)) * sizeof(float);
}

hipError_t launch_bfly_bwd(const void* x, const void* dy, void* dx, const float* ang, const int32_t* offsets,
                           float* part, float* dang, int rows, int n_experts, int log2n, int transpose, int act,
                           hipStream_t s) {
  BflyBwdArgs a{x, dy, dx, ang, offsets, part, dang, rows, n_experts, transpose, bfly_bwd_tile_rows(log2n), 0};
  const int L = log2n, n = 1 << L;
  if (rows > 0) {
    a.n_tiles = (rows + a.rt - 1) / a.rt + n_experts;
    const size_t lds = size_t(2) * a.rt * n * sizeof(float);
    static int attr_done[2][64] = {{0}};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const void* k = act == ACT_BF16 ? (const void*)bfly_bwd_kernel<ACT_BF16> : (const void*)bfly_bwd_kernel<ACT_F32>;
    if (lds > 64 * 1024 && (dev < 0 || dev >= 64 || !attr_done[act][dev])) {
      err = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
      if (err != hipSuccess) return err;
      if (dev >= 0 && dev < 64) attr_done[act][dev] = 1;
    }
    if (act == ACT_BF16)
      hipLaunchKernelGGL(bfly_bwd_kernel<ACT_BF16>, dim3(a.n_tiles), dim3(BB_THREADS), lds, s, a, L);
    else
      hipLaunchKernelGGL(bfly_bwd_kernel<ACT_F32>, dim3(a.n_tiles), dim3(BB_THREADS), lds, s, a, L);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int LH = L * (n >> 1);
  hipLaunchKernelGGL(bfly_bwd_reduce_kernel, dim3((LH + BB_THREADS - 1) / BB_THREADS, n_experts), dim3(BB_THREADS), 0,
                     s, a, L);
  return hipGetLastError();
}

}  // namespace bmoe
