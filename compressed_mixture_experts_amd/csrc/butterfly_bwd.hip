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
// So a workgroup holds a tile of one expert's rows in LDS (fp32), runs the
// forward stages on them, then walks the stages back: each thread owns whole
// pairs of the stage, and for every row of the tile adds the pair's angle
// gradient (dy_a d a'/dt + dy_b d b'/dt), turns the pair's gradient back
// through the stage and the pair's values back to the stage input.
//
// Work split: a workgroup takes a chunk of up to CH consecutive rows of one
// expert and runs it through LDS RT = min(64, 16384 / n) rows at a time (the
// two fp32 tiles fit 128 KiB).  Each thread owns the same pairs of every stage
// for the whole chunk (up to four per stage: n/2 threads, at least 256 and at
// most 1024) and keeps their angle gradients in registers, so a chunk leaves
// one partial row; a second kernel sums each expert's partial rows in chunk
// order (the result does not depend on scheduling).  CH is a multiple of RT,
// at most 256 rows, as large as still gives about two chunks per CU
// (bfly_bwd_chunk).  Expert e's chunks are indices floor(off_e / CH) + e + j,
// j < ceil(cnt_e / CH) (at most one unused index between two experts), so the
// grid and the partial buffer have ceil(R / CH) + N entries.  (cos, sin) come
// from the hardware transcendental unit (~1e-6 error, as in the forward
// passes); each stage's angles are loaded during the stage before.
#include "common.hpp"

namespace bmoe {

constexpr int bb_threads(int L) { return L <= 9 ? 256 : L == 10 ? 512 : 1024; }

static int bb_tile_rows(int log2n) {
  const int rt = 16384 >> log2n;
  return rt > 64 ? 64 : rt;
}

// rows per chunk for `rows` routed rows at width 2^log2n
static int bfly_bwd_chunk(int log2n, int rows) {
  const int rt = bb_tile_rows(log2n);
  int k = rows / (rt * 512);  // about 512 chunks: two per CU
  const int kmax = 256 / rt > 0 ? 256 / rt : 1;
  k = k < 1 ? 1 : k > kmax ? kmax : k;
  return rt * k;
}

struct BflyBwdArgs {
  const void* x;          // [R][n] rows, bucketed by expert
  const void* dy;         // [R][n]
  void* dx;               // [R][n]
  const float* ang;       // [N][L][n/2]
  const int32_t* offsets; // [N+1]
  float* part;            // [n_chunks][L][n/2] per-chunk angle gradients
  float* dang;            // [N][L][n/2]
  int32_t rows, n_experts, transpose, rt, chunk, n_chunks;
};

// lower index of pair p in stage s
__device__ __forceinline__ int pair_lo(int p, int s) { return ((p >> s) << (s + 1)) | (p & ((1 << s) - 1)); }

__device__ __forceinline__ float2 bb_sincos(float a) {
  const float r = a * 0.15915494309189535f;  // revolutions
  return make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
}

// clamped row range of expert e
__device__ __forceinline__ void bb_range(const BflyBwdArgs& a, int e, int& off, int& cnt) {
  off = min(max(a.offsets[e], 0), a.rows);
  cnt = min(max(a.offsets[e + 1], off), a.rows) - off;
}

template <int L, int ACT>
__global__ __launch_bounds__(bb_threads(L)) void bfly_bwd_kernel(BflyBwdArgs a) {
  constexpr int NT = bb_threads(L), n = 1 << L, half = n / 2;
  constexpr int PPT = half > NT ? half / NT : 1;  // pairs per thread per stage
  extern __shared__ __attribute__((aligned(16))) float tile[];  // V [RT][n], then G [RT][n]
  __shared__ int s_info[3];
  const int tid = threadIdx.x, RT = a.rt, CH = a.chunk;
  float* V = tile;
  float* G = tile + size_t(RT) * n;

  // ---- this chunk's expert and rows (experts are at most 256)
  if (tid == 0) s_info[0] = -1;
  __syncthreads();
  for (int e = tid; e < a.n_experts; e += NT) {
    int off, cnt;
    bb_range(a, e, off, cnt);
    const int base = off / CH + e, nt = (cnt + CH - 1) / CH, b = blockIdx.x;
    if (b >= base && b < base + nt) {
      s_info[0] = e;
      s_info[1] = off + (b - base) * CH;
      s_info[2] = min(CH, cnt - (b - base) * CH);
    }
  }
  __syncthreads();
  const int e = s_info[0];
  if (e < 0) return;
  const int c0 = s_info[1], ccnt = s_info[2];
  const float* ang = a.ang + size_t(e) * L * half;
  const bool tr = a.transpose != 0;
  auto stage_of = [&](int kk) { return tr ? L - 1 - kk : kk; };  // kk-th stage applied
  auto load_angles = [&](int s, float (&an)[PPT]) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = tid + k * NT;
      an[k] = p < half ? ang[s * half + p] : 0.f;
    }
  };

  float acc[L][PPT];
#pragma unroll
  for (int s = 0; s < L; ++s)
#pragma unroll
    for (int k = 0; k < PPT; ++k) acc[s][k] = 0.f;

  for (int t0 = 0; t0 < ccnt; t0 += RT) {
    const int r0 = c0 + t0, nr = min(RT, ccnt - t0);
    float an[PPT];
    load_angles(stage_of(0), an);
    // ---- rows -> LDS
    for (int q = tid; q < nr * n; q += NT) {
      const size_t gi = size_t(r0) * n + q;
      V[q] = load1<ACT>(a.x, gi);
      G[q] = load1<ACT>(a.dy, gi);
    }
    __syncthreads();
    // ---- forward stages: B applies stage 0 first, B^T stage L-1 first
#pragma unroll
    for (int kk = 0; kk < L; ++kk) {
      const int s = stage_of(kk);
      float ac[PPT];
#pragma unroll
      for (int k = 0; k < PPT; ++k) ac[k] = an[k];
      load_angles(stage_of(kk + 1 < L ? kk + 1 : L - 1), an);  // next stage (backward's first at the end)
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const int p = tid + k * NT;
        if (p < half) {
          const int i = pair_lo(p, s), j = i + (1 << s);
          const float2 cs = bb_sincos(ac[k]);
          for (int r = 0; r < nr; ++r) {
            const float x0 = V[r * n + i], x1 = V[r * n + j];
            V[r * n + i] = tr ? cs.x * x0 + cs.y * x1 : cs.x * x0 - cs.y * x1;
            V[r * n + j] = tr ? -cs.y * x0 + cs.x * x1 : cs.y * x0 + cs.x * x1;
          }
        }
      }
      __syncthreads();
    }
    // ---- backward: stages in the reverse order of application
#pragma unroll
    for (int kk = L - 1; kk >= 0; --kk) {
      const int s = stage_of(kk);
      float ac[PPT];
#pragma unroll
      for (int k = 0; k < PPT; ++k) ac[k] = an[k];
      if (kk > 0) load_angles(stage_of(kk - 1), an);
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const int p = tid + k * NT;
        if (p < half) {
          const int i = pair_lo(p, s), j = i + (1 << s);
          const float2 cs = bb_sincos(ac[k]);
          const float c = cs.x, sn = cs.y;
          float g = 0.f;
          for (int r = 0; r < nr; ++r) {
            const float o0 = V[r * n + i], o1 = V[r * n + j];  // stage outputs
            const float g0 = G[r * n + i], g1 = G[r * n + j];  // their gradients
            if (!tr) {
              g += g1 * o0 - g0 * o1;
              G[r * n + i] = c * g0 + sn * g1;   // through S^T
              G[r * n + j] = -sn * g0 + c * g1;
              V[r * n + i] = c * o0 + sn * o1;   // stage input
              V[r * n + j] = -sn * o0 + c * o1;
            } else {
              g += g0 * o1 - g1 * o0;
              G[r * n + i] = c * g0 - sn * g1;   // through S
              G[r * n + j] = sn * g0 + c * g1;
              V[r * n + i] = c * o0 - sn * o1;
              V[r * n + j] = sn * o0 + c * o1;
            }
          }
          acc[s][k] += g;
        }
      }
      __syncthreads();
    }
    // ---- input gradients of the sub-tile
    for (int q = tid; q < nr * n; q += NT) {
      const size_t gi = size_t(r0) * n + q;
      if constexpr (ACT == ACT_BF16) {
        reinterpret_cast<uint16_t*>(a.dx)[gi] = uint16_t(pack_bf16x2(G[q], 0.f) & 0xFFFFu);
      } else {
        reinterpret_cast<float*>(a.dx)[gi] = G[q];
      }
    }
    __syncthreads();  // the tile is reloaded next
  }

  float* part = a.part + size_t(blockIdx.x) * L * half;
#pragma unroll
  for (int s = 0; s < L; ++s)
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = tid + k * NT;
      if (p < half) part[s * half + p] = acc[s][k];
    }
}

// dang[e] = sum over e's chunks, in chunk order, of their partial rows (zero
// for an expert without rows).  Grid: (ceil(L n/2 / 256), N).
__global__ __launch_bounds__(256) void bfly_bwd_reduce_kernel(BflyBwdArgs a, int L) {
  const int half = 1 << (L - 1), LH = L * half, CH = a.chunk;
  const int e = blockIdx.y, q = blockIdx.x * 256 + threadIdx.x;
  if (q >= LH) return;
  int nt = 0, base = 0;
  if (a.rows > 0) {
    int off, cnt;
    bb_range(a, e, off, cnt);
    base = off / CH + e;
    nt = (cnt + CH - 1) / CH;
  }
  float s = 0.f;
  for (int j = 0; j < nt; ++j) s += a.part[size_t(base + j) * LH + q];
  a.dang[size_t(e) * LH + q] = s;
}

size_t bfly_bwd_workspace(int log2n, int n_experts, int rows) {
  if (rows <= 0) return 0;
  const int ch = bfly_bwd_chunk(log2n, rows);
  const size_t chunks = size_t((rows + ch - 1) / ch + n_experts);
  return chunks * size_t(log2n) * (size_t(1) << (log2n - 1)) * sizeof(float);
}

template <int L, int ACT>
static hipError_t bb_launch(const BflyBwdArgs& a, hipStream_t s) {
  const size_t lds = size_t(2) * a.rt * (1 << L) * sizeof(float);
  static int attr_done[64] = {0};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (lds > 64 * 1024 && (dev < 0 || dev >= 64 || !attr_done[dev])) {
    err = hipFuncSetAttribute((const void*)bfly_bwd_kernel<L, ACT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              int(lds));
    if (err != hipSuccess) return err;
    if (dev >= 0 && dev < 64) attr_done[dev] = 1;
  }
  hipLaunchKernelGGL((bfly_bwd_kernel<L, ACT>), dim3(a.n_chunks), dim3(bb_threads(L)), lds, s, a);
  return hipGetLastError();
}

template <int ACT>
static hipError_t bb_launch_act(const BflyBwdArgs& a, int L, hipStream_t s) {
  switch (L) {
    case 1: return bb_launch<1, ACT>(a, s);
    case 2: return bb_launch<2, ACT>(a, s);
    case 3: return bb_launch<3, ACT>(a, s);
    case 4: return bb_launch<4, ACT>(a, s);
    case 5: return bb_launch<5, ACT>(a, s);
    case 6: return bb_launch<6, ACT>(a, s);
    case 7: return bb_launch<7, ACT>(a, s);
    case 8: return bb_launch<8, ACT>(a, s);
    case 9: return bb_launch<9, ACT>(a, s);
    case 10: return bb_launch<10, ACT>(a, s);
    case 11: return bb_launch<11, ACT>(a, s);
    case 12: return bb_launch<12, ACT>(a, s);
    case 13: return bb_launch<13, ACT>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bfly_bwd(const void* x, const void* dy, void* dx, const float* ang, const int32_t* offsets,
                           float* part, float* dang, int rows, int n_experts, int log2n, int transpose, int act,
                           hipStream_t s) {
  BflyBwdArgs a{x, dy, dx, ang, offsets, part, dang, rows, n_experts, transpose, bb_tile_rows(log2n), 1, 0};
  const int L = log2n, n = 1 << L;
  if (rows > 0) {
    a.chunk = bfly_bwd_chunk(log2n, rows);
    a.n_chunks = (rows + a.chunk - 1) / a.chunk + n_experts;
    const hipError_t err = act == ACT_BF16 ? bb_launch_act<ACT_BF16>(a, L, s) : bb_launch_act<ACT_F32>(a, L, s);
    if (err != hipSuccess) return err;
  }
  const int LH = L * (n >> 1);
  hipLaunchKernelGGL(bfly_bwd_reduce_kernel, dim3((LH + 255) / 256, n_experts), dim3(256), 0, s, a, L);
  return hipGetLastError();
}

}  // namespace bmoe
