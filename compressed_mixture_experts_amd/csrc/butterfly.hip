// Butterfly rotations of token rows (ButterflyMoE, gist.science/zh/paper/2601.13563,
// technical summary §2.2: each expert's rotations are hierarchical Givens
// rotations and permutations; §2.1: inference rotates the input, multiplies by
// the ternary substrate, rotates the output, without materialising the expert).
//
// One workgroup owns a tile of rows that all belong to one expert (rows are
// bucketed by expert beforehand), so each of the expert's angles is turned
// into (cos, sin) once per tile and reused for every row of the tile.
//
// The tile lives in LDS as fp32.  The log2(n) stages are applied in passes of
// up to three consecutive stages: in a pass every thread holds the 2^m
// elements of one closed group (indices that differ only in the pass's stage
// bits) in registers, applies the m stages there and writes the group back.
// LDS layout: element i of a row sits at i ^ ((i >> 3) & 7) (low three bits
// swizzled by the next three) plus 8 padding floats every 64; with this every
// pass and the row loads/stores touch 64 distinct banks per wave access.
//
// cos/sin: each angle is converted once per tile by one thread.  Widths up to
// 1024 convert all of the expert's angles into an LDS table at kernel start;
// width 2048 builds one table per pass from angles prefetched into registers;
// wider rows (the FFN hidden width) convert the angles of each group in the
// registers of the thread that owns the group.
//
// Modes:
//   DBG  rows in -> rows out, one shared angle set (test hook)
//   IN   gather x[token of bucket row q] -> B(theta_e)^T -> U[q]
//   MID  H[q] -> B(phi_up,e) -> GELU -> B(theta_dn,e)^T -> A[q] (in place)
//   OUT  Z[q] -> B(phi_e) -> * gate -> Y[slot of q]
#include "common.hpp"

namespace bmoe {

constexpr int BF_THREADS = 256;
constexpr int BF_FULL_MAX_LOG2N = 10;  // widths up to 1024: whole (cos, sin) table in LDS
constexpr int BF_TAB_MAX_LOG2N = 11;   // width 2048: one table per pass
constexpr int BF_MAX_ANG_REGS = 44;    // (11 * 1024) / 256 angles per thread at n = 2048
enum TabMode { TAB_NONE = 0, TAB_PASS = 1, TAB_FULL = 2 };
constexpr float kInv2Pi = 0.15915494309189535f;

// swizzled + padded position of element i in a tile row
__device__ __forceinline__ int lds_pos(int i) {
  const int j = i ^ ((i >> 3) & 7);
  return j + ((j >> 6) << 3);
}

__device__ __forceinline__ float gelu_erf(float h) {
  return h * 0.5f * (1.0f + erff(h * 0.70710678118654752f));
}

// cos and sin of an angle in radians with the hardware transcendental unit
// (v_sin_f32 / v_cos_f32 take the angle in revolutions).
__device__ __forceinline__ float2 sincos_rev(float a) {
  const float r = a * kInv2Pi;
  return make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
}

int bfly_rows_per_tile(int log2n) {
  // LDS per workgroup = tile (rows x 1.125 n fp32) + (cos, sin) table; sized
  // so that at least two workgroups share a CU's 160 KiB.
  switch (log2n) {
    case 3: case 4: case 5: case 6: case 7: case 8: return 32;
    case 9: return 16;    // 36 KiB tile + 18 KiB table: 2 workgroups per CU
    case 10: return 8;    // 36 KiB tile + 40 KiB table: 2 workgroups per CU
    case 11: return 5;    // 45 KiB tile + 24 KiB pass table: 2 per CU
    case 12: return 8;
    default: return 4;
  }
}

static int bfly_tab_mode(int log2n) {
  return log2n <= BF_FULL_MAX_LOG2N ? TAB_FULL : (log2n <= BF_TAB_MAX_LOG2N ? TAB_PASS : TAB_NONE);
}

static size_t bfly_lds_bytes(int log2n) {
  const size_t n = size_t(1) << log2n;
  const size_t tile = size_t(bfly_rows_per_tile(log2n)) * (n + (n >> 3)) * sizeof(float);
  const int tm = bfly_tab_mode(log2n);
  const size_t tab = tm == TAB_FULL ? size_t(log2n) * (n / 2) * sizeof(float2)
                   : tm == TAB_PASS ? 3 * (n / 2) * sizeof(float2) : 0;
  return tile + tab;
}

// Element e of group g in a pass starting at stage s0 with m stages.
__device__ __forceinline__ int group_base(int g, int s0, int m) {
  return (g & ((1 << s0) - 1)) | ((g >> s0) << (s0 + m));
}

// Apply stages s0..s0+M-1 to the values of one group, forward (B) or transposed
// (B^T), with cos/sin cs[k][q] for stage k and pair q of the group.
template <int M, bool TRANS>
__device__ __forceinline__ void rotate_group(float* v, const float2 (&cs)[M][1 << (M - 1)]) {
  constexpr int P = 1 << (M - 1);
  if constexpr (!TRANS) {
#pragma unroll
    for (int k = 0; k < M; ++k)
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int e = ((q >> k) << (k + 1)) | (q & ((1 << k) - 1));
        const int f = e + (1 << k);
        const float a = v[e], b = v[f], c = cs[k][q].x, s = cs[k][q].y;
        v[e] = c * a - s * b;
        v[f] = s * a + c * b;
      }
  } else {
#pragma unroll
    for (int k = M - 1; k >= 0; --k)
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int e = ((q >> k) << (k + 1)) | (q & ((1 << k) - 1));
        const int f = e + (1 << k);
        const float a = v[e], b = v[f], c = cs[k][q].x, s = cs[k][q].y;
        v[e] = c * a + s * b;
        v[f] = c * b - s * a;
      }
  }
}

// One pass of M stages over rows [0, nr) of the tile.  TAB: cos/sin come from
// the LDS table `tab` ([M][n/2] float2, stage-relative); otherwise they are
// computed here from the global angles `ang` ([L][n/2]).
template <int M, bool TRANS, bool POST_GELU, bool TAB>
__device__ __forceinline__ void bfly_pass(float* __restrict__ tile, int stride, int n, int s0, int nr,
                                          const float2* __restrict__ tab, const float* __restrict__ ang) {
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
    const int base = group_base(g, s0, M);
    float2 cs[M][P];
#pragma unroll
    for (int k = 0; k < M; ++k) {
      const int s = s0 + k;
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int e = ((q >> k) << (k + 1)) | (q & ((1 << k) - 1));
        const int i = base + (e << s0);
        const int p = ((i >> (s + 1)) << s) | (i & ((1 << s) - 1));
        if constexpr (TAB) cs[k][q] = tab[k * half + p];
        else cs[k][q] = sincos_rev(ang[s * half + p]);
      }
    }
    int addr[E];
#pragma unroll
    for (int e = 0; e < E; ++e) addr[e] = lds_pos(base + (e << s0));
    for (int r = r0; r < nr; r += rstep) {
      float* row = tile + r * stride;
      float v[E];
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = row[addr[e]];
      rotate_group<M, TRANS>(v, cs);
      if constexpr (POST_GELU) {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = gelu_erf(v[e]);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) row[addr[e]] = v[e];
    }
  }
}

template <bool TRANS, bool POST_GELU, bool TAB>
__device__ __forceinline__ void bfly_pass_m(int m, float* tile, int stride, int n, int s0, int nr,
                                            const float2* tab, const float* ang) {
  if (m == 3) bfly_pass<3, TRANS, POST_GELU, TAB>(tile, stride, n, s0, nr, tab, ang);
  else if (m == 2) bfly_pass<2, TRANS, POST_GELU, TAB>(tile, stride, n, s0, nr, tab, ang);
  else bfly_pass<1, TRANS, POST_GELU, TAB>(tile, stride, n, s0, nr, tab, ang);
}

// Angles of one butterfly held by this thread: flat index t + 256 j of [L][n/2].
struct AngleRegs {
  float a[BF_MAX_ANG_REGS];
};

__device__ __forceinline__ void load_angles(AngleRegs& R, const float* __restrict__ ang, int total) {
#pragma unroll
  for (int j = 0; j < BF_MAX_ANG_REGS; ++j) {
    const int idx = threadIdx.x + BF_THREADS * j;
    if (idx < total) R.a[j] = ang[idx];
  }
}

// Whole (cos, sin) table of one butterfly: entry s * n/2 + p for stage s,
// pair p.  Loads are issued before any conversion.
__device__ __forceinline__ void fill_full_table(float2* tab, const float* __restrict__ ang, int total) {
  constexpr int B = 20;  // (10 * 512) / 256 angles per thread at n = 1024
  float v[B];
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const int idx = threadIdx.x + BF_THREADS * j;
    if (idx < total) v[j] = ang[idx];
  }
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const int idx = threadIdx.x + BF_THREADS * j;
    if (idx < total) tab[idx] = sincos_rev(v[j]);
  }
}

// All L stages of one butterfly over the tile; passes of three stages.
// Forward (B v): stage 0 first.  Transposed (B^T v): stage L-1 first.
template <bool TRANS, int TM>
__device__ void bfly_all(float* tile, int stride, int L, int nr, const float* ang, const AngleRegs& R,
                         float2* tab, bool post_gelu) {
  const int n = 1 << L;
  const int half = n >> 1;
  const int np = (L + 2) / 3;
  for (int t = 0; t < np; ++t) {
    const int P = TRANS ? (np - 1 - t) : t;
    const int s0 = 3 * P;
    const int m = (L - s0) < 3 ? (L - s0) : 3;
    const float2* ptab = tab;
    if constexpr (TM == TAB_PASS) {
      // this pass's (cos, sin) table from the prefetched angles
      const int lo = s0 * half, hi = (s0 + m) * half;
#pragma unroll
      for (int j = 0; j < BF_MAX_ANG_REGS; ++j) {
        const int idx = threadIdx.x + BF_THREADS * j;
        if (idx >= lo && idx < hi) tab[idx - lo] = sincos_rev(R.a[j]);
      }
      __syncthreads();
    } else if constexpr (TM == TAB_FULL) {
      ptab = tab + s0 * half;
    }
    constexpr bool TB = TM != TAB_NONE;
    const bool last = (t == np - 1);
    if (post_gelu && last) bfly_pass_m<TRANS, true, TB>(m, tile, stride, n, s0, nr, ptab, ang);
    else bfly_pass_m<TRANS, false, TB>(m, tile, stride, n, s0, nr, ptab, ang);
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

template <int MODE, int ACT, bool DBG_TRANS, int TM>
__global__ __launch_bounds__(BF_THREADS) void bfly_kernel(BflyArgs a, int L, int RT) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int s_info[3];
  __shared__ int s_tmp[4];
  __shared__ size_t s_src[32], s_dst[32];
  __shared__ float s_gate[32];
  const int n = 1 << L;
  const int stride = n + (n >> 3);
  float* tile = smem;
  float2* tab = reinterpret_cast<float2*>(smem + size_t(RT) * stride);
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const int angs = L * (n >> 1);

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

  const float* ang0 = a.ang0 + size_t(e) * angs;
  AngleRegs R;
  if constexpr (TM == TAB_PASS) load_angles(R, ang0, angs);
  if constexpr (TM == TAB_FULL) fill_full_table(tab, ang0, angs);

  // source / destination rows of the tile
  if (tid < nr) {
    const int q = r0 + tid;
    if constexpr (MODE == BFLY_IN) {
      const int slot = a.perm[q];
      s_src[tid] = size_t(slot / a.top_k) * n;
      s_dst[tid] = size_t(q) * n;
    } else if constexpr (MODE == BFLY_OUT) {
      const int slot = a.perm[q];
      s_src[tid] = size_t(q) * n;
      s_dst[tid] = size_t(slot) * n;
      s_gate[tid] = a.gate[slot];
    } else {
      s_src[tid] = size_t(q) * n;
      s_dst[tid] = size_t(q) * n;
    }
  }
  __syncthreads();

  // ---- prologue: rows -> fp32 tile.  Loads are issued in batches of eight
  // chunks per thread before any is used, so their latencies overlap.
  const int cpr = n >> 3;  // 8-element chunks per row
  const int nch = nr * cpr;
  for (int c0 = 0; c0 < nch; c0 += 8 * BF_THREADS) {
    float v[8][8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int c = c0 + b * BF_THREADS + tid;
      if (c < nch) {
        const int r = c / cpr;
        load8<ACT>(a.in, s_src[r] + ((c - r * cpr) << 3), v[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int c = c0 + b * BF_THREADS + tid;
      if (c < nch) {
        const int r = c / cpr;
        const int col = (c - r * cpr) << 3;
        float* dst = tile + r * stride;
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[lds_pos(col + j)] = v[b][j];
      }
    }
  }
  __syncthreads();

  // ---- rotations
  if constexpr (MODE == BFLY_DBG) {
    bfly_all<DBG_TRANS, TM>(tile, stride, L, nr, ang0, R, tab, false);
  } else if constexpr (MODE == BFLY_IN) {
    bfly_all<true, TM>(tile, stride, L, nr, ang0, R, tab, false);
  } else if constexpr (MODE == BFLY_MID) {
    bfly_all<false, TM>(tile, stride, L, nr, ang0, R, tab, a.gelu != 0);
    const float* ang1 = a.ang1 + size_t(e) * angs;
    if constexpr (TM == TAB_PASS) load_angles(R, ang1, angs);
    if constexpr (TM == TAB_FULL) {
      fill_full_table(tab, ang1, angs);  // the last pass ended with a barrier
      __syncthreads();
    }
    bfly_all<true, TM>(tile, stride, L, nr, ang1, R, tab, false);
  } else {
    bfly_all<false, TM>(tile, stride, L, nr, ang0, R, tab, false);
  }

  // ---- epilogue: fp32 tile -> rows
  for (int c = tid; c < nch; c += BF_THREADS) {
    const int r = c / cpr;
    const int col = (c - r * cpr) << 3;
    const float* srcp = tile + r * stride;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = srcp[lds_pos(col + j)];
    if constexpr (MODE == BFLY_OUT) {
      const float g = s_gate[r];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] *= g;
    }
    store8<ACT>(a.out, s_dst[r] + col, v);
  }
}

template <int MODE, int ACT, bool TR, int TM>
static hipError_t launch_one(const BflyArgs& a, int log2n, hipStream_t s) {
  const int RT = bfly_rows_per_tile(log2n);
  const size_t lds = bfly_lds_bytes(log2n);
  int grid = (a.rows + RT - 1) / RT;
  if (MODE != BFLY_DBG) grid += a.n_experts;
  if (grid == 0) return hipSuccess;
  auto k = bfly_kernel<MODE, ACT, TR, TM>;
  static int attr_done[64] = {0};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64 || !attr_done[dev]) {
    size_t mx = 0;
    for (int l = 3; l <= 13; ++l) mx = bfly_lds_bytes(l) > mx ? bfly_lds_bytes(l) : mx;
    err = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, int(mx));
    if (err != hipSuccess) return err;
    if (dev >= 0 && dev < 64) attr_done[dev] = 1;
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(BF_THREADS), lds, s, a, log2n, RT);
  return hipGetLastError();
}

template <int MODE, int ACT, bool TR>
static hipError_t launch_tm(const BflyArgs& a, int log2n, hipStream_t s) {
  switch (bfly_tab_mode(log2n)) {
    case TAB_FULL: return launch_one<MODE, ACT, TR, TAB_FULL>(a, log2n, s);
    case TAB_PASS: return launch_one<MODE, ACT, TR, TAB_PASS>(a, log2n, s);
    default: return launch_one<MODE, ACT, TR, TAB_NONE>(a, log2n, s);
  }
}

template <int MODE, bool TR>
static hipError_t launch_mode(const BflyArgs& a, int act, int log2n, hipStream_t s) {
  if (act == ACT_BF16) return launch_tm<MODE, ACT_BF16, TR>(a, log2n, s);
  return launch_tm<MODE, ACT_F32, TR>(a, log2n, s);
}

hipError_t launch_butterfly(const BflyArgs& a, int mode, int act, int log2n, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  switch (mode) {
    case BFLY_DBG:
      return a.transpose ? launch_mode<BFLY_DBG, true>(a, act, log2n, s)
                         : launch_mode<BFLY_DBG, false>(a, act, log2n, s);
    case BFLY_IN: return launch_mode<BFLY_IN, false>(a, act, log2n, s);
    case BFLY_MID: return launch_mode<BFLY_MID, false>(a, act, log2n, s);
    default: return launch_mode<BFLY_OUT, false>(a, act, log2n, s);
  }
}

}  // namespace bmoe
