// Butterfly rotations of token rows (ButterflyMoE, gist.science/zh/paper/2601.13563,
// technical summary §2.2: each expert's rotations are hierarchical Givens
// rotations and permutations; §2.1: inference rotates the input, multiplies by
// the ternary substrate, rotates the output, without materialising the expert).
//
// One workgroup owns a tile of rows that all belong to one expert (rows are
// bucketed by expert beforehand), so each of the expert's angles is turned
// into (cos, sin) once per tile and reused for every row of the tile.
//
// The row width n = 2^L is a template parameter: pass structure, tile height,
// table layout and every LDS offset are compile-time constants.
//
// The tile lives in LDS as fp32, 8 padding floats after every 64 elements.
// The L stages are applied in passes of up to three consecutive stages
// (stages 3P .. 3P+2): in a pass every thread holds the 2^m elements of one
// closed group (indices that differ only in the pass's stage bits) in
// registers, applies the m stages there and writes the group back.  Within a
// group the elements sit at a fixed stride, so the LDS accesses use immediate
// offsets; the stride-1 pass reads and writes its 8 contiguous floats as two
// 16-byte accesses.
//
// (cos, sin): every angle is converted once per tile by one thread into an LDS
// table laid out group-major (the pairs one group needs are contiguous).
// Widths up to 1024 hold the whole table; width 2048 one pass at a time (angles
// prefetched into registers); wider rows (the FFN hidden width) convert each
// group's angles in the registers of the thread that owns the group.
#pragma once
#include "common.hpp"

namespace bmoe {

constexpr int BF_THREADS = 256;
constexpr float kInv2Pi = 0.15915494309189535f;
enum TabMode { TAB_NONE = 0, TAB_PASS = 1, TAB_FULL = 2 };

template <int L>
struct BflyCfg {
  static constexpr int n = 1 << L;
  static constexpr int half = n / 2;
  static constexpr int stride = n + (n >> 3);
  static constexpr int NP = (L + 2) / 3;
  static constexpr int TM = L <= 10 ? TAB_FULL : (L == 11 ? TAB_PASS : TAB_NONE);
  // tile rows: at least two workgroups per CU (160 KiB LDS) up to n = 2048
  static constexpr int RT = L <= 8 ? 32 : L == 9 ? 16 : L == 10 ? 8 : L == 11 ? 5 : L == 12 ? 8 : 4;
  static constexpr size_t tile_floats = size_t(RT) * stride;
  static constexpr size_t tab_float2 = TM == TAB_FULL ? size_t(L) * half : TM == TAB_PASS ? size_t(3) * half : 0;
  static constexpr size_t lds_bytes = tile_floats * 4 + tab_float2 * 8;
};

// padded position of element i in a tile row
__device__ __forceinline__ int pos(int i) { return i + ((i >> 6) << 3); }

// distance between consecutive elements of a group in a pass starting at stage S0
template <int S0>
constexpr int elem_off() { return S0 == 0 ? 1 : S0 == 3 ? 8 : (1 << S0) + (1 << (S0 - 3)); }

// erf from the rational approximation 7.1.26 of Abramowitz & Stegun's Handbook
// of Mathematical Functions (|error| <= 1.5e-7 for all z):
//   erf(|z|) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2),  t = 1 / (1 + p |z|)
// with one hardware reciprocal and one hardware exp2 and no branch, odd in z.
__device__ __forceinline__ float erf_as(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, az, 1.0f));
  float q = fmaf(t, 1.061405429f, -1.453152027f);
  q = fmaf(t, q, 1.421413741f);
  q = fmaf(t, q, -0.284496736f);
  q = fmaf(t, q, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * az * az);
  return copysignf(fmaf(-q * t, e, 1.0f), z);
}

// GELU with the exact (erf) form, h Phi(h) = h (1 + erf(h / sqrt 2)) / 2,
// written as relu(h) - |h| Q(|h|) with Q(a) = Phi(-a) the upper normal tail
// (no cancellation on either side).  log2 Q is smooth, so it is a degree-7
// polynomial in a = min(|h|, 5.75) (a minimax fit of log2 Q on [0, 5.75],
// printed by gelu_tail_fit.py beside this file; Q's relative error is below
// 6e-6 in fp32, GELU's absolute error below 1e-6 |h| + 1e-6).  Past 5.75 the
// tail term is under 3e-8 and is kept at Q(5.75) * 5.75.  One exp2 and seven
// FMAs instead of a reciprocal, an exp2 and the A&S polynomial; the FFN middle
// passes are bound by this arithmetic.  NaN and +inf pass through.
__device__ __forceinline__ float gelu_erf(float h) {
  const float a = __builtin_amdgcn_fmed3f(fabsf(h), 0.0f, 5.75f);  // min(|h|, 5.75), one instruction
  float p = -1.825512868e-06f;
  p = fmaf(p, a, 6.144048530e-05f);
  p = fmaf(p, a, -9.294924675e-04f);
  p = fmaf(p, a, 8.504617028e-03f);
  p = fmaf(p, a, -5.395488441e-02f);
  p = fmaf(p, a, -4.584681690e-01f);
  p = fmaf(p, a, -1.151250005e+00f);
  p = fmaf(p, a, -9.999953508e-01f);
  const float q = __builtin_amdgcn_exp2f(p);
  return fmaf(0.5f, h + fabsf(h), -a * q);
}

// cos and sin with the hardware transcendental unit (angle in revolutions)
__device__ __forceinline__ float2 sincos_rev(float a) {
  const float r = a * kInv2Pi;
  return make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
}

__device__ __forceinline__ int group_base(int g, int s0, int m) {
  return (g & ((1 << s0) - 1)) | ((g >> s0) << (s0 + m));
}

// Position in a group-major (cos, sin) table of angle p of stage s
// (pass P = s / 3 with m stages starting at s0 = 3P; tables start at s0 * n/2
// in the full table, at 0 in a one-pass table).
__device__ __forceinline__ int table_slot(int s, int p, int L, bool full) {
  const int P = s / 3;
  const int s0 = 3 * P;
  const int m = min(3, L - s0);
  const int k = s - s0;
  const int i = ((p >> s) << (s + 1)) | (p & ((1 << s) - 1));  // lower index of the pair
  const int g = (i & ((1 << s0) - 1)) | ((i >> (s0 + m)) << s0);
  const int e = (i >> s0) & ((1 << m) - 1);
  const int q = ((e >> (k + 1)) << k) | (e & ((1 << k) - 1));
  const int pp = 1 << (m - 1);
  return (full ? s0 * (1 << (L - 1)) : 0) + g * (m * pp) + k * pp + q;
}

// Rotate the values of one group: stages k = 0..M-1 of the pass; cs[k*P + q]
// is the (cos, sin) of pair q of stage k.
template <int M, bool TRANS>
__device__ __forceinline__ void rotate_group(float* v, const float2* cs) {
  constexpr int P = 1 << (M - 1);
  if constexpr (!TRANS) {
#pragma unroll
    for (int k = 0; k < M; ++k)
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int e = ((q >> k) << (k + 1)) | (q & ((1 << k) - 1));
        const int f = e + (1 << k);
        const float a = v[e], b = v[f], c = cs[k * P + q].x, s = cs[k * P + q].y;
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
        const float a = v[e], b = v[f], c = cs[k * P + q].x, s = cs[k * P + q].y;
        v[e] = c * a + s * b;
        v[f] = c * b - s * a;
      }
  }
}

// One pass (stages 3P .. 3P+M-1) over rows [0, nr) of the tile.  TMODE picks
// where (cos, sin) come from (default: the width's own table mode).
template <int L, int P, bool TRANS, bool POST_GELU, int TMODE = BflyCfg<L>::TM>
__device__ __forceinline__ void bfly_pass(float* __restrict__ tile, int nr, const float2* __restrict__ tab,
                                          const float* __restrict__ ang) {
  using C = BflyCfg<L>;
  constexpr int S0 = 3 * P;
  constexpr int M = (L - S0) < 3 ? (L - S0) : 3;
  constexpr int E = 1 << M, PP = E / 2, NCS = M * PP;
  constexpr int G = C::n >> M;
  constexpr int OFF = elem_off<S0>();
  constexpr int TPG = G >= BF_THREADS ? 1 : BF_THREADS / G;   // threads per group
  constexpr int GPT = G >= BF_THREADS ? G / BF_THREADS : 1;   // groups per thread
  constexpr bool VEC = (S0 == 0 && M == 3 && (C::stride % 4) == 0);
  const int tid = threadIdx.x;
  const int gsub = G >= BF_THREADS ? tid : (tid & (G - 1));
  const int r0 = G >= BF_THREADS ? 0 : tid / G;
#pragma unroll
  for (int gi = 0; gi < GPT; ++gi) {
    const int g = gsub + gi * BF_THREADS;
    const int base = group_base(g, S0, M);
    float2 cs[NCS];
    if constexpr (TMODE != TAB_NONE) {
      const float2* t = tab + (TMODE == TAB_FULL ? S0 * C::half : 0) + g * NCS;
      if constexpr ((NCS % 2) == 0) {
#pragma unroll
        for (int j = 0; j < NCS / 2; ++j) {
          const float4 w = reinterpret_cast<const float4*>(t)[j];
          cs[2 * j] = make_float2(w.x, w.y);
          cs[2 * j + 1] = make_float2(w.z, w.w);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NCS; ++j) cs[j] = t[j];
      }
    } else {
#pragma unroll
      for (int k = 0; k < M; ++k) {
        const int s = S0 + k;
#pragma unroll
        for (int q = 0; q < PP; ++q) {
          const int e = ((q >> k) << (k + 1)) | (q & ((1 << k) - 1));
          const int i = base + (e << S0);
          const int p = ((i >> (s + 1)) << s) | (i & ((1 << s) - 1));
          cs[k * PP + q] = sincos_rev(ang[s * C::half + p]);
        }
      }
    }
    float* gp = tile + pos(base);
    for (int r = r0; r < nr; r += TPG) {
      float* rp = gp + r * C::stride;
      float v[E];
      if constexpr (VEC) {
        const float4 x0 = reinterpret_cast<const float4*>(rp)[0];
        const float4 x1 = reinterpret_cast<const float4*>(rp)[1];
        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = rp[e * OFF];
      }
      rotate_group<M, TRANS>(v, cs);
      if constexpr (POST_GELU) {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = gelu_erf(v[e]);
      }
      if constexpr (VEC) {
        reinterpret_cast<float4*>(rp)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4*>(rp)[1] = make_float4(v[4], v[5], v[6], v[7]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) rp[e * OFF] = v[e];
      }
    }
  }
}

// Whole group-major (cos, sin) table of one butterfly, loads issued first.
template <int L>
__device__ __forceinline__ void fill_full_table(float2* tab, const float* __restrict__ ang) {
  using C = BflyCfg<L>;
  constexpr int TOTAL = L * C::half;
  constexpr int PER = (TOTAL + BF_THREADS - 1) / BF_THREADS;
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int idx = threadIdx.x + BF_THREADS * j;
    if (idx < TOTAL) v[j] = ang[idx];
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int idx = threadIdx.x + BF_THREADS * j;
    if (idx < TOTAL) tab[table_slot(idx >> (L - 1), idx & (C::half - 1), L, true)] = sincos_rev(v[j]);
  }
}

// Angles of one butterfly held in registers (one-pass-table mode).
template <int L, int TMODE = BflyCfg<L>::TM>
struct AngleRegs {
  float a[TMODE == TAB_PASS ? (L * BflyCfg<L>::half + BF_THREADS - 1) / BF_THREADS : 1];
};

template <int L, int TMODE>
__device__ __forceinline__ void load_angle_regs(AngleRegs<L, TMODE>& R, const float* __restrict__ ang) {
  constexpr int TOTAL = L * BflyCfg<L>::half;
  constexpr int PER = (TOTAL + BF_THREADS - 1) / BF_THREADS;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int idx = threadIdx.x + BF_THREADS * j;
    if (idx < TOTAL) R.a[j] = ang[idx];
  }
}

template <int L, int TMODE>
__device__ __forceinline__ void fill_pass_table(float2* tab, const AngleRegs<L, TMODE>& R, int P) {
  constexpr int TOTAL = L * BflyCfg<L>::half;
  constexpr int PER = (TOTAL + BF_THREADS - 1) / BF_THREADS;
  const int s_lo = 3 * P, s_hi = min(3 * P + 3, L);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int idx = threadIdx.x + BF_THREADS * j;
    const int s = idx >> (L - 1);
    if (idx < TOTAL && s >= s_lo && s < s_hi)
      tab[table_slot(s, idx & (BflyCfg<L>::half - 1), L, false)] = sincos_rev(R.a[j]);
  }
}

// Passes T = 0 .. NP-1 of one butterfly (forward: P = T; transposed: P = NP-1-T).
template <int L, bool TRANS, bool GELU_LAST, int T = 0, int TMODE = BflyCfg<L>::TM>
__device__ __forceinline__ void run_passes(float* tile, int nr, float2* tab, const float* ang,
                                           const AngleRegs<L, TMODE>& R) {
  using C = BflyCfg<L>;
  if constexpr (T < C::NP) {
    constexpr int P = TRANS ? C::NP - 1 - T : T;
    if constexpr (TMODE == TAB_PASS) {
      fill_pass_table<L, TMODE>(tab, R, P);
      __syncthreads();
    }
    bfly_pass<L, P, TRANS, GELU_LAST && (T == C::NP - 1), TMODE>(tile, nr, tab, ang);
    __syncthreads();
    run_passes<L, TRANS, GELU_LAST, T + 1, TMODE>(tile, nr, tab, ang, R);
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

// Modes:
//   DBG  rows in -> rows out, one shared angle set (test hook)
//   IN   gather x[token of bucket row q] -> B(theta_e)^T -> U[q]
//   MID  H[q] -> B(phi_up,e) -> GELU -> B(theta_dn,e)^T -> A[q] (in place)
//   OUT  Z[q] -> B(phi_e) -> * gate -> Y[slot of q]
template <int MODE, int ACT, bool DBG_TRANS, int L>
__global__ __launch_bounds__(BF_THREADS) void bfly_kernel(BflyArgs a) {
  using C = BflyCfg<L>;
  constexpr int n = C::n;
  constexpr int RT = C::RT;
  constexpr int angs = L * C::half;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int s_info[3];
  __shared__ int s_tmp[4];
  __shared__ size_t s_src[RT], s_dst[RT];
  __shared__ float s_gate[RT];
  float* tile = smem;
  float2* tab = reinterpret_cast<float2*>(smem + C::tile_floats);
  const int tid = threadIdx.x;
  const int t = blockIdx.x;

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
  AngleRegs<L> R;
  if constexpr (C::TM == TAB_PASS) load_angle_regs<L>(R, ang0);
  if constexpr (C::TM == TAB_FULL) fill_full_table<L>(tab, ang0);

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

  // ---- prologue: rows -> fp32 tile; each thread's loads are issued together
  constexpr int CPR = n / 8;                     // 8-element chunks per row
  constexpr int CPT = (RT * CPR + BF_THREADS - 1) / BF_THREADS;  // chunks per thread
  constexpr bool VST = (C::stride % 4) == 0;
  constexpr int BATCH = CPT < 8 ? CPT : 8;
  for (int c0 = 0; c0 < CPT; c0 += BATCH) {
    float v[BATCH][8];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int c = (c0 + b) * BF_THREADS + tid;
      const int r = c / CPR;
      if (r < nr) load8<ACT>(a.in, s_src[r] + (c % CPR) * 8, v[b]);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int c = (c0 + b) * BF_THREADS + tid;
      const int r = c / CPR;
      if (r < nr) {
        float* d = tile + r * C::stride + pos((c % CPR) * 8);
        if constexpr (VST) {
          reinterpret_cast<float4*>(d)[0] = make_float4(v[b][0], v[b][1], v[b][2], v[b][3]);
          reinterpret_cast<float4*>(d)[1] = make_float4(v[b][4], v[b][5], v[b][6], v[b][7]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) d[j] = v[b][j];
        }
      }
    }
  }
  __syncthreads();

  // ---- rotations
  if constexpr (MODE == BFLY_DBG || MODE == BFLY_ROT) {
    run_passes<L, DBG_TRANS, false>(tile, nr, tab, ang0, R);
  } else if constexpr (MODE == BFLY_IN) {
    run_passes<L, true, false>(tile, nr, tab, ang0, R);
  } else if constexpr (MODE == BFLY_MID) {
    if (a.gelu) run_passes<L, false, true>(tile, nr, tab, ang0, R);
    else run_passes<L, false, false>(tile, nr, tab, ang0, R);
    const float* ang1 = a.ang1 + size_t(e) * angs;
    if constexpr (C::TM == TAB_PASS) load_angle_regs<L>(R, ang1);
    if constexpr (C::TM == TAB_FULL) {
      fill_full_table<L>(tab, ang1);  // the last pass ended with a barrier
      __syncthreads();
    }
    run_passes<L, true, false>(tile, nr, tab, ang1, R);
  } else {
    run_passes<L, false, false>(tile, nr, tab, ang0, R);
  }

  // ---- epilogue: fp32 tile -> rows
#pragma unroll
  for (int cc = 0; cc < CPT; ++cc) {
    const int c = cc * BF_THREADS + tid;
    const int r = c / CPR;
    if (r < nr) {
      const float* sp = tile + r * C::stride + pos((c % CPR) * 8);
      float v[8];
      if constexpr (VST) {
        const float4 x0 = reinterpret_cast<const float4*>(sp)[0];
        const float4 x1 = reinterpret_cast<const float4*>(sp)[1];
        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = sp[j];
      }
      if constexpr (MODE == BFLY_OUT) {
        const float g = s_gate[r];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] *= g;
      }
      store8<ACT>(a.out, s_dst[r] + (c % CPR) * 8, v);
    }
  }
}

template <int MODE, int ACT, bool TR, int L>
hipError_t launch_bfly_L(const BflyArgs& a, hipStream_t s) {
  using C = BflyCfg<L>;
  int grid = (a.rows + C::RT - 1) / C::RT;
  if (MODE != BFLY_DBG) grid += a.n_experts;
  if (grid == 0) return hipSuccess;
  auto k = bfly_kernel<MODE, ACT, TR, L>;
  const hipError_t err = allow_dynamic_lds((const void*)k, C::lds_bytes);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k, dim3(grid), dim3(BF_THREADS), C::lds_bytes, s, a);
  return hipGetLastError();
}

// Dispatch on the row width for one mode; log2n in [LO, 13].
template <int MODE, int ACT, bool TR, int LO>
hipError_t launch_bfly_width(const BflyArgs& a, int log2n, hipStream_t s) {
  switch (log2n) {
#define BMOE_BF_CASE(LL) \
  case LL:               \
    if constexpr (LL >= LO) return launch_bfly_L<MODE, ACT, TR, LL>(a, s); \
    break;
    BMOE_BF_CASE(3) BMOE_BF_CASE(4) BMOE_BF_CASE(5) BMOE_BF_CASE(6) BMOE_BF_CASE(7)
    BMOE_BF_CASE(8) BMOE_BF_CASE(9) BMOE_BF_CASE(10) BMOE_BF_CASE(11) BMOE_BF_CASE(12)
    BMOE_BF_CASE(13)
#undef BMOE_BF_CASE
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bfly_dbg(const BflyArgs& a, int act, int log2n, hipStream_t s);
hipError_t launch_bfly_in(const BflyArgs& a, int act, int log2n, hipStream_t s);
hipError_t launch_bfly_rot(const BflyArgs& a, int act, int log2n, bool transpose, hipStream_t s);
hipError_t launch_bfly_mid(const BflyArgs& a, int act, int log2n, hipStream_t s);
hipError_t launch_bfly_out(const BflyArgs& a, int act, int log2n, hipStream_t s);

}  // namespace bmoe
