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
// expert and runs it through LDS RT rows at a time: min(64, 8192 / n) up to
// width 512 (the two fp32 tiles fit 64 KiB, two 256-thread workgroups per
// CU), 16384 / n for widths 1024 and 2048 (128 KiB).  Each thread owns the same pairs of every stage
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
//
// Widths 4096 and 8192 (L = S + 4, S = 8 or 9) would leave a few rows per LDS
// tile and too many angle sums per thread, so they run in the forward's two
// parts: the low part (stages 0 .. S-1) on chunks of 2^S consecutive
// indices and the high part (stages S .. S+3) on the 16 indices v + 2^S j of
// 64 columns v at a time, each a butterfly of its own with many rows per
// tile.  For y = high(low(x)): z = low(x) into an fp32 buffer, the high part's
// backward from (z, dy) gives dz (fp32 buffer) and the high stages' angle
// gradients, the low part's backward from (x, dz) gives dx and the low
// stages'; B^T runs high^T first, so the roles swap.  Every (chunk of rows,
// group of indices) workgroup writes the partial angle gradients of its own
// pairs, and the same reduction sums them per expert.
#include <type_traits>
#include <utility>

#include "common.hpp"

namespace bmoe {

constexpr int bb_threads(int L) { return L <= 9 ? 256 : L == 10 ? 512 : 1024; }

// rows per LDS tile: up to 64 KiB for the two fp32 tiles where a workgroup has
// 256 threads (two workgroups per CU), 128 KiB with 512 or 1024 threads
constexpr int bb_tile_rows_c(int L) {
  return L <= 9 ? ((8192 >> L) < 64 ? (8192 >> L) : 64) : (16384 >> L);
}
static int bb_tile_rows(int log2n) { return bb_tile_rows_c(log2n); }

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

// Row loops of one pair (lo, hi) over rows 0 .. nr-1 of an LDS tile with row
// stride W.  U rows at a time (8, or 4 where registers are capped at 128),
// all their loads before any store: the compiler keeps LDS loads behind
// earlier LDS stores, so a plain row loop waits a full LDS round trip per row.
// s is sin(t) for a stage of B and -sin(t) for a stage of B^T (the transposed
// stage is the rotation by -t).

// v, as a value the compiler cannot see through: LDS addresses derived from it
// inside the tile loop are recomputed per tile instead of being hoisted out of
// it and held in registers for every (stage, row) at once
__device__ __forceinline__ int bb_opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// forward: (a, b) <- (c a - s b, s a + c b)
template <int BB_U = 8>
__device__ __forceinline__ void bb_rot_rows(float* V, int W, int nr, int lo, int hi, float c, float s) {
  int r = 0;
  for (; r + BB_U <= nr; r += BB_U) {
    float x0[BB_U], x1[BB_U];
#pragma unroll
    for (int u = 0; u < BB_U; ++u) {
      x0[u] = V[(r + u) * W + lo];
      x1[u] = V[(r + u) * W + hi];
    }
#pragma unroll
    for (int u = 0; u < BB_U; ++u) {
      V[(r + u) * W + lo] = c * x0[u] - s * x1[u];
      V[(r + u) * W + hi] = s * x0[u] + c * x1[u];
    }
  }
  for (; r < nr; ++r) {
    const float x0 = V[r * W + lo], x1 = V[r * W + hi];
    V[r * W + lo] = c * x0 - s * x1;
    V[r * W + hi] = s * x0 + c * x1;
  }
}

// backward through one stage: V holds the stage's outputs and G their
// gradients; afterwards V holds its inputs and G their gradients.  Returns the
// sum over the rows of g_b a' - g_a b' (the angle gradient of a stage of B;
// its negative for a stage of B^T).
template <int BB_U = 8>
__device__ __forceinline__ float bb_back_rows(float* V, float* G, int W, int nr, int lo, int hi, float c, float s) {
  float gs = 0.f;
  int r = 0;
  for (; r + BB_U <= nr; r += BB_U) {
    float o0[BB_U], o1[BB_U], g0[BB_U], g1[BB_U];
#pragma unroll
    for (int u = 0; u < BB_U; ++u) {
      o0[u] = V[(r + u) * W + lo];
      o1[u] = V[(r + u) * W + hi];
      g0[u] = G[(r + u) * W + lo];
      g1[u] = G[(r + u) * W + hi];
    }
#pragma unroll
    for (int u = 0; u < BB_U; ++u) {
      gs += g1[u] * o0[u] - g0[u] * o1[u];
      G[(r + u) * W + lo] = c * g0[u] + s * g1[u];
      G[(r + u) * W + hi] = -s * g0[u] + c * g1[u];
      V[(r + u) * W + lo] = c * o0[u] + s * o1[u];
      V[(r + u) * W + hi] = -s * o0[u] + c * o1[u];
    }
  }
  for (; r < nr; ++r) {
    const float o0 = V[r * W + lo], o1 = V[r * W + hi];
    const float g0 = G[r * W + lo], g1 = G[r * W + hi];
    gs += g1 * o0 - g0 * o1;
    G[r * W + lo] = c * g0 + s * g1;
    G[r * W + hi] = -s * g0 + c * g1;
    V[r * W + lo] = c * o0 + s * o1;
    V[r * W + hi] = -s * o0 + c * o1;
  }
  return gs;
}

// Tiles between HBM and LDS in 16-byte vectors (8 bf16 or 4 fp32 elements):
// vector q (q = tid, tid + NT, ... < nq) is element gidx(q) of the rows and
// lidx(q) of the LDS tile (nq >= 1).  Loads go eight vectors per thread at a
// time, all issued before their LDS stores, so HBM latency is paid once per
// eight.
template <int A>
constexpr int bb_vec() { return A == ACT_BF16 ? 8 : 4; }

template <int A, int NT, int NV, class GI, class LI>
__device__ __forceinline__ void bb_load_tile(const void* src, float* T, int nq, GI gidx, LI lidx) {
  constexpr int ES = A == ACT_BF16 ? 2 : 4;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i0 = 0; i0 < NV; i0 += 8) {
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // unconditional (a vector past the tile re-reads the tile's last one), so
      // v stays in registers
      const int q = min(tid + (i0 + i) * NT, nq - 1);
      if (i0 + i < NV) v[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(src) + gidx(q) * ES);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + (i0 + i) * NT;
      if (i0 + i < NV && q < nq) {
        float* d = T + lidx(q);
        if constexpr (A == ACT_BF16) {
          const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
          float f[8];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            f[2 * k] = __uint_as_float(w[k] << 16);
            f[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
          }
          *reinterpret_cast<float4*>(d) = make_float4(f[0], f[1], f[2], f[3]);
          *reinterpret_cast<float4*>(d + 4) = make_float4(f[4], f[5], f[6], f[7]);
        } else {
          *reinterpret_cast<uint4*>(d) = v[i];
        }
      }
    }
  }
}

template <int A, int NT, int NV, class GI, class LI>
__device__ __forceinline__ void bb_store_tile(void* dst, const float* T, int nq, GI gidx, LI lidx) {
  constexpr int ES = A == ACT_BF16 ? 2 : 4;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int q = tid + i * NT;
    if (q < nq) {
      const float* src = T + lidx(q);
      uint4 o;
      if constexpr (A == ACT_BF16) {
        const float4 f0 = *reinterpret_cast<const float4*>(src);
        const float4 f1 = *reinterpret_cast<const float4*>(src + 4);
        o = make_uint4(pack_bf16x2(f0.x, f0.y), pack_bf16x2(f0.z, f0.w), pack_bf16x2(f1.x, f1.y),
                       pack_bf16x2(f1.z, f1.w));
      } else {
        o = *reinterpret_cast<const uint4*>(src);
      }
      *reinterpret_cast<uint4*>(static_cast<char*>(dst) + gidx(q) * ES) = o;
    }
  }
}

template <int L, int ACT>
__global__ __launch_bounds__(bb_threads(L), L <= 9 ? 2 : 1) void bfly_bwd_kernel(BflyBwdArgs a) {
  constexpr int NT = bb_threads(L), n = 1 << L, half = n / 2;
  constexpr int PPT = half > NT ? half / NT : 1;  // pairs per thread per stage
  constexpr int RT = bb_tile_rows_c(L);            // rows per LDS tile
  constexpr int VEC = bb_vec<ACT>();
  constexpr bool VECTOR = n >= 8;                  // tile rows start on 16-byte boundaries
  constexpr int NV = (RT * n / VEC + NT - 1) / NT; // vectors per thread per tile
  constexpr int U = NT >= 1024 ? 4 : 8;            // rows per LDS batch
  extern __shared__ __attribute__((aligned(16))) float tile[];  // V [RT][n], then G [RT][n]
  __shared__ int s_info[3];
  const int tid = threadIdx.x, CH = a.chunk;
  float* V = tile;
  float* G = tile + RT * n;

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

  // (cos, sin) of this thread's pairs, once per chunk, sin negated for B^T,
  // and their angle gradients; both indexed by the order of application kk
  // (a compile-time index once unrolled: the stage stage_of(kk) is not)
  float2 cs[L][PPT];
  float acc[L][PPT];
#pragma unroll
  for (int kk = 0; kk < L; ++kk)
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = tid + k * NT;
      const float2 v = bb_sincos(p < half ? ang[stage_of(kk) * half + p] : 0.f);
      cs[kk][k] = make_float2(v.x, tr ? -v.y : v.y);
      acc[kk][k] = 0.f;
    }

  for (int t0 = 0; t0 < ccnt; t0 += RT) {
    const int r0 = c0 + t0, nr = min(RT, ccnt - t0);
    const int ptid = bb_opaque(tid);
    // ---- rows -> LDS
    if constexpr (VECTOR) {
      const size_t base = size_t(r0) * n;
      auto gi = [&](int q) { return base + size_t(q) * VEC; };
      auto li = [&](int q) { return q * VEC; };
      bb_load_tile<ACT, NT, NV>(a.x, V, nr * n / VEC, gi, li);
      bb_load_tile<ACT, NT, NV>(a.dy, G, nr * n / VEC, gi, li);
    } else {
      for (int q = tid; q < nr * n; q += NT) {
        const size_t gi = size_t(r0) * n + q;
        V[q] = load1<ACT>(a.x, gi);
        G[q] = load1<ACT>(a.dy, gi);
      }
    }
    __syncthreads();
    // ---- forward stages: B applies stage 0 first, B^T stage L-1 first
#pragma unroll
    for (int kk = 0; kk < L; ++kk) {
      const int s = stage_of(kk);
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const int p = ptid + k * NT;
        if (p < half) {
          const int i = pair_lo(p, s), j = i + (1 << s);
          bb_rot_rows<U>(V, n, nr, i, j, cs[kk][k].x, cs[kk][k].y);
        }
      }
      __syncthreads();
    }
    // ---- backward: stages in the reverse order of application
#pragma unroll
    for (int kk = L - 1; kk >= 0; --kk) {
      const int s = stage_of(kk);
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const int p = ptid + k * NT;
        if (p < half) {
          const int i = pair_lo(p, s), j = i + (1 << s);
          const float g = bb_back_rows<U>(V, G, n, nr, i, j, cs[kk][k].x, cs[kk][k].y);
          acc[kk][k] += tr ? -g : g;
        }
      }
      __syncthreads();
    }
    // ---- input gradients of the sub-tile
    if constexpr (VECTOR) {
      const size_t base = size_t(r0) * n;
      bb_store_tile<ACT, NT, NV>(a.dx, G, nr * n / VEC, [&](int q) { return base + size_t(q) * VEC; },
                                 [&](int q) { return q * VEC; });
    } else {
      for (int q = tid; q < nr * n; q += NT) {
        const size_t gi = size_t(r0) * n + q;
        if constexpr (ACT == ACT_BF16) {
          reinterpret_cast<uint16_t*>(a.dx)[gi] = uint16_t(pack_bf16x2(G[q], 0.f) & 0xFFFFu);
        } else {
          reinterpret_cast<float*>(a.dx)[gi] = G[q];
        }
      }
    }
    __syncthreads();  // the tile is reloaded next
  }

  float* part = a.part + size_t(blockIdx.x) * L * half;
#pragma unroll
  for (int kk = 0; kk < L; ++kk)
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = tid + k * NT;
      if (p < half) part[stage_of(kk) * half + p] = acc[kk][k];
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

// ---------------------------------------------------------------- parts (L >= 12)
enum { BP_LOW = 0, BP_HIGH = 1 };

struct BflyPartArgs {
  const void* in0;        // rows the part's forward is recomputed from [R][n]
  const void* in1;        // gradient rows at the part's output [R][n] (backward)
  void* out;              // forward: part(in0); backward: gradient at the part's input
  const float* ang;       // [N][L][n/2]
  const int32_t* offsets; // [N+1]
  float* part;            // [n_chunks][L][n/2]
  int32_t rows, n_experts, transpose, chunk, n_chunks;
};

// A part as a butterfly over GW local indices of a row: LOW, chunk c: local l
// is index c 2^S + l, local stage t is stage t (MS = S stages); HIGH, columns
// v0 .. v0+63: local l = 64 jj + vl is index v0 + vl + 2^S jj, local stage t is
// stage S + t (MS = 4), with 8 local pairs per column.
template <int S, int PART>
struct BpCfg {
  static constexpr int L = S + 4, n = 1 << L, half = n / 2;
  static constexpr int GW = PART == BP_LOW ? (1 << S) : 1024;   // local indices per row
  static constexpr int MS = PART == BP_LOW ? S : 4;             // local stages
  static constexpr int NG = PART == BP_LOW ? 16 : (1 << S) / 64; // groups per row
  static constexpr int RT = 8192 / GW;                          // rows per LDS tile (64 KiB for two)
  static constexpr int NT = GW / 2 < 256 ? GW / 2 : 256;
  static constexpr int PPT = GW / 2 / NT;                       // local pairs per thread per stage
};

template <int S, int PART>
__device__ __forceinline__ int bp_global(int g, int l) {  // local index -> index in the row
  if constexpr (PART == BP_LOW) return (g << S) + l;
  else return g * 64 + (l & 63) + ((l >> 6) << S);
}
// local pair k of local stage t: its two local indices and its angle's pair number
template <int S, int PART>
__device__ __forceinline__ void bp_pair(int g, int t, int k, int& lo, int& hi, int& gp) {
  if constexpr (PART == BP_LOW) {
    lo = pair_lo(k, t);
    hi = lo + (1 << t);
    gp = (g << (S - 1)) + k;
  } else {
    const int q = k >> 6, vl = k & 63;
    const int jl = pair_lo(q, t);
    lo = jl * 64 + vl;
    hi = (jl + (1 << t)) * 64 + vl;
    gp = (q << S) + g * 64 + vl;
  }
}

// One (row chunk, index group) of a part.  BWD = 0: out = part(in0) (or its
// transpose); BWD = 1: the part's backward, out = gradient at its input.
template <int S, int PART, int A0, int A1, int AO, int BWD>
__global__ __launch_bounds__(256, 2) void bfly_part_kernel(BflyPartArgs a) {
  using C = BpCfg<S, PART>;
  constexpr int NT = C::NT, GW = C::GW, MS = C::MS, PPT = C::PPT, RT = C::RT, n = C::n, half = C::half;
  constexpr int s_base = PART == BP_LOW ? 0 : S;
  extern __shared__ __attribute__((aligned(16))) float tile[];  // V [RT][GW], then G [RT][GW]
  __shared__ int s_info[3];
  const int tid = threadIdx.x, CH = a.chunk;
  const int cb = blockIdx.x / C::NG, g = blockIdx.x % C::NG;
  float* V = tile;
  float* G = tile + RT * GW;

  if (tid == 0) s_info[0] = -1;
  __syncthreads();
  for (int e = tid; e < a.n_experts; e += NT) {
    const int off = min(max(a.offsets[e], 0), a.rows);
    const int cnt = min(max(a.offsets[e + 1], off), a.rows) - off;
    const int base = off / CH + e, nt = (cnt + CH - 1) / CH;
    if (cb >= base && cb < base + nt) {
      s_info[0] = e;
      s_info[1] = off + (cb - base) * CH;
      s_info[2] = min(CH, cnt - (cb - base) * CH);
    }
  }
  __syncthreads();
  const int e = s_info[0];
  if (e < 0) return;
  const int c0 = s_info[1], ccnt = s_info[2];
  const float* ang = a.ang + size_t(e) * (S + 4) * half;
  const bool tr = a.transpose != 0;
  auto stage_of = [&](int kk) { return tr ? MS - 1 - kk : kk; };  // kk-th local stage applied

  // (cos, sin) of this thread's pairs, once per chunk, sin negated for B^T,
  // and their angle gradients; both indexed by the order of application kk
  float2 cs[MS][PPT];
  float acc[MS][PPT];
#pragma unroll
  for (int kk = 0; kk < MS; ++kk)
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      int lo, hi, gp;
      const int t = stage_of(kk);
      bp_pair<S, PART>(g, t, tid + k * NT, lo, hi, gp);
      const float2 v = bb_sincos(ang[(s_base + t) * half + gp]);
      cs[kk][k] = make_float2(v.x, tr ? -v.y : v.y);
      acc[kk][k] = 0.f;
    }

  // tile vectors: q -> row q / PR, local index (q % PR) * VEC
  auto tile_io = [&](auto vec_c, int r0) {
    constexpr int VEC = decltype(vec_c)::value, PR = GW / VEC;
    auto gi = [=](int q) { return size_t(r0 + q / PR) * n + bp_global<S, PART>(g, (q % PR) * VEC); };
    auto li = [=](int q) { return (q / PR) * GW + (q % PR) * VEC; };
    return std::make_pair(gi, li);
  };

  for (int t0 = 0; t0 < ccnt; t0 += RT) {
    const int r0 = c0 + t0, nr = min(RT, ccnt - t0);
    const int ptid = bb_opaque(tid);
    {
      constexpr int V0 = bb_vec<A0>();
      auto io = tile_io(std::integral_constant<int, V0>(), r0);
      bb_load_tile<A0, NT, RT * GW / V0 / NT>(a.in0, V, nr * GW / V0, io.first, io.second);
    }
    if constexpr (BWD) {
      constexpr int V1 = bb_vec<A1>();
      auto io = tile_io(std::integral_constant<int, V1>(), r0);
      bb_load_tile<A1, NT, RT * GW / V1 / NT>(a.in1, G, nr * GW / V1, io.first, io.second);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < MS; ++kk) {
      const int t = stage_of(kk);
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        int lo, hi, gp;
        bp_pair<S, PART>(g, t, ptid + k * NT, lo, hi, gp);
        bb_rot_rows(V, GW, nr, lo, hi, cs[kk][k].x, cs[kk][k].y);
      }
      __syncthreads();
    }
    if constexpr (BWD) {
#pragma unroll
      for (int kk = MS - 1; kk >= 0; --kk) {
        const int t = stage_of(kk);
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
          int lo, hi, gp;
          bp_pair<S, PART>(g, t, ptid + k * NT, lo, hi, gp);
          const float gsum = bb_back_rows(V, G, GW, nr, lo, hi, cs[kk][k].x, cs[kk][k].y);
          acc[kk][k] += tr ? -gsum : gsum;
        }
        __syncthreads();
      }
    }
    {
      constexpr int VO = bb_vec<AO>();
      auto io = tile_io(std::integral_constant<int, VO>(), r0);
      bb_store_tile<AO, NT, RT * GW / VO / NT>(a.out, BWD ? G : V, nr * GW / VO, io.first, io.second);
    }
    __syncthreads();
  }

  if constexpr (BWD) {
    float* part = a.part + size_t(cb) * (S + 4) * half;
#pragma unroll
    for (int kk = 0; kk < MS; ++kk)
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        int lo, hi, gp;
        const int t = stage_of(kk);
        bp_pair<S, PART>(g, t, tid + k * NT, lo, hi, gp);
        part[(s_base + t) * half + gp] = acc[kk][k];
      }
  }
}

template <int S, int PART, int A0, int A1, int AO, int BWD>
static hipError_t bp_launch(const BflyPartArgs& a, hipStream_t s) {
  using C = BpCfg<S, PART>;
  const size_t lds = size_t(BWD ? 2 : 1) * C::RT * C::GW * sizeof(float);
  static int attr_done[64] = {0};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  auto k = bfly_part_kernel<S, PART, A0, A1, AO, BWD>;
  if (lds > 64 * 1024 && (dev < 0 || dev >= 64 || !attr_done[dev])) {
    err = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (err != hipSuccess) return err;
    if (dev >= 0 && dev < 64) attr_done[dev] = 1;
  }
  hipLaunchKernelGGL(k, dim3(a.n_chunks * C::NG), dim3(C::NT), lds, s, a);
  return hipGetLastError();
}

// the three part passes of a wide backward (see the header comment)
template <int S, int ACT>
static hipError_t bp_run(BflyPartArgs a, const void* x, const void* dy, void* dx, float* zbuf, float* dzbuf,
                         hipStream_t s) {
  const bool tr = a.transpose != 0;
  hipError_t err;
  // z = first part applied (low for B, high^T for B^T)
  a.in0 = x; a.in1 = nullptr; a.out = zbuf;
  err = tr ? bp_launch<S, BP_HIGH, ACT, ACT_F32, ACT_F32, 0>(a, s) : bp_launch<S, BP_LOW, ACT, ACT_F32, ACT_F32, 0>(a, s);
  if (err != hipSuccess) return err;
  // second part's backward from (z, dy): dz
  a.in0 = zbuf; a.in1 = dy; a.out = dzbuf;
  err = tr ? bp_launch<S, BP_LOW, ACT_F32, ACT, ACT_F32, 1>(a, s) : bp_launch<S, BP_HIGH, ACT_F32, ACT, ACT_F32, 1>(a, s);
  if (err != hipSuccess) return err;
  // first part's backward from (x, dz): dx
  a.in0 = x; a.in1 = dzbuf; a.out = dx;
  return tr ? bp_launch<S, BP_HIGH, ACT, ACT_F32, ACT, 1>(a, s) : bp_launch<S, BP_LOW, ACT, ACT_F32, ACT, 1>(a, s);
}

static size_t align256z(size_t v) { return (v + 255) & ~size_t(255); }

// rows per chunk of the part passes: a multiple of 32, at most 256, about 256
// chunks (every part has at least 4 index groups per chunk)
static int bp_chunk(int rows) {
  int k = rows / (32 * 256);
  k = k < 1 ? 1 : k > 8 ? 8 : k;
  return 32 * k;
}

static int bwd_chunk(int log2n, int rows) { return log2n >= 12 ? bp_chunk(rows) : bfly_bwd_chunk(log2n, rows); }

size_t bfly_bwd_workspace(int log2n, int n_experts, int rows) {
  if (rows <= 0) return 0;
  const int ch = bwd_chunk(log2n, rows);
  const size_t chunks = size_t((rows + ch - 1) / ch + n_experts);
  size_t b = chunks * size_t(log2n) * (size_t(1) << (log2n - 1)) * sizeof(float);
  if (log2n >= 12) b = align256z(b) + 2 * align256z((size_t(rows) << log2n) * sizeof(float));  // z, dz (fp32)
  return b;
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
    default: return hipErrorInvalidValue;  // widths of 4096 and more take the part passes
  }
}

hipError_t launch_bfly_bwd(const void* x, const void* dy, void* dx, const float* ang, const int32_t* offsets,
                           float* part, float* dang, int rows, int n_experts, int log2n, int transpose, int act,
                           hipStream_t s) {
  BflyBwdArgs a{x, dy, dx, ang, offsets, part, dang, rows, n_experts, transpose, bb_tile_rows(log2n), 1, 0};
  const int L = log2n, n = 1 << L;
  if (rows > 0 && L >= 12) {
    a.chunk = bp_chunk(rows);
    a.n_chunks = (rows + a.chunk - 1) / a.chunk + n_experts;
    const size_t pbytes = align256z(size_t(a.n_chunks) * L * (n >> 1) * sizeof(float));
    float* zbuf = reinterpret_cast<float*>(reinterpret_cast<char*>(part) + pbytes);
    float* dzbuf = reinterpret_cast<float*>(reinterpret_cast<char*>(zbuf) + align256z((size_t(rows) << L) * 4));
    BflyPartArgs pa{nullptr, nullptr, nullptr, ang, offsets, part, rows, n_experts, transpose, a.chunk, a.n_chunks};
    hipError_t err;
    if (L == 12) err = act == ACT_BF16 ? bp_run<8, ACT_BF16>(pa, x, dy, dx, zbuf, dzbuf, s) : bp_run<8, ACT_F32>(pa, x, dy, dx, zbuf, dzbuf, s);
    else err = act == ACT_BF16 ? bp_run<9, ACT_BF16>(pa, x, dy, dx, zbuf, dzbuf, s) : bp_run<9, ACT_F32>(pa, x, dy, dx, zbuf, dzbuf, s);
    if (err != hipSuccess) return err;
  } else if (rows > 0) {
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
