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
struct BflyPartArgs {
  const void* in0;        // rows the part's forward is recomputed from [R][n]
  const void* in1;        // gradient rows at the part's output [R][n] (backward)
  void* out;              // forward: part(in0); backward: gradient at the part's input
  const float* ang;       // [N][L][n/2]
  const int32_t* offsets; // [N+1]
  float* part;            // [n_chunks][L][n/2]
  int32_t rows, n_experts, chunk, n_chunks;
};

// expert, first row and row count of chunk cb (e = -1 for an unused index),
// broadcast through LDS to the whole workgroup
__device__ __forceinline__ void bp_chunk_info(const BflyPartArgs& a, int cb, int* s_info) {
  const int tid = threadIdx.x, CH = a.chunk;
  if (tid == 0) s_info[0] = -1;
  __syncthreads();
  for (int e = tid; e < a.n_experts; e += blockDim.x) {
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
}

// the same for the wave's own chunk cb, without LDS or barriers: the lane
// that finds it broadcasts it (at most one expert owns an index)
__device__ __forceinline__ void bp_wave_chunk(const BflyPartArgs& a, int cb, int& e, int& c0, int& ccnt) {
  const int lane = threadIdx.x & 63, CH = a.chunk;
  int fe = -1, f0 = 0, fc = 0;
  for (int x = lane; x < a.n_experts; x += 64) {
    const int off = min(max(a.offsets[x], 0), a.rows);
    const int cnt = min(max(a.offsets[x + 1], off), a.rows) - off;
    const int base = off / CH + x, nt = (cnt + CH - 1) / CH;
    if (cb >= base && cb < base + nt) {
      fe = x;
      f0 = off + (cb - base) * CH;
      fc = min(CH, cnt - (cb - base) * CH);
    }
  }
  const unsigned long long m = __ballot(fe >= 0);
  if (m == 0) {
    e = -1;
    return;
  }
  const int src = __ffsll(m) - 1;
  e = __shfl(fe, src);
  c0 = __shfl(f0, src);
  ccnt = __shfl(fc, src);
}

// number of stage t's pair whose lower index is i
__device__ __forceinline__ int pair_of(int i, int t) { return ((i >> (t + 1)) << t) | (i & ((1 << t) - 1)); }

template <int A>
__device__ __forceinline__ void store1(void* p, size_t i, float v) {
  if constexpr (A == ACT_BF16) {
    reinterpret_cast<uint16_t*>(p)[i] = uint16_t(pack_bf16x2(v, 0.f) & 0xFFFFu);
  } else {
    reinterpret_cast<float*>(p)[i] = v;
  }
}

// one rotation of a pair and the backward through it (s already negated for B^T)
__device__ __forceinline__ void bp_rot(float& x0, float& x1, float c, float s) {
  const float a = x0, b = x1;
  x0 = c * a - s * b;
  x1 = s * a + c * b;
}
// returns g_b a' - g_a b' for outputs (o0, o1) with gradients (g0, g1), and
// turns both pairs back through the rotation
__device__ __forceinline__ float bp_back(float& o0, float& o1, float& g0, float& g1, float c, float s) {
  const float a = o0, b = o1, ga = g0, gb = g1;
  o0 = c * a + s * b;
  o1 = -s * a + c * b;
  g0 = c * ga + s * gb;
  g1 = -s * ga + c * gb;
  return gb * a - ga * b;
}

// ---- low part: stages 0 .. S-1 on 2^S consecutive indices of rows of 2^LW
// elements (LW = S + 4 for the split widths; LW = S = 9 for rows of 512, where
// the low part is the whole butterfly).  A wave owns a 512-element slot of a
// row (one segment for S = 9, two for S = 8) and walks the chunk's rows
// (rows of 512: the four waves of a workgroup take every fourth row of one
// chunk and add their angle gradients in LDS, in wave order, at the end); a lane holds 8 elements of the slot whose index
// differs in three bits, so three stages run in registers between exchanges.
// Layout G (G = 0, 1, 2) puts the 3 bits at base bit BB(G) = 0, 3, and 6
// (S = 9) or 5 (S = 8; its stages are 6 and 7, the lowest bit is stage 5,
// already done): element of (lane l, j) = (l mod 2^BB) | j << BB | (l >> BB)
// << (BB + 3).  Exchanges go through the wave's own 512 floats of LDS (no
// workgroup barrier), stored at e ^ (((e >> 6) & 7) << 3) so that every
// layout's accesses spread over the banks.
template <int S>
struct BpLow {
  static constexpr int bb(int G) { return G == 0 ? 0 : G == 1 ? 3 : (S == 9 ? 6 : 5); }
  static constexpr int first(int G) { return G * 3; }                   // first stage of group G
  static constexpr int nst(int G) { return G < 2 ? 3 : S - 6; }         // stages in group G
  static __device__ __forceinline__ int elem(int G, int l, int j) {
    const int b = bb(G);
    return (l & ((1 << b) - 1)) | (j << b) | ((l >> b) << (b + 3));
  }
  static __device__ __forceinline__ int swz(int e) { return e ^ (((e >> 6) & 7) << 3); }
};

template <int S, int LW, int TR, int A0, int A1, int AO, int BWD>
__global__ __launch_bounds__(256) void bfly_low_kernel(BflyPartArgs a) {
  using P = BpLow<S>;
  constexpr int L = LW, n = 1 << L, half = n / 2;
  constexpr int NSLOT = n / 512;                   // slots per row
  constexpr bool SPLIT = NSLOT == 1;               // four waves share a chunk's rows
  static_assert(SPLIT || NSLOT % 4 == 0, "slots per row");
  constexpr int G0 = TR ? 2 : 0, G2 = TR ? 0 : 2;   // first and last layout applied
  __shared__ __attribute__((aligned(16))) float xch[4][2][512];
  __shared__ int s_info[3];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int cb, slot, e, c0, ccnt;
  if constexpr (SPLIT) {
    cb = blockIdx.x;
    slot = 0;
    bp_chunk_info(a, cb, s_info);
    e = s_info[0];
    if (e < 0) return;
    c0 = s_info[1];
    ccnt = s_info[2];
  } else {
    const int unit = blockIdx.x * 4 + w;
    cb = unit / NSLOT;
    slot = unit % NSLOT;
    bp_wave_chunk(a, cb, e, c0, ccnt);
    if (e < 0) return;
  }
  const float* ang = a.ang + size_t(e) * L * half;
  const int sbase = slot * 512;
  float* XV = xch[w][0];
  float* XG = xch[w][1];

  // (cos, sin) and angle gradients of this lane's pairs: [group][stage in group][pair]
  float cc[3][3][4], ss[3][3][4], acc[3][3][4];
#pragma unroll
  for (int G = 0; G < 3; ++G)
#pragma unroll
    for (int ti = 0; ti < 3; ++ti)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        cc[G][ti][k] = 1.f;
        ss[G][ti][k] = 0.f;
        acc[G][ti][k] = 0.f;
        if (ti < P::nst(G)) {
          const int t = P::first(G) + ti, p = t - P::bb(G);
          const int j = pair_lo(k, p);
          const float2 v = bb_sincos(ang[t * half + pair_of(sbase + P::elem(G, lane, j), t)]);
          cc[G][ti][k] = v.x;
          ss[G][ti][k] = TR ? -v.y : v.y;
        }
      }

  // the stages of group G in the order of application, forward and backward
  auto fwd_group = [&](int G, float (&x)[8]) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int ti = TR ? P::nst(G) - 1 - q : q;
      if (ti < 0 || ti >= P::nst(G)) continue;
      const int p = P::first(G) + ti - P::bb(G);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = pair_lo(k, p);
        bp_rot(x[j], x[j + (1 << p)], cc[G][ti][k], ss[G][ti][k]);
      }
    }
  };
  auto bwd_group = [&](int G, float (&x)[8], float (&g)[8]) {
#pragma unroll
    for (int q = 2; q >= 0; --q) {
      const int ti = TR ? P::nst(G) - 1 - q : q;
      if (ti < 0 || ti >= P::nst(G)) continue;
      const int p = P::first(G) + ti - P::bb(G);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = pair_lo(k, p), jh = j + (1 << p);
        const float d = bp_back(x[j], x[jh], g[j], g[jh], cc[G][ti][k], ss[G][ti][k]);
        acc[G][ti][k] += TR ? -d : d;
      }
    }
  };
  // layout change through the wave's LDS (wavefront-scope fences: LDS accesses
  // of one wave take effect in order; the fences keep the compiler from
  // moving them across each other)
  auto exchange = [&](float* X, float (&x)[8], int Gf, int Gt) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int j = 0; j < 8; ++j) X[P::swz(P::elem(Gf, lane, j))] = x[j];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = X[P::swz(P::elem(Gt, lane, j))];
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // rows <-> registers in layout G (layout 0: 8 consecutive elements)
  auto load = [&](auto act_c, const void* src, int r, int G, float (&x)[8]) {
    constexpr int A = decltype(act_c)::value;
    const size_t base = size_t(r) * n + sbase;
    if (G == 0) {
      load8<A>(src, base + P::elem(0, lane, 0), x);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = load1<A>(src, base + P::elem(G, lane, j));
    }
  };
  auto store = [&](auto act_c, void* dst, int r, int G, const float (&x)[8]) {
    constexpr int A = decltype(act_c)::value;
    const size_t base = size_t(r) * n + sbase;
    if (G == 0) {
      store8<A>(dst, base + P::elem(0, lane, 0), x);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) store1<A>(dst, base + P::elem(G, lane, j), x[j]);
    }
  };
  using C0 = std::integral_constant<int, A0>;
  using C1 = std::integral_constant<int, A1>;
  using CO = std::integral_constant<int, AO>;

  constexpr int RSTEP = SPLIT ? 4 : 1;
  const int rend = c0 + ccnt;
  float xn[8], gn[8];  // next row's inputs, loaded while this row is worked on
  if (c0 + (SPLIT ? w : 0) < rend) {
    load(C0(), a.in0, c0 + (SPLIT ? w : 0), G0, xn);
    if constexpr (BWD) load(C1(), a.in1, c0 + (SPLIT ? w : 0), G2, gn);
  }
  for (int r = c0 + (SPLIT ? w : 0); r < rend; r += RSTEP) {
    float x[8], g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = xn[j];
      if constexpr (BWD) g[j] = gn[j];
    }
    if (r + RSTEP < rend) {
      load(C0(), a.in0, r + RSTEP, G0, xn);
      if constexpr (BWD) load(C1(), a.in1, r + RSTEP, G2, gn);
    }
    // forward: groups in the order of application
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int G = TR ? 2 - q : q;
      if (q > 0) exchange(XV, x, TR ? G + 1 : G - 1, G);
      fwd_group(G, x);
    }
    if constexpr (!BWD) {
      store(CO(), a.out, r, G2, x);
    } else {
#pragma unroll
      for (int q = 2; q >= 0; --q) {
        const int G = TR ? 2 - q : q;
        bwd_group(G, x, g);
        if (q > 0) {
          const int Gp = TR ? G + 1 : G - 1;  // the group applied before G
          exchange(XV, x, G, Gp);
          exchange(XG, g, G, Gp);
        }
      }
      store(CO(), a.out, r, G0, g);
    }
  }

  if constexpr (BWD) {
    float* part = a.part + size_t(cb) * L * half;
    float* red = &xch[0][0][0];  // 4 waves x 1024 floats
#pragma unroll
    for (int G = 0; G < 3; ++G) {
      if constexpr (SPLIT) {
        __syncthreads();  // every wave is past its rows (or the previous group)
#pragma unroll
        for (int ti = 0; ti < 3; ++ti)
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (ti < P::nst(G)) red[w * 1024 + (ti * 4 + k) * 64 + lane] = acc[G][ti][k];
        __syncthreads();
      }
#pragma unroll
      for (int ti = 0; ti < 3; ++ti)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (ti < P::nst(G) && (!SPLIT || w == 0)) {
            const int t = P::first(G) + ti, p = t - P::bb(G), q = (ti * 4 + k) * 64 + lane;
            const float v = SPLIT ? ((red[q] + red[1024 + q]) + red[2048 + q]) + red[3072 + q] : acc[G][ti][k];
            part[t * half + pair_of(sbase + P::elem(G, lane, pair_lo(k, p)), t)] = v;
          }
    }
  }
}

// ---- high part: stages S .. S+3, each on pairs (v + 2^S j, v + 2^S (j + 2^t')).
// A thread owns column v (v < 2^S) and holds its 16 elements j = 0..15 of a
// row: all four stages run in registers.  256 columns per workgroup.
template <int S, int TR, int A0, int A1, int AO, int BWD>
__global__ __launch_bounds__(256) void bfly_high_kernel(BflyPartArgs a) {
  constexpr int L = S + 4, n = 1 << L, half = n / 2;
  constexpr int BPC = (1 << S) / 256;  // workgroups per chunk
  __shared__ int s_info[3];
  const int cb = blockIdx.x / BPC, v = (blockIdx.x % BPC) * 256 + threadIdx.x;
  bp_chunk_info(a, cb, s_info);
  const int e = s_info[0];
  if (e < 0) return;
  const int c0 = s_info[1], ccnt = s_info[2];
  const float* ang = a.ang + size_t(e) * L * half;

  // local stage t (global S + t), local pair q: lower element pair_lo(q, t)
  float cc[4][8], ss[4][8], acc[4][8];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float2 cs = bb_sincos(ang[(S + t) * half + (q << S) + v]);
      cc[t][q] = cs.x;
      ss[t][q] = TR ? -cs.y : cs.y;
      acc[t][q] = 0.f;
    }

  float xn[16], gn[16];
  auto load = [&](auto act_c, const void* src, int r, float (&x)[16]) {
    constexpr int A = decltype(act_c)::value;
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = load1<A>(src, size_t(r) * n + v + (j << S));
  };
  using C0 = std::integral_constant<int, A0>;
  using C1 = std::integral_constant<int, A1>;
  load(C0(), a.in0, c0, xn);
  if constexpr (BWD) load(C1(), a.in1, c0, gn);
  for (int r = c0; r < c0 + ccnt; ++r) {
    float x[16], g[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      x[j] = xn[j];
      if constexpr (BWD) g[j] = gn[j];
    }
    if (r + 1 < c0 + ccnt) {
      load(C0(), a.in0, r + 1, xn);
      if constexpr (BWD) load(C1(), a.in1, r + 1, gn);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = TR ? 3 - k : k;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = pair_lo(q, t);
        bp_rot(x[j], x[j + (1 << t)], cc[t][q], ss[t][q]);
      }
    }
    if constexpr (!BWD) {
#pragma unroll
      for (int j = 0; j < 16; ++j) store1<AO>(a.out, size_t(r) * n + v + (j << S), x[j]);
    } else {
#pragma unroll
      for (int k = 3; k >= 0; --k) {
        const int t = TR ? 3 - k : k;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = pair_lo(q, t), jh = j + (1 << t);
          const float d = bp_back(x[j], x[jh], g[j], g[jh], cc[t][q], ss[t][q]);
          acc[t][q] += TR ? -d : d;
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) store1<AO>(a.out, size_t(r) * n + v + (j << S), g[j]);
    }
  }

  if constexpr (BWD) {
    float* part = a.part + size_t(cb) * L * half;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int q = 0; q < 8; ++q) part[(S + t) * half + (q << S) + v] = acc[t][q];
  }
}

// ---- widths 1024 and 2048 in one pass: NW = n / 512 waves hold a row (the
// workgroup's four waves work on 4 / NW rows at a time), wave w its
// 512-element slot w % NW in the low part's layouts 0..2 (stages 0..8), and a
// fourth layout, lane l' = 64 (w % NW) + lane holding the elements
// l' + 2^(L-3) j (j = 0..7, index bits L-3 .. L-1), runs stages 9 .. L-1.  The
// change between layouts 2 and 3 crosses waves, through a row buffer in LDS
// and a workgroup barrier; the buffers of the forward and the backward change
// are distinct, so two barriers per row step suffice.  Every wave takes the
// same number of row steps (a step past the chunk's end loads and stores
// nothing), and at width 1024 the two rows' waves of a slot add their angle
// gradients in LDS at the end.
template <int L, int TR, int ACT>
__global__ __launch_bounds__(256) void bfly_row_kernel(BflyPartArgs a) {
  using P = BpLow<9>;
  constexpr int n = 1 << L, half = n / 2;
  constexpr int NW = n / 512, RPW = 4 / NW;        // waves per row, rows per step
  constexpr int B3 = L - 3, NST3 = L - 9;          // layout 3: base bit, stages
  static_assert(L == 10 || L == 11, "widths 1024 and 2048");
  constexpr int G0 = TR ? 3 : 0, G3 = TR ? 0 : 3;  // first and last layout applied
  __shared__ __attribute__((aligned(16))) float xw[4][512];   // in-wave layout changes
  __shared__ __attribute__((aligned(16))) float xf[2048];     // forward 2 <-> 3 (RPW rows)
  __shared__ __attribute__((aligned(16))) float xb[2][2048];  // backward 3 <-> 2 (values, gradients)
  __shared__ int s_info[3];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rs = w / NW, slot = w % NW, lp = slot * 64 + lane;
  const int cb = blockIdx.x;
  bp_chunk_info(a, cb, s_info);
  const int e = s_info[0];
  if (e < 0) return;
  const int c0 = s_info[1], ccnt = s_info[2];
  const float* ang = a.ang + size_t(e) * L * half;
  const int sbase = slot * 512;
  // index in the row of element j of this lane in layout G
  auto elem = [&](int G, int j) { return G < 3 ? sbase + P::elem(G, lane, j) : lp | (j << B3); };

  // groups 0..2: stages 3G .. 3G+2; group 3: stages 9 .. L-1 (j bits 12-L ..)
  float cc[4][3][4], ss[4][3][4], acc[4][3][4];
#pragma unroll
  for (int G = 0; G < 4; ++G)
#pragma unroll
    for (int ti = 0; ti < 3; ++ti)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        cc[G][ti][k] = 1.f;
        ss[G][ti][k] = 0.f;
        acc[G][ti][k] = 0.f;
        if (G < 3 || ti < NST3) {
          const int t = G < 3 ? 3 * G + ti : 9 + ti, p = G < 3 ? ti : 12 - L + ti;
          const float2 v = bb_sincos(ang[t * half + pair_of(elem(G, pair_lo(k, p)), t)]);
          cc[G][ti][k] = v.x;
          ss[G][ti][k] = TR ? -v.y : v.y;
        }
      }
  constexpr int NST[4] = {3, 3, 3, NST3};
  auto jbit = [](int G, int ti) { return G < 3 ? ti : 12 - L + ti; };
  auto fwd_group = [&](int G, float (&x)[8]) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int ti = TR ? NST[G] - 1 - q : q;
      if (ti < 0 || ti >= NST[G]) continue;
      const int p = jbit(G, ti);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = pair_lo(k, p);
        bp_rot(x[j], x[j + (1 << p)], cc[G][ti][k], ss[G][ti][k]);
      }
    }
  };
  auto bwd_group = [&](int G, float (&x)[8], float (&g)[8]) {
#pragma unroll
    for (int q = 2; q >= 0; --q) {
      const int ti = TR ? NST[G] - 1 - q : q;
      if (ti < 0 || ti >= NST[G]) continue;
      const int p = jbit(G, ti);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = pair_lo(k, p), jh = j + (1 << p);
        const float d = bp_back(x[j], x[jh], g[j], g[jh], cc[G][ti][k], ss[G][ti][k]);
        acc[G][ti][k] += TR ? -d : d;
      }
    }
  };
  // in-wave layout change (groups 0..2) through the wave's slice
  auto xch_wave = [&](float (&x)[8], int Gf, int Gt) {
    float* X = xw[w];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int j = 0; j < 8; ++j) X[P::swz(P::elem(Gf, lane, j))] = x[j];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = X[P::swz(P::elem(Gt, lane, j))];
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto put = [&](float* X, const float (&x)[8], int G) {
#pragma unroll
    for (int j = 0; j < 8; ++j) X[elem(G, j)] = x[j];
  };
  auto get = [&](const float* X, float (&x)[8], int G) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = X[elem(G, j)];
  };
  auto load = [&](const void* src, int r, int G, float (&x)[8]) {
    const size_t base = size_t(r) * n;
    if (G == 0) {
      load8<ACT>(src, base + elem(0, 0), x);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = load1<ACT>(src, base + elem(G, j));
    }
  };
  auto store = [&](void* dst, int r, int G, const float (&x)[8]) {
    const size_t base = size_t(r) * n;
    if (G == 0) {
      store8<ACT>(dst, base + elem(0, 0), x);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) store1<ACT>(dst, base + elem(G, j), x[j]);
    }
  };

  float* XF = xf + rs * n;
  float* XB0 = xb[0] + rs * n;
  float* XB1 = xb[1] + rs * n;
  const int rend = c0 + ccnt, steps = (ccnt + RPW - 1) / RPW;
  float xn[8], gn[8];
  if constexpr (RPW > 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) xn[j] = gn[j] = 0.f;
  }
  if (RPW == 1 || c0 + rs < rend) {
    load(a.in0, c0 + rs, G0, xn);
    load(a.in1, c0 + rs, G3, gn);
  }
  for (int it = 0; it < steps; ++it) {
    const int r = c0 + it * RPW + rs;
    const bool act = RPW == 1 || r < rend;  // a step past the end works on zeros: no gradient, no store
    float x[8], g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = act ? xn[j] : 0.f;
      g[j] = act ? gn[j] : 0.f;
    }
    if (r + RPW < rend) {
      load(a.in0, r + RPW, G0, xn);
      load(a.in1, r + RPW, G3, gn);
    }
    // forward, layouts in the order of application
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int G = TR ? 3 - q : q;
      if (q > 0) {
        const int Gp = TR ? G + 1 : G - 1;
        if (G == 3 || Gp == 3) {
          put(XF, x, Gp);
          __syncthreads();
          get(XF, x, G);
        } else {
          xch_wave(x, Gp, G);
        }
      }
      fwd_group(G, x);
    }
    // backward, in the reverse order
#pragma unroll
    for (int q = 3; q >= 0; --q) {
      const int G = TR ? 3 - q : q;
      bwd_group(G, x, g);
      if (q > 0) {
        const int Gp = TR ? G + 1 : G - 1;  // the layout applied before G
        if (G == 3 || Gp == 3) {
          put(XB0, x, G);
          put(XB1, g, G);
          __syncthreads();
          get(XB0, x, Gp);
          get(XB1, g, Gp);
        } else {
          xch_wave(x, G, Gp);
          xch_wave(g, G, Gp);
        }
      }
    }
    if (act) store(a.out, r, G0, g);
  }

  float* part = a.part + size_t(cb) * L * half;
  float* red = xb[0];  // 4 waves x 1024 floats (free after the last row step)
#pragma unroll
  for (int G = 0; G < 4; ++G) {
    if constexpr (RPW > 1) {
      __syncthreads();  // every wave is past its rows (or the previous group)
#pragma unroll
      for (int ti = 0; ti < 3; ++ti)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (G < 3 || ti < NST3) red[w * 1024 + (ti * 4 + k) * 64 + lane] = acc[G][ti][k];
      __syncthreads();
    }
#pragma unroll
    for (int ti = 0; ti < 3; ++ti)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if ((G < 3 || ti < NST3) && rs == 0) {
          const int t = G < 3 ? 3 * G + ti : 9 + ti, q = (ti * 4 + k) * 64 + lane;
          float v = acc[G][ti][k];
          if constexpr (RPW > 1) {
            v = red[w * 1024 + q];
#pragma unroll
            for (int o = 1; o < RPW; ++o) v += red[(w + o * NW) * 1024 + q];
          }
          part[t * half + pair_of(elem(G, pair_lo(k, jbit(G, ti))), t)] = v;
        }
  }
}

template <int S, int HIGH, int TR, int A0, int A1, int AO, int BWD>
static hipError_t bp_launch(const BflyPartArgs& a, hipStream_t s) {
  if constexpr (HIGH) {
    hipLaunchKernelGGL((bfly_high_kernel<S, TR, A0, A1, AO, BWD>), dim3(a.n_chunks * ((1 << S) / 256)), dim3(256),
                       0, s, a);
  } else {
    hipLaunchKernelGGL((bfly_low_kernel<S, S + 4, TR, A0, A1, AO, BWD>), dim3(a.n_chunks * ((1 << (S + 4)) / 2048)),
                       dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// the three part passes of a wide backward (see the header comment)
template <int S, int TR, int ACT>
static hipError_t bp_run(BflyPartArgs a, const void* x, const void* dy, void* dx, float* zbuf, float* dzbuf,
                         hipStream_t s) {
  constexpr int FIRST = TR ? 1 : 0;  // the part applied first: low for B, high^T for B^T
  hipError_t err;
  // z = first part applied to x
  a.in0 = x; a.in1 = nullptr; a.out = zbuf;
  err = bp_launch<S, FIRST, TR, ACT, ACT_F32, ACT_F32, 0>(a, s);
  if (err != hipSuccess) return err;
  // second part's backward from (z, dy): dz
  a.in0 = zbuf; a.in1 = dy; a.out = dzbuf;
  err = bp_launch<S, 1 - FIRST, TR, ACT_F32, ACT, ACT_F32, 1>(a, s);
  if (err != hipSuccess) return err;
  // first part's backward from (x, dz): dx
  a.in0 = x; a.in1 = dzbuf; a.out = dx;
  return bp_launch<S, FIRST, TR, ACT, ACT_F32, ACT, 1>(a, s);
}

static size_t align256z(size_t v) { return (v + 255) & ~size_t(255); }

// rows per chunk of the part passes: a multiple of 32, at most 128, about 256
// chunks or more
static int bp_chunk(int rows) {
  int k = rows / (32 * 256);
  k = k < 1 ? 1 : k > 4 ? 4 : k;
  return 32 * k;
}

// rows per chunk at widths 1024 and 2048 (one workgroup per chunk): a multiple
// of 16, at most 128, about 1024 chunks or more
static int row11_chunk(int rows) {
  int k = rows / (16 * 1024);
  k = k < 1 ? 1 : k > 8 ? 8 : k;
  return 16 * k;
}

// rows per chunk at width 512 (one workgroup per chunk): 8 .. 64, about 512
// chunks
static int row9_chunk(int rows) {
  const int k = rows / 512;
  return k < 8 ? 8 : k > 64 ? 64 : k;
}

static int bwd_chunk(int log2n, int rows) {
  return log2n >= 12 ? bp_chunk(rows)
       : log2n == 11 || log2n == 10 ? row11_chunk(rows)
       : log2n == 9  ? row9_chunk(rows)
                     : bfly_bwd_chunk(log2n, rows);
}

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
  const hipError_t err = allow_dynamic_lds((const void*)bfly_bwd_kernel<L, ACT>, lds);
  if (err != hipSuccess) return err;
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
    default: return hipErrorInvalidValue;  // width 2048 and more take the register kernels
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
    BflyPartArgs pa{nullptr, nullptr, nullptr, ang, offsets, part, rows, n_experts, a.chunk, a.n_chunks};
    const bool bf = act == ACT_BF16, tr = transpose != 0;
    hipError_t err;
    if (L == 12) {
      err = tr ? (bf ? bp_run<8, 1, ACT_BF16>(pa, x, dy, dx, zbuf, dzbuf, s) : bp_run<8, 1, ACT_F32>(pa, x, dy, dx, zbuf, dzbuf, s))
               : (bf ? bp_run<8, 0, ACT_BF16>(pa, x, dy, dx, zbuf, dzbuf, s) : bp_run<8, 0, ACT_F32>(pa, x, dy, dx, zbuf, dzbuf, s));
    } else {
      err = tr ? (bf ? bp_run<9, 1, ACT_BF16>(pa, x, dy, dx, zbuf, dzbuf, s) : bp_run<9, 1, ACT_F32>(pa, x, dy, dx, zbuf, dzbuf, s))
               : (bf ? bp_run<9, 0, ACT_BF16>(pa, x, dy, dx, zbuf, dzbuf, s) : bp_run<9, 0, ACT_F32>(pa, x, dy, dx, zbuf, dzbuf, s));
    }
    if (err != hipSuccess) return err;
  } else if (rows > 0 && L == 9) {
    a.chunk = row9_chunk(rows);
    a.n_chunks = (rows + a.chunk - 1) / a.chunk + n_experts;
    const BflyPartArgs pa{x, dy, dx, ang, offsets, part, rows, n_experts, a.chunk, a.n_chunks};
    const dim3 grid(a.n_chunks);
    if (transpose) {
      if (act == ACT_BF16) hipLaunchKernelGGL((bfly_low_kernel<9, 9, 1, ACT_BF16, ACT_BF16, ACT_BF16, 1>), grid, dim3(256), 0, s, pa);
      else hipLaunchKernelGGL((bfly_low_kernel<9, 9, 1, ACT_F32, ACT_F32, ACT_F32, 1>), grid, dim3(256), 0, s, pa);
    } else {
      if (act == ACT_BF16) hipLaunchKernelGGL((bfly_low_kernel<9, 9, 0, ACT_BF16, ACT_BF16, ACT_BF16, 1>), grid, dim3(256), 0, s, pa);
      else hipLaunchKernelGGL((bfly_low_kernel<9, 9, 0, ACT_F32, ACT_F32, ACT_F32, 1>), grid, dim3(256), 0, s, pa);
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  } else if (rows > 0 && (L == 10 || L == 11)) {
    a.chunk = row11_chunk(rows);
    a.n_chunks = (rows + a.chunk - 1) / a.chunk + n_experts;
    const BflyPartArgs pa{x, dy, dx, ang, offsets, part, rows, n_experts, a.chunk, a.n_chunks};
    const bool bf = act == ACT_BF16, tr = transpose != 0;
#define BB_ROW(LL)                                                                                      \
    if (tr) {                                                                                           \
      if (bf) hipLaunchKernelGGL((bfly_row_kernel<LL, 1, ACT_BF16>), dim3(a.n_chunks), dim3(256), 0, s, pa); \
      else hipLaunchKernelGGL((bfly_row_kernel<LL, 1, ACT_F32>), dim3(a.n_chunks), dim3(256), 0, s, pa);    \
    } else {                                                                                            \
      if (bf) hipLaunchKernelGGL((bfly_row_kernel<LL, 0, ACT_BF16>), dim3(a.n_chunks), dim3(256), 0, s, pa); \
      else hipLaunchKernelGGL((bfly_row_kernel<LL, 0, ACT_F32>), dim3(a.n_chunks), dim3(256), 0, s, pa);    \
    }
    if (L == 10) { BB_ROW(10) } else { BB_ROW(11) }
#undef BB_ROW
    const hipError_t err = hipGetLastError();
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
