// Wide butterflies (n = 2^L, L = S + 4 in [10, 13]) of bf16 rows bucketed by
// expert, split into two parts that each touch a small closed set of indices
// (ButterflyMoE, gist.science/zh/paper/2601.13563, technical summary §2.2:
// stage s rotates the pairs of indices that differ in bit s, each pair with its
// own angle):
//   low part  - stages 0 .. S-1: closed on chunks of 2^S consecutive indices;
//               chunk c, stage s uses angles [c 2^(S-1), (c+1) 2^(S-1)) of s.
//   high part - stages S .. S+3: closed on the 16 indices v + j 2^S (j < 16)
//               of one column v < 2^S; stage S+t, local pair q (the pair
//               index of a width-16 butterfly at stage t) uses angle q 2^S + v.
// B = high * low, so B x runs low then high, B^T x high^T then low^T.
//
// Each workgroup owns up to SP_RB rows of ONE expert and one chunk (low) or 64
// columns (high), so the expert's angles for that part are loaded and turned
// into (cos, sin) once per workgroup and reused for all its rows; a width that
// has more angles than a row has elements would otherwise move more angle
// bytes than activation bytes per row.  Rows are read and written as bf16; the
// rotations of a part run in fp32.
//
// Low part: the chunk rows go through an fp32 LDS tile in passes of three
// stages (groups and (cos, sin) table as in butterfly_impl.hpp); every pass
// covers the whole sub-tile with all its LDS reads issued first.
// High part: thread (column v, row lane) keeps the (cos, sin) of its column in
// registers and holds the 16 elements of one row's column at a time (stride
// 2^S; 64 lanes read 64 consecutive bf16), so all four stages, the GELU
// between the FFN's two butterflies and the gate run in registers.
#include "butterfly_impl.hpp"

namespace bmoe {

constexpr int SP_RB = 64;  // rows per workgroup
constexpr int SP_VC = 64;  // high part: columns per workgroup

template <int S>
struct LowCfg {
  static constexpr int n = 1 << S;
  static constexpr int RT = S >= 8 ? 16 : 32;  // rows per sub-tile
  static constexpr size_t tile_floats = size_t(RT) * BflyCfg<S>::stride;
  static constexpr size_t tab_pairs = size_t(S) << (S - 1);
  static constexpr size_t lds_bytes = tile_floats * 4 + tab_pairs * 8;
};

// Workgroup tile t -> (expert e, first bucket row r0, rows nr) with tiles of
// SP_RB rows per expert in expert order; e = -1 past the last tile.
__device__ __forceinline__ void sp_find_tile(const int32_t* offsets, int n_experts, int t, int& e, int& r0,
                                             int& nr) {
  __shared__ int s_info[3];
  __shared__ int s_tmp[4];
  const int tid = threadIdx.x;
  if (tid == 0) s_info[0] = -1;
  int nt = 0, cnt = 0, off = 0;
  if (tid < n_experts) {
    off = offsets[tid];
    cnt = offsets[tid + 1] - off;
    nt = (cnt + SP_RB - 1) / SP_RB;
  }
  int total;
  const int excl = block_excl_scan(nt, s_tmp, total);
  if (tid < n_experts && t >= excl && t < excl + nt) {
    const int j = t - excl;
    s_info[0] = tid;
    s_info[1] = off + j * SP_RB;
    s_info[2] = min(SP_RB, cnt - j * SP_RB);
  }
  __syncthreads();
  e = s_info[0];
  r0 = s_info[1];
  nr = s_info[2];
}

// One pass (stages 3P .. 3P+M-1) of the chunk butterfly over all RT rows of
// the sub-tile: each thread owns one group of 2^M elements in RT * G / 256
// rows, whose reads are all issued before any rotation (rows past the valid
// ones repeat the last valid row and are not stored).
template <int S, int P, bool TRANS>
__device__ __forceinline__ void low_pass(float* __restrict__ tile, const float2* __restrict__ tab) {
  using C = BflyCfg<S>;
  constexpr int RT = LowCfg<S>::RT;
  constexpr int S0 = 3 * P;
  constexpr int M = (S - S0) < 3 ? (S - S0) : 3;
  constexpr int E = 1 << M, NCS = M * (E / 2);
  constexpr int G = C::n >> M;                 // groups per row
  constexpr int RPT = RT * G / BF_THREADS;     // rows per thread
  constexpr int TPG = BF_THREADS / G;          // row stride between a thread's rows
  constexpr int OFF = elem_off<S0>();
  constexpr bool VEC = (S0 == 0 && M == 3);
  static_assert(G <= BF_THREADS && RPT >= 1, "tile shape");
  const int tid = threadIdx.x;
  const int g = tid & (G - 1), r0 = tid / G;
  float2 cs[NCS];
  const float2* t = tab + S0 * C::half + g * NCS;
#pragma unroll
  for (int j = 0; j < NCS; ++j) cs[j] = t[j];
  float* gp = tile + pos(group_base(g, S0, M)) + r0 * C::stride;
  float v[RPT][E];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const float* rp = gp + k * TPG * C::stride;
    if constexpr (VEC) {
      const float4 x0 = reinterpret_cast<const float4*>(rp)[0];
      const float4 x1 = reinterpret_cast<const float4*>(rp)[1];
      v[k][0] = x0.x; v[k][1] = x0.y; v[k][2] = x0.z; v[k][3] = x0.w;
      v[k][4] = x1.x; v[k][5] = x1.y; v[k][6] = x1.z; v[k][7] = x1.w;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) v[k][e] = rp[e * OFF];
    }
  }
#pragma unroll
  for (int k = 0; k < RPT; ++k) rotate_group<M, TRANS>(v[k], cs);
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    float* rp = gp + k * TPG * C::stride;
    if constexpr (VEC) {
      reinterpret_cast<float4*>(rp)[0] = make_float4(v[k][0], v[k][1], v[k][2], v[k][3]);
      reinterpret_cast<float4*>(rp)[1] = make_float4(v[k][4], v[k][5], v[k][6], v[k][7]);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) rp[e * OFF] = v[k][e];
    }
  }
}

template <int S, bool TRANS, int T = 0>
__device__ __forceinline__ void low_passes(float* tile, const float2* tab) {
  constexpr int NP = BflyCfg<S>::NP;
  if constexpr (T < NP) {
    low_pass<S, TRANS ? NP - 1 - T : T, TRANS>(tile, tab);
    __syncthreads();
    low_passes<S, TRANS, T + 1>(tile, tab);
  }
}

// Low part of the butterfly of every row, in place allowed (a.in may equal a.out).
// Sub-tiles of RT rows: the bf16 rows of sub-tile k + 1 are loaded into
// registers while sub-tile k runs its passes.
template <int S, bool TRANS>
__global__ __launch_bounds__(BF_THREADS) void bsplit_low_kernel(BflyArgs a) {
  using C = BflyCfg<S>;
  using LC = LowCfg<S>;
  constexpr int L = S + 4;
  constexpr int n = 1 << L, half = n / 2;
  constexpr int nch = n >> S;
  constexpr int CPR = C::n / 8;                       // 8-element pieces per row
  constexpr int PPT = LC::RT * CPR / BF_THREADS;      // pieces per thread
  static_assert(PPT * BF_THREADS == LC::RT * CPR, "sub-tile shape");
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* tile = smem;
  float2* tab = reinterpret_cast<float2*>(smem + LC::tile_floats);
  const int tid = threadIdx.x;
  const int t = blockIdx.x / nch, c = blockIdx.x % nch;
  int e, r0, nr;
  sp_find_tile(a.offsets, a.n_experts, t, e, r0, nr);
  if (e < 0) return;

  // (cos, sin) of the chunk's S stages, group-major as the passes read them
  const float* ang = a.ang0 + size_t(e) * L * half + size_t(c) * C::half;
  for (int idx = tid; idx < S * C::half; idx += BF_THREADS) {
    const int s = idx >> (S - 1), p = idx & (C::half - 1);
    tab[table_slot(s, p, S, true)] = sincos_rev(ang[s * half + p]);
  }

  const uint16_t* in = reinterpret_cast<const uint16_t*>(a.in) + size_t(r0) * n + c * C::n;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + size_t(r0) * n + c * C::n;
  auto load_raw = [&](int rs, uint4 (&raw)[PPT]) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int q = k * BF_THREADS + tid, r = q / CPR, j = q % CPR;
      raw[k] = *reinterpret_cast<const uint4*>(in + size_t(min(rs + r, nr - 1)) * n + 8 * j);
    }
  };
  uint4 raw[PPT];
  load_raw(0, raw);
  for (int rs = 0; rs < nr; rs += LC::RT) {
    __syncthreads();  // table written / previous sub-tile stored
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int q = k * BF_THREADS + tid, r = q / CPR, j = q % CPR;
      float* d = tile + r * C::stride + pos(8 * j);
      reinterpret_cast<float4*>(d)[0] = make_float4(bf16lo(raw[k].x), bf16hi(raw[k].x), bf16lo(raw[k].y), bf16hi(raw[k].y));
      reinterpret_cast<float4*>(d)[1] = make_float4(bf16lo(raw[k].z), bf16hi(raw[k].z), bf16lo(raw[k].w), bf16hi(raw[k].w));
    }
    __syncthreads();
    if (rs + LC::RT < nr) load_raw(rs + LC::RT, raw);
    low_passes<S, TRANS>(tile, tab);
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int q = k * BF_THREADS + tid, r = q / CPR, j = q % CPR;
      if (rs + r < nr) {
        const float* sp = tile + r * C::stride + pos(8 * j);
        const float4 x0 = reinterpret_cast<const float4*>(sp)[0];
        const float4 x1 = reinterpret_cast<const float4*>(sp)[1];
        uint4 o;
        o.x = pack_bf16x2(x0.x, x0.y);
        o.y = pack_bf16x2(x0.z, x0.w);
        o.z = pack_bf16x2(x1.x, x1.y);
        o.w = pack_bf16x2(x1.z, x1.w);
        *reinterpret_cast<uint4*>(out + size_t(rs + r) * n + 8 * j) = o;
      }
    }
  }
}

enum SplitHigh { SH_IN = 0, SH_MID = 1, SH_OUT = 2 };

// (cos, sin) of the four high stages of column v: cs[t * 8 + q] for stage S+t, local pair q.
template <int S>
__device__ __forceinline__ void sp_high_cs(const float* ang_e, int v, float2 cs[32]) {
  constexpr int half = 1 << (S + 3);
  float a[32];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int q = 0; q < 8; ++q) a[t * 8 + q] = ang_e[(S + t) * half + (q << S) + v];
#pragma unroll
  for (int i = 0; i < 32; ++i) cs[i] = sincos_rev(a[i]);
}

// High part of every row:
//   SH_IN   x[token of bucket row q] -> high^T(theta) -> out[q]
//   SH_MID  in[q] -> high(phi_up) -> GELU (if set) -> high^T(theta_dn) -> out[q]
//   SH_OUT  in[q] -> high(phi) -> * gate -> out[slot of q]
template <int S, int MODE>
__global__ __launch_bounds__(BF_THREADS) void bsplit_high_kernel(BflyArgs a) {
  constexpr int L = S + 4;
  constexpr int n = 1 << L, half = n / 2;
  constexpr int ncb = (1 << S) / SP_VC;
  const int tid = threadIdx.x;
  const int t = blockIdx.x / ncb, cb = blockIdx.x % ncb;
  int e, r0, nr;
  sp_find_tile(a.offsets, a.n_experts, t, e, r0, nr);
  if (e < 0) return;
  const int v = cb * SP_VC + (tid & (SP_VC - 1)), rl = tid / SP_VC;
  constexpr int RL = BF_THREADS / SP_VC;  // row lanes

  float2 cs0[32], cs1[MODE == SH_MID ? 32 : 1];
  sp_high_cs<S>(a.ang0 + size_t(e) * L * half, v, cs0);
  if constexpr (MODE == SH_MID) sp_high_cs<S>(a.ang1 + size_t(e) * L * half, v, cs1);

  const uint16_t* in = reinterpret_cast<const uint16_t*>(a.in);
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  for (int r = rl; r < nr; r += RL) {
    const int q = r0 + r;
    size_t src = size_t(q) * n, dst = size_t(q) * n;
    float g = 1.0f;
    if constexpr (MODE == SH_IN) src = size_t(a.perm[q] / a.top_k) * n;
    if constexpr (MODE == SH_OUT) {
      const int slot = a.perm[q];
      dst = size_t(slot) * n;
      g = a.gate[slot];
    }
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = __uint_as_float(uint32_t(in[src + (j << S) + v]) << 16);
    if constexpr (MODE == SH_IN) {
      rotate_group<4, true>(x, cs0);
    } else {
      rotate_group<4, false>(x, cs0);
      if constexpr (MODE == SH_MID) {
        if (a.gelu) {
#pragma unroll
          for (int j = 0; j < 16; ++j) x[j] = gelu_erf(x[j]);
        }
        rotate_group<4, true>(x, cs1);
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] *= g;
      }
    }
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const uint32_t w = pack_bf16x2(x[j], x[j + 1]);
      out[dst + (j << S) + v] = uint16_t(w & 0xFFFFu);
      out[dst + ((j + 1) << S) + v] = uint16_t(w >> 16);
    }
  }
}

template <typename K>
static hipError_t sp_launch(K k, int grid, size_t lds, const BflyArgs& a, hipStream_t s, int* attr_done) {
  if (grid <= 0) return hipSuccess;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (lds > 64 * 1024 && (dev < 0 || dev >= 64 || !attr_done[dev])) {
    err = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (err != hipSuccess) return err;
    if (dev >= 0 && dev < 64) attr_done[dev] = 1;
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(BF_THREADS), lds, s, a);
  return hipGetLastError();
}

static int sp_tiles(const BflyArgs& a) { return (a.rows + SP_RB - 1) / SP_RB + a.n_experts; }

template <int S>
static hipError_t launch_low_S(const BflyArgs& a, bool trans, hipStream_t s) {
  static int done[2][64] = {{0}};
  const int grid = sp_tiles(a) * 16;
  if (trans) return sp_launch(bsplit_low_kernel<S, true>, grid, LowCfg<S>::lds_bytes, a, s, done[1]);
  return sp_launch(bsplit_low_kernel<S, false>, grid, LowCfg<S>::lds_bytes, a, s, done[0]);
}

template <int S>
static hipError_t launch_high_S(const BflyArgs& a, int mode, hipStream_t s) {
  static int done[64] = {0};
  const int grid = sp_tiles(a) * ((1 << S) / SP_VC);
  switch (mode) {
    case SH_IN: return sp_launch(bsplit_high_kernel<S, SH_IN>, grid, 0, a, s, done);
    case SH_MID: return sp_launch(bsplit_high_kernel<S, SH_MID>, grid, 0, a, s, done);
    default: return sp_launch(bsplit_high_kernel<S, SH_OUT>, grid, 0, a, s, done);
  }
}

bool bfly_split_supported(int log2n) { return log2n >= 10 && log2n <= 13; }

hipError_t launch_bfly_split(const BflyArgs& a, int part, int log2n, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const bool low = part == SPLIT_LOW || part == SPLIT_LOW_T;
  const bool trans = part == SPLIT_LOW_T;
  const int mode = part == SPLIT_HIGH_IN ? SH_IN : part == SPLIT_HIGH_MID ? SH_MID : SH_OUT;
  switch (log2n) {
    case 10: return low ? launch_low_S<6>(a, trans, s) : launch_high_S<6>(a, mode, s);
    case 11: return low ? launch_low_S<7>(a, trans, s) : launch_high_S<7>(a, mode, s);
    case 12: return low ? launch_low_S<8>(a, trans, s) : launch_high_S<8>(a, mode, s);
    case 13: return low ? launch_low_S<9>(a, trans, s) : launch_high_S<9>(a, mode, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bmoe
