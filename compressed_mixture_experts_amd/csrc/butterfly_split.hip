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
// Low part: the chunk rows go through an fp32 LDS tile and the passes of
// butterfly_impl.hpp (three stages per pass, table of the chunk's (cos, sin)).
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

// Low part of the butterfly of every row, in place allowed (a.in may equal a.out).
template <int S, bool TRANS>
__global__ __launch_bounds__(BF_THREADS) void bsplit_low_kernel(BflyArgs a) {
  using C = BflyCfg<S>;
  using LC = LowCfg<S>;
  constexpr int L = S + 4;
  constexpr int n = 1 << L, half = n / 2;
  constexpr int nch = n >> S;
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
  AngleRegs<S, TAB_FULL> none;

  constexpr int CPR = C::n / 8;  // 8-element chunks per row
  const uint16_t* in = reinterpret_cast<const uint16_t*>(a.in);
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  for (int rs = 0; rs < nr; rs += LC::RT) {
    const int m = min(LC::RT, nr - rs);
    __syncthreads();  // table written / previous sub-tile stored
    for (int k = tid; k < m * CPR; k += BF_THREADS) {
      const int r = k / CPR, j = k % CPR;
      float v[8];
      load8<ACT_BF16>(in, size_t(r0 + rs + r) * n + c * C::n + 8 * j, v);
      float* d = tile + r * C::stride + pos(8 * j);
      reinterpret_cast<float4*>(d)[0] = make_float4(v[0], v[1], v[2], v[3]);
      reinterpret_cast<float4*>(d)[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
    __syncthreads();
    run_passes<S, TRANS, false, 0, TAB_FULL>(tile, m, tab, nullptr, none);
    for (int k = tid; k < m * CPR; k += BF_THREADS) {
      const int r = k / CPR, j = k % CPR;
      const float* sp = tile + r * C::stride + pos(8 * j);
      const float4 x0 = reinterpret_cast<const float4*>(sp)[0];
      const float4 x1 = reinterpret_cast<const float4*>(sp)[1];
      const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      store8<ACT_BF16>(out, size_t(r0 + rs + r) * n + c * C::n + 8 * j, v);
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
