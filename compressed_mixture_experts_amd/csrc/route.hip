// Top-k softmax router and per-expert bucketing (ButterflyMoE,
// gist.science/nl/paper/2601.13563, §2 "Drie Fasen van de Methode": a standard
// top-k gating network selects the active experts).
//
// Logits l = W_g x are computed in fp32: bf16 activations on MFMA
// (v_mfma_f32_16x16x32_bf16, exact bf16 products, fp32 accumulation), fp32
// activations with one FMA chain per logit.  Every fp32 logit is within
//     eps_t = gamma_D * |x_t| * max_e |w_e|,   gamma_D = D u / (1 - D u)
// of its exact value, where D bounds the rounding depth of the sum (K/32 MFMA
// accumulations plus 32 adds inside one MFMA, or d for an FMA chain) and
// u = 2^-22 (twice the fp32 unit roundoff, as the MFMA's internal rounding is
// not documented).  A token's top-k is taken from the fp32 logits unless one
// of its decisive gaps (between consecutive chosen logits, or between the k-th
// and the (k+1)-th) is below 2 eps_t.  Then every expert whose fp32 logit is
// at least (k-th fp32 logit - 2 eps_t) - the only experts that can belong to
// the exact top-k - is recomputed in fp64 (exact bf16 products) and the top-k
// is taken among those.  Gates are the fp32 softmax probabilities.
#include "common.hpp"
#include <float.h>
#include <type_traits>

namespace bmoe {

constexpr int RT_THREADS = 256;
constexpr int RT_BK = 64;            // K per pipeline step (two MFMA k-steps)
constexpr int RT_XLD = RT_BK + 8;    // padded LDS row of the token tile (bf16)
constexpr int RT_KMAX = 8;           // largest supported top_k

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}
__device__ __forceinline__ bool better(double v, int i, double bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Insert (v, i) into the sorted list (tv, ti) of length KK, branch-free.
template <int KK, typename T>
__device__ __forceinline__ void topk_insert(T* tv, int* ti, T v, int i) {
#pragma unroll
  for (int j = 0; j < KK; ++j) {
    const bool sw = better(v, i, tv[j], ti[j]);
    const T a = tv[j];
    const int b = ti[j];
    tv[j] = sw ? v : a;
    ti[j] = sw ? i : b;
    v = sw ? a : v;
    i = sw ? b : i;
  }
}

// Per-token decision: 4 threads per token (q = lane & 3) each scan every 4th
// expert.  Round j picks the best entry strictly below the pick of round j-1
// in the order (larger value, then lower index), so kk rounds give the sorted
// top-kk.  Writes idx/gates of the fp32 decision and flags tokens whose
// decisive gaps are within the error bound.
__device__ void decide(const float* Lrow, int N, int k, int kk, int renorm, float tau, int q,
                       int* out_idx, float* out_gate, float* out_thr, float* out_max,
                       float* out_sum, bool* flag) {
  float tv[RT_KMAX + 1];
  int ti[RT_KMAX + 1];
  float pv = INFINITY;
  int pi = -1;
#pragma unroll
  for (int j = 0; j < RT_KMAX + 1; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    if (j < kk) {
      for (int e = q; e < N; e += 4) {
        const float v = Lrow[e];
        const bool below = v < pv || (v == pv && e > pi);
        if (below && better(v, e, bv, bi)) { bv = v; bi = e; }
      }
#pragma unroll
      for (int o = 1; o <= 2; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
    }
    tv[j] = bv;
    ti[j] = bi;
    pv = bv;
    pi = bi;
  }
  const float mx = tv[0];
  float s = 0.f;
  for (int e = q; e < N; e += 4) s += __expf(Lrow[e] - mx);
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  if (q == 0) {
    bool f = false;
    const int ngap = min(k, N - 1);
    float g[RT_KMAX];
    float gs = 0.f;
    float kth = tv[0];
#pragma unroll
    for (int j = 0; j < RT_KMAX; ++j) {
      if (j < ngap && tv[j] - tv[j + 1] < tau) f = true;
      g[j] = (j < k) ? __expf(tv[j] - mx) / s : 0.f;
      gs += g[j];
      if (j == k - 1) kth = tv[j];
    }
#pragma unroll
    for (int j = 0; j < RT_KMAX; ++j) {
      if (j < k) {
        out_idx[j] = ti[j];
        out_gate[j] = renorm ? g[j] / gs : g[j];
      }
    }
    *out_thr = kth - tau;
    *out_max = mx;
    *out_sum = s;
    *flag = f;
  }
}

template <int ACT, int BT>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(RouteArgs a) {
  constexpr int TB = BT / 16;                 // token blocks of 16
  constexpr int XCH = BT * (RT_BK / 8);       // 16-byte chunks of the token tile per step
  constexpr int XPT = (XCH + RT_THREADS - 1) / RT_THREADS;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sx = reinterpret_cast<uint16_t*>(smem);  // [2][BT][RT_XLD] token tile (bf16)
  float* sL = reinterpret_cast<float*>(smem);         // [BT][LS] logits (after the K loop)
  __shared__ float sX2[BT];
  __shared__ int sIdx[BT][RT_KMAX];
  __shared__ float sGate[BT][RT_KMAX];
  __shared__ float sThr[BT], sMax[BT], sSum[BT];
  __shared__ int sFlag[BT];
  __shared__ int sNF;
  __shared__ float sWmax[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * BT;
  const int N = a.N, d = a.d, k = a.k;
  const int NB = (N + 15) >> 4;
  const int LS = NB * 16 + 4;  // logit row stride (conflict-free quarter reads)
  if (tid == 0) sNF = 0;

  int depth;
  if constexpr (ACT == ACT_BF16) {
    const uint16_t* xg = reinterpret_cast<const uint16_t*>(a.x);
    const uint16_t* wg = reinterpret_cast<const uint16_t*>(a.w_gate);
    // wave w owns expert blocks b = w + 4 i (i < 4) and all token blocks
    f32x4_t acc[4][TB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < TB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float wsq[4] = {0.f, 0.f, 0.f, 0.f};
    float xsq[XPT];
#pragma unroll
    for (int r = 0; r < XPT; ++r) xsq[r] = 0.f;
    // two register sets (compile-time indexed): gate-weight fragments and
    // token chunks two steps ahead
    uint4 afr0[4][2], afr1[4][2];
    uint4 xr0[XPT], xr1[XPT];

    auto load_a = [&](int k0, uint4 (&dst)[4][2]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 16 * (wave + 4 * i) + (lane & 15);
#pragma unroll
        for (int s = 0; s < 2; ++s)
          dst[i][s] = (e < N) ? *reinterpret_cast<const uint4*>(wg + size_t(e) * d + k0 + 32 * s + 8 * (lane >> 4))
                              : make_uint4(0, 0, 0, 0);
      }
    };
    auto load_x = [&](int k0, uint4 (&dst)[XPT]) {
#pragma unroll
      for (int r = 0; r < XPT; ++r) {
        const int c = tid + RT_THREADS * r;
        const int tok = t0 + (c >> 3);
        dst[r] = (c < XCH && tok < a.T) ? *reinterpret_cast<const uint4*>(xg + size_t(tok) * d + k0 + 8 * (c & 7))
                                        : make_uint4(0, 0, 0, 0);
      }
    };
    auto store_x = [&](int buf, const uint4 (&src)[XPT]) {
#pragma unroll
      for (int r = 0; r < XPT; ++r) {
        const int c = tid + RT_THREADS * r;
        if (c < XCH) {
          const uint4 v = src[r];
          const float f[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                              bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
#pragma unroll
          for (int j = 0; j < 8; ++j) xsq[r] = fmaf(f[j], f[j], xsq[r]);
          *reinterpret_cast<uint4*>(sx + (buf * BT + (c >> 3)) * RT_XLD + 8 * (c & 7)) = v;
        }
      }
    };

    const int nk = d / RT_BK;
    auto step = [&](auto bufc, int kt, uint4 (&acur)[4][2], uint4 (&xcur)[XPT], uint4 (&xnext)[XPT]) {
      constexpr int buf = decltype(bufc)::value;
      const uint16_t* xb = sx + buf * BT * RT_XLD;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8_t bx[TB];
#pragma unroll
        for (int j = 0; j < TB; ++j)
          bx[j] = *reinterpret_cast<const bf16x8_t*>(xb + (16 * j + (lane & 15)) * RT_XLD + 32 * s + 8 * (lane >> 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (wave + 4 * i < NB) {
            const uint4 av = acur[i][s];
            const float f[8] = {bf16lo(av.x), bf16hi(av.x), bf16lo(av.y), bf16hi(av.y),
                                bf16lo(av.z), bf16hi(av.z), bf16lo(av.w), bf16hi(av.w)};
#pragma unroll
            for (int j = 0; j < 8; ++j) wsq[i] = fmaf(f[j], f[j], wsq[i]);
            const bf16x8_t ab = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
            for (int j = 0; j < TB; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bx[j], acc[i][j], 0, 0, 0);
          }
        }
      }
      // the gate fragments and token chunks of step kt are consumed: fetch
      // step kt+2 into their registers, then publish step kt+1 to LDS
      if (kt + 2 < nk) {
        load_a((kt + 2) * RT_BK, acur);
        load_x((kt + 2) * RT_BK, xcur);
      }
      if (kt + 1 < nk) store_x(buf ^ 1, xnext);
      __syncthreads();
    };

    load_x(0, xr0);
    load_a(0, afr0);
    if (nk > 1) {
      load_x(RT_BK, xr1);
      load_a(RT_BK, afr1);
    }
    store_x(0, xr0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      step(std::integral_constant<int, 0>{}, kt, afr0, xr0, xr1);
      if (kt + 1 < nk) step(std::integral_constant<int, 1>{}, kt + 1, afr1, xr1, xr0);
    }
    // |x_t|^2: 8 threads share a token row per pipeline step
#pragma unroll
    for (int r = 0; r < XPT; ++r) {
      float v = xsq[r];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      const int c = tid + RT_THREADS * r;
      if ((tid & 7) == 0 && c < XCH) sX2[c >> 3] = v;
    }
    // max_e |w_e|^2: lanes l, l^16, l^32, l^48 hold the same expert
    float wm = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = wsq[i];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      wm = fmaxf(wm, v);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o, 64));
    if (lane == 0) sWmax[wave] = wm;
    // logits -> LDS (the token tile is dead after the last barrier)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = wave + 4 * i;
      if (b < NB) {
#pragma unroll
        for (int j = 0; j < TB; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sL[(16 * j + (lane & 15)) * LS + 16 * b + 4 * (lane >> 4) + r] = acc[i][j][r];
      }
    }
    depth = d / 32 + 32;
  } else {
    // fp32 activations: one sequential FMA chain per (token, expert)
    const float* xf = reinterpret_cast<const float*>(a.x);
    const float* wf = reinterpret_cast<const float*>(a.w_gate);
    for (int p = tid; p < BT * N; p += RT_THREADS) {
      const int tl = p / N, e = p - tl * N;
      const int tok = t0 + tl;
      float s = 0.f;
      if (tok < a.T) {
        const float* xrow = xf + size_t(tok) * d;
        const float* wrow = wf + size_t(e) * d;
        for (int i = 0; i < d; ++i) s = fmaf(xrow[i], wrow[i], s);
      }
      sL[tl * LS + e] = s;
    }
    for (int tl = tid; tl < BT; tl += RT_THREADS) {
      const int tok = t0 + tl;
      float s = 0.f;
      if (tok < a.T) {
        const float* xrow = xf + size_t(tok) * d;
        for (int i = 0; i < d; ++i) s = fmaf(xrow[i], xrow[i], s);
      }
      sX2[tl] = s;
    }
    float wm = 0.f;
    for (int e = tid; e < N; e += RT_THREADS) {
      const float* wrow = wf + size_t(e) * d;
      float s = 0.f;
      for (int i = 0; i < d; ++i) s = fmaf(wrow[i], wrow[i], s);
      wm = fmaxf(wm, s);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o, 64));
    if (lane == 0) sWmax[wave] = wm;
    depth = d;
  }
  __syncthreads();

  // ---- fp32 decision: 4 threads per token
  {
    const float u = 2.384185791015625e-07f;  // 2^-22
    const float Du = depth * u;
    const float gamma = Du / (1.f - Du);
    const float wmax = sqrtf(fmaxf(fmaxf(sWmax[0], sWmax[1]), fmaxf(sWmax[2], sWmax[3])));
    const int tl = tid >> 2, q = tid & 3;
    if (tl < BT) {  // whole waves
      const float tau = 2.02f * gamma * sqrtf(sX2[tl]) * wmax;
      const int kk = min(k + 1, N);
      bool flag = false;
      const float* Lrow = sL + tl * LS;
      decide(Lrow, N, k, kk, a.renorm, tau, q, sIdx[tl], sGate[tl], &sThr[tl], &sMax[tl], &sSum[tl], &flag);
      if (q == 0 && flag && t0 + tl < a.T) sFlag[atomicAdd(&sNF, 1)] = tl;
    }
  }
  __syncthreads();

  // ---- exact order of the near-tied tokens: candidates recomputed in fp64
  const int nf = sNF;
  for (int f = wave; f < nf; f += RT_THREADS / 64) {
    const int tl = sFlag[f];
    const float thr = sThr[tl];
    const float* Lrow = sL + tl * LS;
    const size_t xo = size_t(t0 + tl) * d;
    double cv[RT_KMAX];
    int ci[RT_KMAX];
#pragma unroll
    for (int j = 0; j < RT_KMAX; ++j) { cv[j] = -INFINITY; ci[j] = 0x7fffffff; }
    for (int u = 0; u < 4; ++u) {
      const int e0 = lane + 64 * u;
      const bool cand = e0 < N && Lrow[e0] >= thr;
      uint64_t m = __ballot(cand);
      while (m) {
        const int bit = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        const int e = 64 * u + bit;
        // lane owns elements 8*lane .. 8*lane+7 of each 512-wide chunk; the
        // chunks' loads are issued four at a time before they are used
        double s = 0.0;
        for (int i0 = 0; i0 < d; i0 += 4 * 512) {
          float xv[4][8], wv[4][8];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = i0 + 512 * u + 8 * lane;
            if (i < d) {
              load8<ACT>(a.x, xo + i, xv[u]);
              load8<ACT>(a.w_gate, size_t(e) * d + i, wv[u]);
            }
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (i0 + 512 * u + 8 * lane < d) {
#pragma unroll
              for (int j = 0; j < 8; ++j) s = fma((double)xv[u][j], (double)wv[u][j], s);
            }
          }
        }
        s = wave_sum(s);
        topk_insert<RT_KMAX>(cv, ci, s, e);
      }
    }
    if (lane == 0) {
      const float mx = sMax[tl], se = sSum[tl];
      float g[RT_KMAX];
      float gs = 0.f;
#pragma unroll
      for (int j = 0; j < RT_KMAX; ++j) {
        g[j] = (j < k) ? __expf(Lrow[ci[j] < N ? ci[j] : 0] - mx) / se : 0.f;
        gs += g[j];
      }
#pragma unroll
      for (int j = 0; j < RT_KMAX; ++j)
        if (j < k) {
          sIdx[tl][j] = ci[j] < N ? ci[j] : 0;
          sGate[tl][j] = a.renorm ? g[j] / gs : g[j];
        }
    }
  }
  __syncthreads();

  for (int p = tid; p < BT * k; p += RT_THREADS) {
    const int tl = p / k, j = p - tl * k;
    const int tok = t0 + tl;
    if (tok < a.T) {
      a.topk_idx[size_t(tok) * k + j] = sIdx[tl][j];
      a.topk_gate[size_t(tok) * k + j] = sGate[tl][j];
    }
  }
}

template <int BT>
static size_t route_lds_bytes(int N) {
  const int NB = (N + 15) >> 4;
  const size_t logits = size_t(BT) * (NB * 16 + 4) * sizeof(float);
  const size_t tiles = size_t(2) * BT * RT_XLD * sizeof(uint16_t);
  return logits > tiles ? logits : tiles;
}

template <int BT>
static hipError_t launch_route_bt(const RouteArgs& a, int act, hipStream_t s) {
  const int grid = (a.T + BT - 1) / BT;
  const size_t lds = route_lds_bytes<BT>(a.N);
  static int attr_done[64] = {0};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  auto kb = route_kernel<ACT_BF16, BT>;
  auto kf = route_kernel<ACT_F32, BT>;
  if (dev < 0 || dev >= 64 || !attr_done[dev]) {
    const int mx = int(route_lds_bytes<BT>(256));
    err = hipFuncSetAttribute((const void*)kb, hipFuncAttributeMaxDynamicSharedMemorySize, mx);
    if (err == hipSuccess) err = hipFuncSetAttribute((const void*)kf, hipFuncAttributeMaxDynamicSharedMemorySize, mx);
    if (err != hipSuccess) return err;
    if (dev >= 0 && dev < 64) attr_done[dev] = 1;
  }
  if (act == ACT_BF16)
    hipLaunchKernelGGL(kb, dim3(grid), dim3(RT_THREADS), lds, s, a);
  else
    hipLaunchKernelGGL(kf, dim3(grid), dim3(RT_THREADS), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, int act, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  // 64-token tiles once they give every CU a workgroup, 16-token tiles below
  if (a.T >= 64 * 256) return launch_route_bt<64>(a, act, s);
  return launch_route_bt<16>(a, act, s);
}

// ------------------------------------------------------------------ bucketing
// One workgroup per expert e.  Pass 1 counts the routed slots of experts below
// e (its first bucket position); pass 2 walks all slots in order and appends
// the ones routed to e, so within an expert slots ascend.
constexpr int BK_THREADS = 1024;

__global__ __launch_bounds__(BK_THREADS) void bucket_kernel(BucketArgs a) {
  __shared__ int s_w[BK_THREADS / 64];
  __shared__ int s_off;
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // optional: unpack the 2-bit substrate (16 weights per word) into one byte
  // per weight holding the high byte of its bf16 value scaled by 1/2
  // (+1 -> 0x3F, -1 -> 0xBF, 0 -> 0), or into fp4 e2m1 nibbles (+1 -> 0x2,
  // -1 -> 0xA, 0 -> 0; weight 2b in the low nibble of byte b)
  for (int w = e * BK_THREADS + tid; w < a.w_words; w += gridDim.x * BK_THREADS) {
    const uint32_t P = a.w_packed[w];
    uint32_t code[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int j = c >> 1, h = c & 1;
      const uint32_t nz = (P >> (16 * h + j)) & 1u, sg = (P >> (16 * h + 8 + j)) & 1u;
      code[c] = a.w_fp4 ? nz * (0x2u | (sg << 3)) : nz * (0x3Fu | (sg << 7));
    }
    if (a.w_fp4) {
      uint32_t o[2] = {0u, 0u};
#pragma unroll
      for (int c = 0; c < 16; ++c) o[c >> 3] |= code[c] << (4 * (c & 7));
      reinterpret_cast<uint2*>(a.w_bytes)[w] = make_uint2(o[0], o[1]);
    } else {
      uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int c = 0; c < 16; ++c) o[c >> 2] |= code[c] << (8 * (c & 3));
      reinterpret_cast<uint4*>(a.w_bytes)[w] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }

  auto load4 = [&](int f0) -> int4 {
    if (f0 + 3 < a.R) return *reinterpret_cast<const int4*>(a.topk_idx + f0);
    int4 q;
    q.x = (f0 + 0 < a.R) ? a.topk_idx[f0 + 0] : 0x7fffffff;
    q.y = (f0 + 1 < a.R) ? a.topk_idx[f0 + 1] : 0x7fffffff;
    q.z = (f0 + 2 < a.R) ? a.topk_idx[f0 + 2] : 0x7fffffff;
    q.w = (f0 + 3 < a.R) ? a.topk_idx[f0 + 3] : 0x7fffffff;
    return q;
  };

  // The routed slots are read in blocks of BK_BATCH int4 per thread, all
  // loads of a block issued before any is used.
  constexpr int BK_BATCH = 8;
  const int span = 4 * BK_THREADS * BK_BATCH;
  int lt = 0;
  for (int b0 = 0; b0 < a.R; b0 += span) {
    int4 q[BK_BATCH];
#pragma unroll
    for (int b = 0; b < BK_BATCH; ++b) q[b] = load4(b0 + 4 * (b * BK_THREADS + tid));
#pragma unroll
    for (int b = 0; b < BK_BATCH; ++b) lt += (q[b].x < e) + (q[b].y < e) + (q[b].z < e) + (q[b].w < e);
  }
  lt = wave_sum(lt);
  if (lane == 0) s_w[wave] = lt;
  __syncthreads();
  if (tid == 0) {
    int o = 0;
    for (int w = 0; w < BK_THREADS / 64; ++w) o += s_w[w];
    s_off = o;
    a.offsets[e] = o;
    if (e == a.N - 1) a.offsets[a.N] = a.R;
  }
  __syncthreads();
  const int off = s_off;
  const uint64_t ltmask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int running = 0;
  for (int b0 = 0; b0 < a.R; b0 += span) {
    int4 qb[BK_BATCH];
#pragma unroll
    for (int b = 0; b < BK_BATCH; ++b) qb[b] = load4(b0 + 4 * (b * BK_THREADS + tid));
#pragma unroll
    for (int b = 0; b < BK_BATCH; ++b) {
      const int f0 = b0 + 4 * (b * BK_THREADS + tid);
      if (b0 + 4 * b * BK_THREADS >= a.R) break;  // uniform
      const int v[4] = {qb[b].x, qb[b].y, qb[b].z, qb[b].w};
      int c = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) c += (v[j] == e);
      const uint64_t m0 = __ballot(c & 1), m1 = __ballot(c & 2), m2 = __ballot(c & 4);
      const int lpre = __popcll(m0 & ltmask) + 2 * __popcll(m1 & ltmask) + 4 * __popcll(m2 & ltmask);
      const int wtot = __popcll(m0) + 2 * __popcll(m1) + 4 * __popcll(m2);
      __syncthreads();
      if (lane == 0) s_w[wave] = wtot;
      __syncthreads();
      int wpre = 0, tot = 0;
      for (int w = 0; w < BK_THREADS / 64; ++w) {
        const int x = s_w[w];
        wpre += (w < wave) ? x : 0;
        tot += x;
      }
      if (c) {
        int qq = off + running + wpre + lpre;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (v[j] == e) a.perm[qq++] = f0 + j;
      }
      running += tot;
    }
  }
}

hipError_t launch_bucket(const BucketArgs& a, hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  hipLaunchKernelGGL(bucket_kernel, dim3(a.N), dim3(BK_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace bmoe
