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
  return (v > bv) | ((v == bv) & (i < bi));
}
__device__ __forceinline__ bool better(double v, int i, double bv, int bi) {
  return (v > bv) | ((v == bv) & (i < bi));
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

// Per-workgroup state of the decision phase.
template <int BT>
struct RouteSh {
  float X2[BT];               // |x_t|^2
  int Idx[BT][RT_KMAX];
  float Gate[BT][RT_KMAX];
  float Thr[BT], Max[BT], Sum[BT];
  int Flag[BT];
  int NF;
  float Wmax[8];              // max_e |w_e|^2 seen by each wave (unused entries 0)
  // the tile's slot sort (routed slots in groups of 64)
  int Cnt[256];                                         // first list position of each expert
  __attribute__((aligned(4))) uint8_t Cg[(BT * RT_KMAX + 63) / 64 * 256];  // per-group expert counts
  uint8_t Sx[BT * RT_KMAX], Sr[BT * RT_KMAX];           // slot's expert, rank in its group
};

// Per-token decision, 16 lanes per token (four tokens per wave at a time):
// lane j of the token's group holds the logits of experts j, j+16, ...,
// j+16(NR-1) in registers.  Round r takes the best remaining entry (larger
// value, then lower index) over the group in four shuffle steps and its owner
// marks it taken, so kk rounds give the sorted top-kk.  The group's lane 0
// writes idx/gates of the fp32 decision; returns whether a decisive gap is
// within the error bound.
template <int NR>
__device__ __forceinline__ bool decide16(const float* Lrow, bool valid, int N, int k, int kk, int renorm,
                                         float tau, int j, int* out_idx, float* out_gate, float* out_thr,
                                         float* out_max, float* out_sum) {
  float v[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int e = j + 16 * r;
    v[r] = (valid && e < N) ? Lrow[e] : -INFINITY;
  }
  uint32_t taken = 0;
  float tv[RT_KMAX + 1];
  int ti[RT_KMAX + 1];
#pragma unroll
  for (int rr = 0; rr < RT_KMAX + 1; ++rr) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    if (rr < kk) {  // uniform
      int br = 0;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int e = j + 16 * r;
        const bool c = (e < N) & (((taken >> r) & 1u) == 0u) & better(v[r], e, bv, bi);
        bv = c ? v[r] : bv;
        bi = c ? e : bi;
        br = c ? r : br;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        const bool c = better(ov, oi, bv, bi);
        bv = c ? ov : bv;
        bi = c ? oi : bi;
      }
      taken |= (j + 16 * br == bi) ? (1u << br) : 0u;
    }
    tv[rr] = bv;
    ti[rr] = bi;
  }
  const float mx = tv[0];
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) s += (j + 16 * r < N) ? __expf(v[r] - mx) : 0.f;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
  bool f = false;
  if (j == 0 && valid) {
    const int ngap = min(k, N - 1);
    float g[RT_KMAX];
    float gs = 0.f;
    float kth = tv[0];
#pragma unroll
    for (int q = 0; q < RT_KMAX; ++q) {
      f |= (q < ngap) & (tv[q] - tv[q + 1] < tau);
      g[q] = (q < k) ? __expf(tv[q] - mx) / s : 0.f;
      gs += g[q];
      kth = (q == k - 1) ? tv[q] : kth;
    }
#pragma unroll
    for (int q = 0; q < RT_KMAX; ++q) {
      if (q < k) {
        out_idx[q] = ti[q];
        out_gate[q] = renorm ? g[q] / gs : g[q];
      }
    }
    *out_thr = kth - tau;
    *out_max = mx;
    *out_sum = s;
  }
  return f;
}

template <int BT, int NR, int NT>
__device__ __forceinline__ void decide_all(const RouteArgs& a, RouteSh<BT>& sh, const float* sL, int LS,
                                           float gamma, float wmax, int t0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kk = min(a.k + 1, a.N);
  const int j = lane & 15;
#pragma unroll
  for (int tl0 = 0; tl0 < BT; tl0 += NT / 16) {
    const int tl = tl0 + 4 * wave + (lane >> 4);
    if (tl < BT) {  // whole 16-lane groups
      const bool valid = t0 + tl < a.T;
      const float tau = 2.02f * gamma * sqrtf(sh.X2[tl]) * wmax;
      const bool flag = decide16<NR>(sL + tl * LS, valid, a.N, a.k, kk, a.renorm, tau, j, sh.Idx[tl],
                                     sh.Gate[tl], &sh.Thr[tl], &sh.Max[tl], &sh.Sum[tl]);
      if (j == 0 && flag && valid) sh.Flag[atomicAdd(&sh.NF, 1)] = tl;
    }
  }
}

__device__ __forceinline__ float route_gamma(int depth) {
  const float u = 2.384185791015625e-07f;  // 2^-22
  const float Du = depth * u;
  return Du / (1.f - Du);
}

template <int BT>
__device__ __forceinline__ float route_wmax(const RouteSh<BT>& sh) {
  float w = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) w = fmaxf(w, sh.Wmax[i]);
  return sqrtf(w);
}

// Decision from the logits in LDS (row stride LS), after X2 / Wmax are set.
// Starts and ends with a barrier.
template <int BT, int NT>
__device__ __forceinline__ void route_decide(const RouteArgs& a, RouteSh<BT>& sh, const float* sL, int LS,
                                             int depth, int t0) {
  const int N = a.N;
  __syncthreads();
  const float gamma = route_gamma(depth), wmax = route_wmax(sh);
  if (N <= 16) decide_all<BT, 1, NT>(a, sh, sL, LS, gamma, wmax, t0);
  else if (N <= 32) decide_all<BT, 2, NT>(a, sh, sL, LS, gamma, wmax, t0);
  else if (N <= 64) decide_all<BT, 4, NT>(a, sh, sL, LS, gamma, wmax, t0);
  else if (N <= 128) decide_all<BT, 8, NT>(a, sh, sL, LS, gamma, wmax, t0);
  else decide_all<BT, 16, NT>(a, sh, sL, LS, gamma, wmax, t0);
  __syncthreads();
}

// Exact re-ranking of the flagged (near-tied) tokens and output of the tile.
// Expects the decision state and the logits in LDS, synchronised.
template <int ACT, int BT, int NT>
__device__ __forceinline__ void route_recheck_store(const RouteArgs& a, RouteSh<BT>& sh, const float* sL, int LS,
                                                    int t0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N, d = a.d, k = a.k;
  const int nf = sh.NF;
  for (int i = tid; i < int(sizeof(sh.Cg)) / 4; i += NT) reinterpret_cast<uint32_t*>(sh.Cg)[i] = 0;
  for (int f = wave; f < nf; f += NT / 64) {
    const int tl = sh.Flag[f];
    const float thr = sh.Thr[tl];
    const float* Lrow = sL + tl * LS;
    const size_t xo = size_t(t0 + tl) * d;
    double cv[RT_KMAX];
    int ci[RT_KMAX];
#pragma unroll
    for (int j = 0; j < RT_KMAX; ++j) { cv[j] = -INFINITY; ci[j] = 0x7fffffff; }
    // candidates (fp32 logit >= thr) in batches of four, in expert order over
    // the whole row: the token's and the four gate rows' chunks are loaded
    // together (lane owns elements 8 lane .. 8 lane + 7 of each 512-wide
    // chunk), one fp64 sum per candidate
    uint64_t m[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e0 = lane + 64 * u;
      m[u] = __ballot(e0 < N && Lrow[e0] >= thr);
    }
    int u = 0;
    while (true) {
      int eb[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        while (u < 4 && !m[u]) ++u;  // uniform
        if (u < 4) {
          eb[c] = 64 * u + __ffsll((unsigned long long)m[u]) - 1;
          m[u] &= m[u] - 1;
        } else {
          eb[c] = -1;
        }
      }
      if (eb[0] < 0) break;
      double s4[4] = {0.0, 0.0, 0.0, 0.0};
      for (int i0 = 0; i0 < d; i0 += 512) {
        const int i = i0 + 8 * lane;
        if (i < d) {
          float xv[8], wv[4][8];
          load8<ACT>(a.x, xo + i, xv);
#pragma unroll
          for (int c = 0; c < 4; ++c) load8<ACT>(a.w_gate, size_t(eb[c] < 0 ? eb[0] : eb[c]) * d + i, wv[c]);
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int j = 0; j < 8; ++j) s4[c] = fma((double)xv[j], (double)wv[c][j], s4[c]);
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double s = wave_sum(s4[c]);
        if (eb[c] >= 0) topk_insert<RT_KMAX>(cv, ci, s, eb[c]);
      }
    }
    if (lane == 0) {
      const float mx = sh.Max[tl], se = sh.Sum[tl];
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
          sh.Idx[tl][j] = ci[j] < N ? ci[j] : 0;
          sh.Gate[tl][j] = a.renorm ? g[j] / gs : g[j];
        }
    }
  }
  __syncthreads();

  // outputs, and the tile's routed slots ordered by expert (a stable counting
  // sort; the bucketing kernel concatenates the tiles' lists per expert).
  // Slots go in groups of 64 (one per wave and round): a slot's rank among
  // the group's slots of its expert comes from eight ballots over the expert
  // bits, the groups' per-expert counts from LDS.  The global stores all come
  // after the last barrier, which would wait for them.
  const int ns = min(BT, a.T - t0) * k;
  const int ng = (ns + 63) >> 6;
  const size_t s0 = size_t(t0) * k;
  for (int p0 = 0; p0 < ns; p0 += NT) {
    const int p = p0 + tid;
    const bool act = p < ns;
    int e = 0;
    if (act) {
      const int tl = p / k, j = p - tl * k;
      e = sh.Idx[tl][j];
    }
    uint64_t peers = __ballot(act);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    if (act) {
      const int r = __popcll(peers & ((1ull << lane) - 1ull));
      sh.Sx[p] = uint8_t(e);
      sh.Sr[p] = uint8_t(r);
      if (r == 0) sh.Cg[(p >> 6) * 256 + e] = uint8_t(__popcll(peers));
    }
  }
  __syncthreads();
  // first list positions: wave 0, lane l owns experts 4l .. 4l + 3 (N <= 256)
  int st[4] = {0, 0, 0, 0};
  if (wave == 0) {
    int c[4] = {0, 0, 0, 0};
    for (int g = 0; g < ng; ++g) {
      const uint32_t q = *reinterpret_cast<const uint32_t*>(&sh.Cg[g * 256 + 4 * lane]);
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] += (q >> (8 * i)) & 0xFF;
    }
    const int own = c[0] + c[1] + c[2] + c[3];
    int x = own;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    int pre = x - own;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st[i] = pre;
      sh.Cnt[4 * lane + i] = pre;
      pre += c[i];
    }
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * lane + i < N) a.tile_start[size_t(blockIdx.x) * N + 4 * lane + i] = st[i];
  }
  for (int p = tid; p < ns; p += NT) {
    const int tl = p / k, j = p - tl * k;
    const int e = sh.Sx[p];
    int r = sh.Cnt[e] + sh.Sr[p];
    for (int g = 0; g < (p >> 6); ++g) r += sh.Cg[g * 256 + e];
    const float gv = sh.Gate[tl][j];
    a.topk_idx[s0 + p] = e;
    a.topk_gate[s0 + p] = gv;
    a.tile_slots[s0 + r] = int32_t(s0) + p;
    a.tile_gates[s0 + r] = gv;
  }
}

// max over the workgroup's gate rows of |w_e|^2 from per-lane partial sums:
// lanes l, l^16, l^32, l^48 hold the same expert
template <int NI>
__device__ __forceinline__ void publish_wmax(const float (&wsq)[NI], float* Wmax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float wm = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float v = wsq[i];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    wm = fmaxf(wm, v);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o, 64));
  if (lane == 0) Wmax[wave] = wm;
}

// Order-preserving 64-bit key of (logit, expert): larger logit first, then
// lower expert index.  Key 0 lies below every real logit.
__device__ __forceinline__ uint64_t rkey(float v, int e) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t(u) << 32) | uint32_t(0xFFFFFFFFu - uint32_t(e));
}
__device__ __forceinline__ float rkey_val(uint64_t k) {
  uint32_t u = uint32_t(k >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}
__device__ __forceinline__ int rkey_idx(uint64_t k) { return int(0xFFFFFFFFu - uint32_t(k)); }

// insert into a descending list of three distinct keys
__device__ __forceinline__ void top3_insert(uint64_t (&t)[3], uint64_t k) {
  const bool c0 = k > t[0], c1 = k > t[1], c2 = k > t[2];
  t[2] = c1 ? t[1] : (c2 ? k : t[2]);
  t[1] = c0 ? t[0] : (c1 ? k : t[1]);
  t[0] = c0 ? k : t[0];
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = __shfl_xor(uint32_t(v), o, 64), hi = __shfl_xor(uint32_t(v >> 32), o, 64);
  return (uint64_t(hi) << 32) | lo;
}

// ----------------------------------------------------------------------------
// Any width: bf16 tokens stream through two LDS steps of 64 contraction
// indices (pipelined), fp32 tokens use one FMA chain per logit.
template <int ACT, int BT, int NW>
__global__ __launch_bounds__(64 * NW) void route_kernel(RouteArgs a) {
  constexpr int NT = 64 * NW;                 // threads
  constexpr int NI = 16 / NW;                 // expert blocks per wave (256 experts at most)
  constexpr int TB = BT / 16;                 // token blocks of 16
  constexpr int XCH = BT * (RT_BK / 8);       // 16-byte chunks of the token tile per step
  constexpr int XPT = (XCH + NT - 1) / NT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sx = reinterpret_cast<uint16_t*>(smem);  // [2][BT][RT_XLD] token tile (bf16)
  float* sL = reinterpret_cast<float*>(smem);         // [BT][LS] logits (after the K loop)
  __shared__ RouteSh<BT> sh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * BT;
  const int N = a.N, d = a.d;
  const int NB = (N + 15) >> 4;
  const int LS = NB * 16 + 4;  // logit row stride
  if (tid == 0) sh.NF = 0;

  int depth;
  if constexpr (ACT == ACT_BF16) {
    const uint16_t* xg = reinterpret_cast<const uint16_t*>(a.x);
    const uint16_t* wg = reinterpret_cast<const uint16_t*>(a.w_gate);
    // wave w owns expert blocks b = w + NW i (i < NI) and all token blocks
    f32x4_t acc[NI][TB];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < TB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float wsq[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) wsq[i] = 0.f;
    float xsq[XPT];
#pragma unroll
    for (int r = 0; r < XPT; ++r) xsq[r] = 0.f;
    // two register sets (compile-time indexed): gate-weight fragments and
    // token chunks two steps ahead
    uint4 afr0[NI][2], afr1[NI][2];
    uint4 xr0[XPT], xr1[XPT];

    // loads are unconditional (a branch around loads in the K loop makes every
    // wait a full drain): experts past N read row N-1, tokens past T row T-1,
    // chunk indices past the tile chunk XCH-1; none of these is used
    // gate fragments of block wave + 4 i, k-step st at abase[i] + st * astep:
    // one contiguous 1 KiB per wave from the fragment copy, else 16 rows of 64
    // bytes from W_g (blocks past the last read the last one)
    const uint16_t* abase[NI];
    const int astep = a.w_frag ? 512 : 32;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int b = min(wave + NW * i, NB - 1);
      abase[i] = a.w_frag ? reinterpret_cast<const uint16_t*>(a.w_frag) + (size_t(b) * (d / 32) * 64 + lane) * 8
                          : wg + size_t(min(16 * b + (lane & 15), N - 1)) * d + 8 * (lane >> 4);
    }
    auto load_a = [&](int k0, uint4 (&dst)[NI][2]) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          dst[i][s] = *reinterpret_cast<const uint4*>(abase[i] + (k0 / 32 + s) * astep);
    };
    auto load_x = [&](int k0, uint4 (&dst)[XPT]) {
#pragma unroll
      for (int r = 0; r < XPT; ++r) {
        const int c = min(tid + NT * r, XCH - 1);
        const int tok = min(t0 + (c >> 3), a.T - 1);
        dst[r] = *reinterpret_cast<const uint4*>(xg + size_t(tok) * d + k0 + 8 * (c & 7));
      }
    };
    auto store_x = [&](int buf, const uint4 (&src)[XPT]) {
#pragma unroll
      for (int r = 0; r < XPT; ++r) {
        const int c = tid + NT * r;
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
    auto step = [&](auto bufc, int kt, uint4 (&acur)[NI][2], uint4 (&xcur)[XPT], uint4 (&xnext)[XPT]) {
      constexpr int buf = decltype(bufc)::value;
      const uint16_t* xb = sx + buf * BT * RT_XLD;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8_t bx[TB];
#pragma unroll
        for (int j = 0; j < TB; ++j)
          bx[j] = *reinterpret_cast<const bf16x8_t*>(xb + (16 * j + (lane & 15)) * RT_XLD + 32 * s + 8 * (lane >> 4));
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if (wave + NW * i < NB) {
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
      // step kt+2 into their registers (past the end: the last step again,
      // unused), then publish step kt+1 to LDS
      load_a(min(kt + 2, nk - 1) * RT_BK, acur);
      load_x(min(kt + 2, nk - 1) * RT_BK, xcur);
      if (kt + 1 < nk) store_x(buf ^ 1, xnext);
      __syncthreads();
    };

    load_x(0, xr0);
    load_a(0, afr0);
    load_x(min(1, nk - 1) * RT_BK, xr1);
    load_a(min(1, nk - 1) * RT_BK, afr1);
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
      const int c = tid + NT * r;
      if ((tid & 7) == 0 && c < XCH) sh.X2[c >> 3] = v;
    }
    publish_wmax(wsq, sh.Wmax);
    // logits -> LDS (the token tile is dead after the last barrier)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int b = wave + NW * i;
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
    for (int p = tid; p < BT * N; p += NT) {
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
    for (int tl = tid; tl < BT; tl += NT) {
      const int tok = t0 + tl;
      float s = 0.f;
      if (tok < a.T) {
        const float* xrow = xf + size_t(tok) * d;
        for (int i = 0; i < d; ++i) s = fmaf(xrow[i], xrow[i], s);
      }
      sh.X2[tl] = s;
    }
    float wm = 0.f;
    for (int e = tid; e < N; e += NT) {
      const float* wrow = wf + size_t(e) * d;
      float s = 0.f;
      for (int i = 0; i < d; ++i) s = fmaf(wrow[i], wrow[i], s);
      wm = fmaxf(wm, s);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o, 64));
    if (lane == 0) sh.Wmax[wave] = wm;
    depth = d;
  }
  if (tid < 8 - NW) sh.Wmax[NW + tid] = 0.f;  // entries of waves this workgroup does not have
  route_decide<BT, NT>(a, sh, sL, LS, depth, t0);
  route_recheck_store<ACT, BT, NT>(a, sh, sL, LS, t0);
}

// ----------------------------------------------------------------------------
// bf16 tokens, width d = 64 NK, the whole token tile in LDS.  Eight waves:
// wave w owns expert blocks w (and w + 8 when NI = 2; 16 experts each) and
// holds its whole share of the gate matrix in registers (at most 128 per
// lane), loaded at the start together with the
// token tile; the contraction loop is unrolled at compile time.  For k <= 2
// the top-(k+1) is taken from the accumulators: each lane keeps the three best
// (logit, expert) keys of its experts per token, the four lanes of a token
// merge theirs by shuffles, the waves' lists meet in LDS.  Larger k uses the
// decision over the logits in LDS.
constexpr int RW_THREADS = 512;
constexpr int RW_WAVES = RW_THREADS / 64;

template <int BT, int NK, int NI>
__global__ __launch_bounds__(RW_THREADS) void route_whole_kernel(RouteArgs a) {
  constexpr int TB = BT / 16;
  constexpr int D = NK * RT_BK;
  constexpr int KS = D / 32;                          // MFMA k-steps
  constexpr int XST = D + 8;                          // LDS row stride (bf16)
  constexpr int CPR = D / 8;                          // 16-byte chunks per row
  constexpr int NCH = BT * CPR;
  constexpr int CPT = (NCH + RW_THREADS - 1) / RW_THREADS;
  constexpr int G = CPR < 64 ? CPR : 64;              // lanes sharing a row in one load
  static_assert(NI == 1 || NI == 2, "expert blocks per wave");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sx = reinterpret_cast<uint16_t*>(smem);  // [BT][XST] token tile
  float* sL = reinterpret_cast<float*>(smem);         // [BT][LS] logits (after the contraction)
  __shared__ RouteSh<BT> sh;
  __shared__ uint64_t sTop[BT][RW_WAVES][3];
  __shared__ float sPart[BT][RW_WAVES];
  __shared__ int sTflag[BT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * BT;
  const int N = a.N, k = a.k;
  const int NB = (N + 15) >> 4;
  const int LS = NB * 16 + 4;
  const uint16_t* xg = reinterpret_cast<const uint16_t*>(a.x);
  const uint16_t* wg = reinterpret_cast<const uint16_t*>(a.w_gate);
  if (tid == 0) sh.NF = 0;
  if (tid < BT) sh.X2[tid] = 0.f;

  // token tile and this wave's gate rows (block b = wave + 8 i, k-step st, 8
  // values per lane), all loads issued before any wait.  The loads are
  // unconditional (a branch around a load makes the wait at its join a full
  // drain): chunks past the tile read its last chunk, tokens past T row T-1,
  // experts past N row N-1 (or zeros in the fragment copy), blocks past the
  // last the last one; none of these values reaches an output (tokens past T
  // are never stored, experts past N never ranked, blocks past the last never
  // multiplied, and a repeated row leaves max_e |w_e| unchanged).
  uint4 xv[CPT];
#pragma unroll
  for (int r = 0; r < CPT; ++r) {
    const int c = min(r * RW_THREADS + tid, NCH - 1);
    const int tok = min(t0 + c / CPR, a.T - 1);
    xv[r] = *reinterpret_cast<const uint4*>(xg + size_t(tok) * D + 8 * (c % CPR));
  }
  bool bval[NI];
  uint4 A[NI][KS];
  const int astep = a.w_frag ? 512 : 32;  // fragment copy: 1 KiB per wave per k-step
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int b = wave + RW_WAVES * i, bc = min(b, NB - 1);
    bval[i] = b < NB;
    const uint16_t* ab = a.w_frag ? reinterpret_cast<const uint16_t*>(a.w_frag) + (size_t(bc) * KS * 64 + lane) * 8
                                  : wg + size_t(min(16 * bc + l16, N - 1)) * D + 8 * g;
#pragma unroll
    for (int st = 0; st < KS; ++st) A[i][st] = *reinterpret_cast<const uint4*>(ab + st * astep);
  }
  // tile -> LDS; |x|^2 partial sums reduced over the lanes sharing a row
  float xs[CPT];
#pragma unroll
  for (int r = 0; r < CPT; ++r) {
    const int c = r * RW_THREADS + tid;
    const uint4 q = xv[r];
    float ss = 0.f;
    ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x), __builtin_bit_cast(bf16x2_t, q.x), ss, false);
    ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y), __builtin_bit_cast(bf16x2_t, q.y), ss, false);
    ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z), __builtin_bit_cast(bf16x2_t, q.z), ss, false);
    ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w), __builtin_bit_cast(bf16x2_t, q.w), ss, false);
    xs[r] = ss;
    if (c < NCH) *reinterpret_cast<uint4*>(sx + (c / CPR) * XST + 8 * (c % CPR)) = q;
  }
#pragma unroll
  for (int r = 0; r < CPT; ++r)
#pragma unroll
    for (int o = 1; o < G; o <<= 1) xs[r] += __shfl_xor(xs[r], o, 64);
  __syncthreads();  // tile in LDS, X2 cleared
#pragma unroll
  for (int r = 0; r < CPT; ++r) {
    const int c = r * RW_THREADS + tid;
    if (c < NCH && (lane % G) == 0) atomicAdd(&sh.X2[c / CPR], xs[r]);
  }

  f32x4_t acc[NI][TB];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    bf16x8_t bx[TB];
#pragma unroll
    for (int j = 0; j < TB; ++j)
      bx[j] = *reinterpret_cast<const bf16x8_t*>(sx + (16 * j + l16) * XST + 32 * st + 8 * g);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (bval[i]) {
#pragma unroll
        for (int j = 0; j < TB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A[i][st]), bx[j],
                                                              acc[i][j], 0, 0, 0);
      }
  }
  // max_e |w_e|^2 of the wave's rows (two-term dot products of the bf16 pairs)
  float wsq[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const uint4 q = A[i][st];
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x), __builtin_bit_cast(bf16x2_t, q.x), ss, false);
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y), __builtin_bit_cast(bf16x2_t, q.y), ss, false);
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z), __builtin_bit_cast(bf16x2_t, q.z), ss, false);
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w), __builtin_bit_cast(bf16x2_t, q.w), ss, false);
    }
    wsq[i] = ss;
  }
  publish_wmax(wsq, sh.Wmax);

  if (k <= 2) {
    // lane's best three (logit, expert) keys per token block, merged over the
    // four lanes of each token, published per wave
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      uint64_t t3[3] = {0, 0, 0};
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 16 * (wave + RW_WAVES * i) + 4 * g + r;
          if (bval[i] && e < N) top3_insert(t3, rkey(acc[i][j][r], e));
        }
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const uint64_t p0 = shfl_xor_u64(t3[0], o), p1 = shfl_xor_u64(t3[1], o), p2 = shfl_xor_u64(t3[2], o);
        top3_insert(t3, p0);
        top3_insert(t3, p1);
        top3_insert(t3, p2);
      }
      if (g == 0) {
        sTop[16 * j + l16][wave][0] = t3[0];
        sTop[16 * j + l16][wave][1] = t3[1];
        sTop[16 * j + l16][wave][2] = t3[2];
      }
    }
  }
  __syncthreads();  // token tile dead; wave lists and Wmax published
  // logits -> LDS (fp64 re-ranking of near-tied tokens reads them)
#pragma unroll
  for (int i = 0; i < NI; ++i)
    if (bval[i]) {
#pragma unroll
      for (int j = 0; j < TB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sL[(16 * j + l16) * LS + 16 * (wave + RW_WAVES * i) + 4 * g + r] = acc[i][j][r];
    }

  if (k <= 2) {
    const int kk = min(k + 1, N);
    if (tid < BT) {
      uint64_t t3[3] = {0, 0, 0};
#pragma unroll
      for (int w = 0; w < RW_WAVES; ++w)
        if (w < NB) {
          top3_insert(t3, sTop[tid][w][0]);
          top3_insert(t3, sTop[tid][w][1]);
          top3_insert(t3, sTop[tid][w][2]);
        }
      float tv[3];
#pragma unroll
      for (int q = 0; q < 3; ++q) tv[q] = rkey_val(t3[q]);
      const float tau = 2.02f * route_gamma(D / 32 + 32) * sqrtf(sh.X2[tid]) * route_wmax(sh);
      const int ngap = min(k, N - 1);
      bool f = false;
#pragma unroll
      for (int q = 0; q < 2; ++q) f |= (q < ngap) & (q + 1 < kk) & (tv[q] - tv[q + 1] < tau);
      sh.Max[tid] = tv[0];
      sh.Thr[tid] = tv[k - 1] - tau;
      sh.Idx[tid][0] = rkey_idx(t3[0]);
      sh.Idx[tid][1] = rkey_idx(t3[1]);
      sh.Gate[tid][0] = tv[0];
      sh.Gate[tid][1] = tv[1];
      sTflag[tid] = f;
    }
    __syncthreads();
    // softmax denominators: per lane over its experts, then the token's lanes and waves
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const float mx = sh.Max[16 * j + l16];
      float se = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 16 * (wave + RW_WAVES * i) + 4 * g + r;
          se += (bval[i] && e < N) ? __expf(acc[i][j][r] - mx) : 0.f;
        }
      se += __shfl_xor(se, 16, 64);
      se += __shfl_xor(se, 32, 64);
      if (g == 0) sPart[16 * j + l16][wave] = se;
    }
    __syncthreads();
    if (tid < BT) {
      float se = 0.f;
#pragma unroll
      for (int w = 0; w < RW_WAVES; ++w) se += sPart[tid][w];
      const float mx = sh.Max[tid];
      float g0 = __expf(sh.Gate[tid][0] - mx) / se;
      float g1 = k > 1 ? __expf(sh.Gate[tid][1] - mx) / se : 0.f;
      if (a.renorm) {
        const float gs = g0 + g1;
        g0 /= gs;
        g1 /= gs;
      }
      sh.Gate[tid][0] = g0;
      sh.Gate[tid][1] = g1;
      sh.Sum[tid] = se;
      if (sTflag[tid] && t0 + tid < a.T) sh.Flag[atomicAdd(&sh.NF, 1)] = tid;
    }
    __syncthreads();
  } else {
    route_decide<BT, RW_THREADS>(a, sh, sL, LS, D / 32 + 32, t0);
  }
  route_recheck_store<ACT_BF16, BT, RW_THREADS>(a, sh, sL, LS, t0);
}

template <int BT>
static size_t route_lds_bytes(int N, size_t tiles) {
  const int NB = (N + 15) >> 4;
  const size_t logits = size_t(BT) * (NB * 16 + 4) * sizeof(float);
  return logits > tiles ? logits : tiles;
}

constexpr size_t RT_WHOLE_MAX = 72 * 1024;  // whole token tile in LDS up to this size

template <typename K>
static hipError_t route_launch(K kern, int grid, int threads, size_t lds, hipStream_t s, const RouteArgs& a) {
  const hipError_t err = allow_dynamic_lds((const void*)kern, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, s, a);
  return hipGetLastError();
}

template <int BT, int NK, int NI>
static hipError_t launch_whole(const RouteArgs& a, hipStream_t s) {
  const size_t lds = route_lds_bytes<BT>(a.N, size_t(BT) * (NK * RT_BK + 8) * sizeof(uint16_t));
  return route_launch(route_whole_kernel<BT, NK, NI>, (a.T + BT - 1) / BT, RW_THREADS, lds, s, a);
}

// the pipelined kernel with NW waves per workgroup of BT tokens
template <int BT, int NW>
static hipError_t launch_pipelined(const RouteArgs& a, int act, hipStream_t s) {
  const size_t lds = route_lds_bytes<BT>(a.N, size_t(2) * BT * RT_XLD * sizeof(uint16_t));
  const int grid = (a.T + BT - 1) / BT;
  if (act == ACT_BF16) return route_launch(route_kernel<ACT_BF16, BT, NW>, grid, 64 * NW, lds, s, a);
  return route_launch(route_kernel<ACT_F32, BT, NW>, grid, 64 * NW, lds, s, a);
}

// whole-tile kernel when the tile fits LDS and a wave's gate rows fit 128
// registers per lane (width <= 1024 with one 16-expert block per wave, <= 512 with two)
template <int BT>
static hipError_t launch_route_bt(const RouteArgs& a, int act, hipStream_t s) {
  if (act == ACT_BF16 && size_t(BT) * (a.d + 8) * sizeof(uint16_t) <= RT_WHOLE_MAX) {
    if (a.N <= 128) {
      switch (a.d / RT_BK) {
        case 1: return launch_whole<BT, 1, 1>(a, s);
        case 2: return launch_whole<BT, 2, 1>(a, s);
        case 4: return launch_whole<BT, 4, 1>(a, s);
        case 8: return launch_whole<BT, 8, 1>(a, s);
        case 16: if constexpr (BT <= 32) return launch_whole<BT, 16, 1>(a, s); break;
        default: break;
      }
    } else {
      switch (a.d / RT_BK) {
        case 1: return launch_whole<BT, 1, 2>(a, s);
        case 2: return launch_whole<BT, 2, 2>(a, s);
        case 4: return launch_whole<BT, 4, 2>(a, s);
        case 8: return launch_whole<BT, 8, 2>(a, s);
        default: break;
      }
    }
  }
  return launch_pipelined<BT, 4>(a, act, s);
}

// the largest token tile that still gives every CU a workgroup (each
// workgroup reads the whole gate matrix once): 64, 32 or 16 tokens, or 128
// (one eight-wave workgroup per CU, half the gate traffic) for bf16 tokens
// too wide for the whole-tile kernel
int route_tile_tokens(int T, int d, int act) {
  if (act == ACT_BF16 && T >= 128 * 256 && size_t(64) * (d + 8) * sizeof(uint16_t) > RT_WHOLE_MAX) return 128;
  return T >= 64 * 256 ? 64 : T >= 32 * 256 ? 32 : 16;
}

hipError_t launch_route(const RouteArgs& a, int act, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (!a.tile_slots || !a.tile_gates || !a.tile_start || a.N > 256) return hipErrorInvalidValue;
  switch (route_tile_tokens(a.T, a.d, act)) {
    case 128: return launch_pipelined<128, 8>(a, act, s);
    case 64: return launch_route_bt<64>(a, act, s);
    case 32: return launch_route_bt<32>(a, act, s);
    default: return launch_route_bt<16>(a, act, s);
  }
}

// ------------------------------------------------------------------ gate fragments
// One thread per 16-byte fragment: copies W_g's 8 values of (expert, k-step,
// lane) to fragment order (zeros for experts past N).
__global__ __launch_bounds__(256) void gate_frag_kernel(const uint16_t* __restrict__ w, uint4* __restrict__ out,
                                                        int N, int d, int units) {
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int ks = d / 32, lane = u & 63, st = (u >> 6) % ks, b = (u >> 6) / ks;
  const int e = 16 * b + (lane & 15);
  out[u] = e < N ? *reinterpret_cast<const uint4*>(w + size_t(e) * d + 32 * st + 8 * (lane >> 4))
                 : make_uint4(0, 0, 0, 0);
}

bool gate_frag_supported(int d) { return d > 0 && d % 32 == 0; }

size_t gate_frag_bytes(int N, int d) {
  return gate_frag_supported(d) ? size_t((N + 15) / 16) * 16 * size_t(d) * 2 : 0;
}

hipError_t launch_gate_frag(const void* w_gate, void* out, int N, int d, hipStream_t s) {
  if (N <= 0 || !gate_frag_supported(d)) return hipErrorInvalidValue;
  const int units = int(gate_frag_bytes(N, d) / 16);
  hipLaunchKernelGGL(gate_frag_kernel, dim3((units + 255) / 256), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(w_gate), reinterpret_cast<uint4*>(out), N, d, units);
  return hipGetLastError();
}

// ------------------------------------------------------------------ bucketing
// BK_SPLIT workgroups per expert e (so one popular expert's rows are copied
// by several CUs).  The expert's first bucket position is the number of slots
// routed to lower experts, the sum over token tiles of the position of e in
// the tile's list.  Its slots are the tiles' runs of e, concatenated in tile
// order (so slots ascend within the expert): tiles are taken BK_THREADS at a
// time, their run lengths scanned, and the runs copied by all threads; part s
// of the expert copies its positions [s c, (s + 1) c), c = ceil(count / BK_SPLIT).
// With `rec` set the expert's tile records are written too (headers by part 0).
constexpr int BK_THREADS = 256;
constexpr int BK_UNROLL = 4;   // copies in flight per thread
constexpr int BK_SPLIT = 4;    // workgroups per expert
static_assert(BK_THREADS == 256, "the run search takes 8 halvings");

__global__ __launch_bounds__(BK_THREADS) void bucket_kernel(BucketArgs a) {
  __shared__ int s_w[2][BK_THREADS / 64];
  __shared__ int s_pre[BK_THREADS + 1];  // run starts of the round's tiles in its output
  __shared__ int s_src[BK_THREADS];      // run starts in the tile lists
  if (a.zero)
    for (size_t i = size_t(blockIdx.x) * BK_THREADS + threadIdx.x; i < a.zero16; i += size_t(gridDim.x) * BK_THREADS)
      a.zero[i] = make_uint4(0u, 0u, 0u, 0u);
  const int e = blockIdx.x / BK_SPLIT, part = blockIdx.x % BK_SPLIT, N = a.N, G = a.G, C = a.C;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // slots of lower experts and of e
  int below = 0, cnt = 0;
  for (int b = tid; b < G; b += BK_THREADS) {
    const int st = a.tile_start[size_t(b) * N + e];
    const int en = e + 1 < N ? a.tile_start[size_t(b) * N + e + 1] : min(C, a.R - b * C);
    below += st;
    cnt += en - st;
  }
  below = wave_sum(below);
  cnt = wave_sum(cnt);
  if (lane == 0) {
    s_w[0][wave] = below;
    s_w[1][wave] = cnt;
  }
  __syncthreads();
  below = cnt = 0;
#pragma unroll
  for (int w = 0; w < BK_THREADS / 64; ++w) {
    below += s_w[0][w];
    cnt += s_w[1][w];
  }
  if (tid == 0 && part == 0) {
    a.offsets[e] = below;
    if (e == N - 1) a.offsets[N] = a.R;
  }
  const int rrows = a.rec_rows;
  const int rbase = a.rec ? below / rrows + e : 0;  // first tile record of e
  const int chunk = (cnt + BK_SPLIT - 1) / BK_SPLIT;
  const int q_lo = part * chunk, q_hi = min(cnt, q_lo + chunk);  // this part's positions in e's list
  if (a.rec && part == 0) {
    const int nt = (cnt + rrows - 1) / rrows;
    const int next = e + 1 < N ? (below + cnt) / rrows + e + 1 : a.n_rec;
    for (int j = tid; j < next - rbase; j += BK_THREADS) {
      TileRec* r = a.rec + rbase + j;
      r->e = j < nt ? e : -1;
      r->nr = j < nt ? min(rrows, cnt - rrows * j) : 0;
    }
  }

  int base = 0;  // position in e's list
  for (int b0 = 0; b0 < G && base < q_hi; b0 += BK_THREADS) {
    const int b = b0 + tid;
    int st = 0, h = 0;
    if (b < G) {
      st = a.tile_start[size_t(b) * N + e];
      const int en = e + 1 < N ? a.tile_start[size_t(b) * N + e + 1] : min(C, a.R - b * C);
      h = en - st;
    }
    int x = h;  // inclusive scan of the run lengths over the round's tiles
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    __syncthreads();  // s_w, s_pre, s_src of the previous round are dead
    if (lane == 63) s_w[0][wave] = x;
    __syncthreads();
    int pre = 0, total = 0;
#pragma unroll
    for (int w = 0; w < BK_THREADS / 64; ++w) {
      pre += w < wave ? s_w[0][w] : 0;
      total += s_w[0][w];
    }
    s_pre[tid + 1] = pre + x;
    if (tid == 0) s_pre[0] = 0;
    s_src[tid] = b * C + st;
    __syncthreads();
    // output position f of the round: the tile i with s_pre[i] <= f < s_pre[i + 1];
    // this part copies f in [f_lo, f_hi)
    const int f_lo = max(0, q_lo - base), f_hi = min(total, q_hi - base);
    for (int f0 = f_lo; f0 < f_hi; f0 += BK_THREADS * BK_UNROLL) {
      int v[BK_UNROLL];
      float g[BK_UNROLL];
#pragma unroll
      for (int u = 0; u < BK_UNROLL; ++u) {
        const int f = f0 + u * BK_THREADS + tid;
        if (f < f_hi) {
          int lo = 0, hi = BK_THREADS;
#pragma unroll
          for (int it = 0; it < 8; ++it) {
            const int mid = (lo + hi) >> 1;
            if (s_pre[mid] <= f) lo = mid; else hi = mid;
          }
          const int src = s_src[lo] + f - s_pre[lo];
          v[u] = a.tile_slots[src];
          if (a.rec) g[u] = a.tile_gates[src];
        }
      }
#pragma unroll
      for (int u = 0; u < BK_UNROLL; ++u) {
        const int f = f0 + u * BK_THREADS + tid;
        if (f < f_hi) {
          const int q = base + f;
          a.perm[below + q] = v[u];
          if (a.rec) {
            TileRec* r = a.rec + rbase + q / rrows;
            r->slot[q % rrows] = v[u];
            r->gate[q % rrows] = g[u];
          }
        }
      }
    }
    base += total;
  }
}

hipError_t launch_bucket(const BucketArgs& a, hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  if (a.G != (a.R / max(a.C, 1) + (a.R % max(a.C, 1) != 0)) || a.N > 256) return hipErrorInvalidValue;
  if (a.rec && (!a.tile_gates || (a.rec_rows != 32 && a.rec_rows != 48 && a.rec_rows != TILE_ROWS_MAX) ||
                a.n_rec != (a.R + a.rec_rows - 1) / a.rec_rows + a.N))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(bucket_kernel, dim3(a.N * BK_SPLIT), dim3(BK_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace bmoe
