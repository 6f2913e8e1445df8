// Top-k softmax router and per-expert bucketing (ButterflyMoE,
// gist.science/nl/paper/2601.13563, §2 "Drie Fasen van de Methode": a standard
// top-k gating network selects the active experts).
//
// Logits l = W_g x are computed in fp32 (bf16 activations: MFMA
// 16x16x32 bf16 -> fp32; fp32 activations: one FMA chain per logit).  Each
// token's top-k order is then decided in fp32 unless one of its decisive gaps
// (between consecutive chosen logits, and between the k-th and the (k+1)-th)
// is within twice the worst-case fp32 error of a logit,
//     gamma_D * |x| * max_e |w_e|,  gamma_D = D u / (1 - D u),
// where D bounds the rounding depth of the sum (K/32 MFMA accumulations plus
// 32 adds inside one MFMA; or d for an FMA chain) and u = 2^-22 (twice the fp32
// unit roundoff, as the MFMA's internal rounding mode is not documented).
// Such tokens are recomputed in fp64 (bf16 x bf16 products are exact), so the
// chosen experts equal those of exact arithmetic except for gaps below fp64
// rounding.
#include "common.hpp"
#include <float.h>

namespace bmoe {

constexpr int RT_THREADS = 256;
constexpr int RT_TOK = 32;     // tokens per workgroup
constexpr int RT_KMAX = 8;     // largest supported top_k

// ------------------------------------------------------------------ prep
// Squared row norms of W_g (for the error bound) and zeroed expert counters.
__global__ __launch_bounds__(64) void prep_kernel(const void* w_gate, int act, int d,
                                                  float* wnorm2, int32_t* counts) {
  const int e = blockIdx.x;
  float s = 0.f;
  for (int i = threadIdx.x; i < d; i += 64) {
    const float v = act == ACT_BF16 ? load1<ACT_BF16>(w_gate, size_t(e) * d + i)
                                    : load1<ACT_F32>(w_gate, size_t(e) * d + i);
    s = fmaf(v, v, s);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (threadIdx.x == 0) {
    wnorm2[e] = s;
    counts[e] = 0;
  }
}

hipError_t launch_prep(const void* w_gate, int act, int32_t N, int32_t d, float* wnorm2,
                       int32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL(prep_kernel, dim3(N), dim3(64), 0, s, w_gate, act, d, wnorm2, counts);
  return hipGetLastError();
}

// ------------------------------------------------------------------ wave top-k
// Better = larger value, or equal value and lower index.
template <typename T>
__device__ __forceinline__ bool better(T v, int i, T bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Top-kk of the N values a wave holds (lane owns indices lane + 64 j).
// Results are uniform over the wave.
template <typename T>
__device__ __forceinline__ void wave_topk(T v[4], int N, int kk, T* tv, int* ti) {
  const int lane = threadIdx.x & 63;
  for (int j = 0; j < kk; ++j) {
    T bv = v[0];
    int bi = lane;
#pragma unroll
    for (int u = 1; u < 4; ++u) {
      const int i = lane + 64 * u;
      if (i < N && better(v[u], i, bv, bi)) { bv = v[u]; bi = i; }
    }
    if (lane >= N) bi = 0x7fffffff;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const T ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    tv[j] = bv;
    ti[j] = bi;
    // remove the winner
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (lane + 64 * u == bi) v[u] = -(T)INFINITY;
  }
}

// Decide one token from its N logits held in LDS (fp32 or fp64).  Writes the
// chosen experts and gates to the per-token slots; returns true (uniform) if a
// decisive gap is below `tau`.
template <typename T>
__device__ bool decide_token(const T* logits, int N, int k, int renorm, T tau, int* out_idx,
                             float* out_gate) {
  const int lane = threadIdx.x & 63;
  T v[4], orig[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = lane + 64 * u;
    v[u] = i < N ? logits[i] : -(T)INFINITY;
    orig[u] = v[u];
  }
  const int kk = min(k + 1, N);
  T tv[RT_KMAX + 1];
  int ti[RT_KMAX + 1];
  wave_topk<T>(v, N, kk, tv, ti);
  const T mx = tv[0];
  T se = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = lane + 64 * u;
    if (i < N) se += (sizeof(T) == 8) ? (T)exp((double)(orig[u] - mx)) : (T)expf((float)(orig[u] - mx));
  }
  se = wave_sum(se);
  bool flag = false;
  const int ngap = min(k, N - 1);
  for (int j = 0; j < ngap; ++j)
    if (tv[j] - tv[j + 1] < tau) flag = true;
  if (lane == 0) {
    T g[RT_KMAX];
    T gs = 0;
    for (int j = 0; j < k; ++j) {
      g[j] = ((sizeof(T) == 8) ? (T)exp((double)(tv[j] - mx)) : (T)expf((float)(tv[j] - mx))) / se;
      gs += g[j];
    }
    for (int j = 0; j < k; ++j) {
      out_idx[j] = ti[j];
      out_gate[j] = (float)(renorm ? g[j] / gs : g[j]);
    }
  }
  return flag;
}

// ------------------------------------------------------------------ router
template <int ACT>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(RouteArgs a) {
  // LDS: logits [RT_TOK][257] fp32, gate-weight chunk [256][40] bf16 (bf16 path)
  __shared__ float sL[RT_TOK][257];
  __shared__ __attribute__((aligned(16))) uint16_t sG[256 * 40];
  __shared__ float sX2[RT_TOK];
  __shared__ double sL64[256];
  __shared__ int sIdx[RT_TOK][RT_KMAX];
  __shared__ float sGate[RT_TOK][RT_KMAX];
  __shared__ int sFlag[RT_TOK];
  __shared__ int sNF;
  __shared__ float sWmax;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT_TOK;
  const int N = a.N, d = a.d, k = a.k;
  if (tid == 0) sNF = 0;

  // max_e |w_e|^2 (wave 0)
  if (wave == 0) {
    float m = 0.f;
    for (int i = lane; i < N; i += 64) m = fmaxf(m, a.wnorm2[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) sWmax = m;
  }

  int depth;
  if constexpr (ACT == ACT_BF16) {
    // wave (tg, eg): tokens 16*tg .. +15, expert blocks eg, eg+2, ...
    const int tg = wave & 1, eg = wave >> 1;
    const int NB = (N + 15) >> 4;
    f32x4_t acc[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float x2 = 0.f;
    const int tok = t0 + 16 * tg + (lane & 15);
    const bool tok_ok = tok < a.T;
    const uint16_t* xg = reinterpret_cast<const uint16_t*>(a.x);
    const uint16_t* wg = reinterpret_cast<const uint16_t*>(a.w_gate);
    const int Npad = NB * 16;
    for (int k0 = 0; k0 < d; k0 += 32) {
      // gate-weight chunk [Npad][32] -> LDS (row stride 40 bf16)
      for (int c = tid; c < Npad * 4; c += RT_THREADS) {
        const int row = c >> 2, ch = c & 3;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < N) v = *reinterpret_cast<const uint4*>(wg + size_t(row) * d + k0 + 8 * ch);
        *reinterpret_cast<uint4*>(&sG[row * 40 + 8 * ch]) = v;
      }
      uint4 xv = make_uint4(0, 0, 0, 0);
      if (tok_ok) xv = *reinterpret_cast<const uint4*>(xg + size_t(tok) * d + k0 + 8 * (lane >> 4));
      {
        const float f[8] = {bf16lo(xv.x), bf16hi(xv.x), bf16lo(xv.y), bf16hi(xv.y),
                            bf16lo(xv.z), bf16hi(xv.z), bf16lo(xv.w), bf16hi(xv.w)};
#pragma unroll
        for (int j = 0; j < 8; ++j) x2 = fmaf(f[j], f[j], x2);
      }
      const bf16x8_t xf = __builtin_bit_cast(bf16x8_t, xv);
      __syncthreads();
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        const int b = eg + 2 * bb;
        if (b < NB) {
          const bf16x8_t gf = *reinterpret_cast<const bf16x8_t*>(&sG[(16 * b + (lane & 15)) * 40 + 8 * (lane >> 4)]);
          acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gf, xf, acc[bb], 0, 0, 0);
        }
      }
      __syncthreads();
    }
    // D[expert][token]: lane holds experts 16b + 4(lane>>4) + r, token lane & 15
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const int b = eg + 2 * bb;
      if (b < NB) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 16 * b + 4 * (lane >> 4) + r;
          if (e < N) sL[16 * tg + (lane & 15)][e] = acc[bb][r];
        }
      }
    }
    x2 += __shfl_xor(x2, 16, 64);
    x2 += __shfl_xor(x2, 32, 64);
    if (eg == 0 && lane < 16) sX2[16 * tg + lane] = x2;
    depth = d / 32 + 32;
  } else {
    // fp32: one sequential FMA chain per (token, expert)
    const float* xf = reinterpret_cast<const float*>(a.x);
    const float* wf = reinterpret_cast<const float*>(a.w_gate);
    for (int p = tid; p < RT_TOK * N; p += RT_THREADS) {
      const int tl = p / N, e = p - tl * N;
      const int tok = t0 + tl;
      float s = 0.f;
      if (tok < a.T) {
        const float* xr = xf + size_t(tok) * d;
        const float* wr = wf + size_t(e) * d;
        for (int i = 0; i < d; ++i) s = fmaf(xr[i], wr[i], s);
      }
      sL[tl][e] = s;
    }
    for (int tl = tid; tl < RT_TOK; tl += RT_THREADS) {
      const int tok = t0 + tl;
      float s = 0.f;
      if (tok < a.T) {
        const float* xr = xf + size_t(tok) * d;
        for (int i = 0; i < d; ++i) s = fmaf(xr[i], xr[i], s);
      }
      sX2[tl] = s;
    }
    depth = d;
  }
  __syncthreads();

  // ---- fp32 decision, one wave per token
  const float u = 2.384185791015625e-07f;  // 2^-22
  const float Du = depth * u;
  const float gamma = Du / (1.f - Du);
  const float wmax = sqrtf(sWmax);
  for (int tl = wave; tl < RT_TOK; tl += RT_THREADS / 64) {
    if (t0 + tl >= a.T) break;
    const float tau = 2.02f * gamma * sqrtf(sX2[tl]) * wmax;
    const bool flag = decide_token<float>(sL[tl], N, k, a.renorm, tau, sIdx[tl], sGate[tl]);
    if (flag && lane == 0) sFlag[atomicAdd(&sNF, 1)] = tl;
  }
  __syncthreads();

  // ---- fp64 recheck of flagged tokens (whole workgroup per token)
  const int nf = sNF;
  for (int f = 0; f < nf; ++f) {
    const int tl = sFlag[f];
    const size_t xo = size_t(t0 + tl) * d;
    for (int e = wave; e < N; e += RT_THREADS / 64) {
      double s = 0.0;
      for (int i = lane; i < d; i += 64) {
        const double xv = ACT == ACT_BF16 ? (double)load1<ACT_BF16>(a.x, xo + i) : (double)load1<ACT_F32>(a.x, xo + i);
        const double wv = ACT == ACT_BF16 ? (double)load1<ACT_BF16>(a.w_gate, size_t(e) * d + i)
                                          : (double)load1<ACT_F32>(a.w_gate, size_t(e) * d + i);
        s = fma(xv, wv, s);
      }
      s = wave_sum(s);
      if (lane == 0) sL64[e] = s;
    }
    __syncthreads();
    if (wave == 0) decide_token<double>(sL64, N, k, a.renorm, 0.0, sIdx[tl], sGate[tl]);
    __syncthreads();
  }

  // ---- outputs and expert counts
  for (int p = tid; p < RT_TOK * k; p += RT_THREADS) {
    const int tl = p / k, j = p - tl * k;
    const int tok = t0 + tl;
    if (tok < a.T) {
      const int e = sIdx[tl][j];
      a.topk_idx[size_t(tok) * k + j] = e;
      a.topk_gate[size_t(tok) * k + j] = sGate[tl][j];
      atomicAdd(&a.counts[e], 1);
    }
  }
}

hipError_t launch_route(const RouteArgs& a, int act, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int grid = (a.T + RT_TOK - 1) / RT_TOK;
  if (act == ACT_BF16)
    hipLaunchKernelGGL(route_kernel<ACT_BF16>, dim3(grid), dim3(RT_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(route_kernel<ACT_F32>, dim3(grid), dim3(RT_THREADS), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ bucketing
// One workgroup per expert: its first bucket position is the sum of the
// counts of the lower experts; it then walks all routed slots in order and
// appends the ones routed to it, so within an expert slots ascend.
constexpr int BK_THREADS = 1024;

__global__ __launch_bounds__(BK_THREADS) void bucket_kernel(BucketArgs a) {
  __shared__ int s_w[BK_THREADS / 64];
  __shared__ int s_off;
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int part = (tid < e) ? a.counts[tid] : 0;  // e < 256 <= BK_THREADS
  part = wave_sum(part);
  if (lane == 0) s_w[wave] = part;
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
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int running = 0;
  for (int base = 0; base < a.R; base += 4 * BK_THREADS) {
    const int f0 = base + 4 * tid;
    int v[4];
    if (f0 + 3 < a.R) {
      const int4 q = *reinterpret_cast<const int4*>(a.topk_idx + f0);
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (f0 + j < a.R) ? a.topk_idx[f0 + j] : -1;
    }
    int c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) c += (v[j] == e);
    const uint64_t b0 = __ballot(c & 1), b1 = __ballot(c & 2), b2 = __ballot(c & 4);
    const int lpre = __popcll(b0 & lt) + 2 * __popcll(b1 & lt) + 4 * __popcll(b2 & lt);
    const int wtot = __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
    __syncthreads();
    if (lane == 0) s_w[wave] = wtot;
    __syncthreads();
    int wpre = 0, tot = 0;
    for (int w = 0; w < BK_THREADS / 64; ++w) {
      const int x = s_w[w];
      wpre += (w < wave) ? x : 0;
      tot += x;
    }
    int q = off + running + wpre + lpre;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (v[j] == e) a.perm[q++] = f0 + j;
    running += tot;
  }
}

hipError_t launch_bucket(const BucketArgs& a, hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  hipLaunchKernelGGL(bucket_kernel, dim3(a.N), dim3(BK_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace bmoe
