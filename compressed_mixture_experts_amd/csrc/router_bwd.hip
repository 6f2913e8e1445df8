// Backward of the gating network with the chosen experts held (ButterflyMoE,
// gist.science/nl/paper/2601.13563, §2 "Gated Routing": a standard top-k
// gating network).  Logits l = W_g x_t, p = softmax(l) over all N experts,
// gate_j = p_{e_j} (or renormalised over the k chosen).  Given the gates'
// gradients:
//   without renormalisation  dl_n = p_n (a_n - s), a_n = sum_j dgate_j [n = e_j],
//                            s = sum_j dgate_j p_{e_j}
//   with renormalisation     dl_{e_j} = g_j (dgate_j - sum_i dgate_i g_i), else 0
// then dx_t = W_g^T dl_t and dW_g = sum_t dl_t x_t^T.
//
// Three passes, fp32 arithmetic, every output written once (no atomics):
//   router_dl_kernel   16 tokens per workgroup (32 or 64 on the matrix cores
//                      when the tokens are many), a thread per expert: the
//                      logits again (bf16 rows on the matrix cores, the token
//                      tile in LDS 512 columns at a time; fp32 rows on the
//                      VALU with the tile read by broadcast), softmax over the
//                      workgroup, dl [T][N] to the workspace;
//   router_dx_kernel   16 tokens per workgroup (64 when the tokens are many,
//                      512 columns each), their dl in LDS, a thread per
//                      column of x, four experts' gate rows loaded ahead;
//                      bf16 rows of width a multiple of 256 take
//                      router_dx_mfma_kernel instead;
//   router_dwg_kernel  16 experts x 256 columns per workgroup (dl of 256
//                      tokens at a time in LDS), the tokens split in ranges of
//                      at least 256 for about 2048 workgroups; the ranges'
//                      partial sums added in order by router_red_kernel.
#include "common.hpp"

namespace bmoe {

constexpr int RB_BT = 16;   // tokens per workgroup (dl, dx)
constexpr int RB_NB = 16;   // experts per workgroup (dW_g)

struct RouterBwdArgs {
  const void* x;         // [T][d]
  const void* wg;        // [N][d]
  const int32_t* idx;    // [T][k]
  const float* dgate;    // [T][k]
  float* dl;             // [T][N] (workspace)
  float* dx;             // [T][d]
  float* dwg;            // [N][d]
  float* part;           // [S][N][d] (workspace) when S > 1
  int32_t T, d, N, k, renorm, S, tchunk;
};

constexpr int RB_XC = 512;  // columns of the token tile staged in LDS at a time

// TB blocks of 16 tokens per workgroup; TB > 1 only for bf16 rows of width a
// multiple of 32 (the matrix-core path), where each gate-row fragment read
// from memory then serves TB token blocks.
template <int A, int TB>
__global__ __launch_bounds__(256) void router_dl_kernel(RouterBwdArgs a) {
  constexpr int XC = TB == 1 ? RB_XC : 256;  // bf16 columns of the token tile staged at a time
  constexpr int XS = XC + 8;
  constexpr int SXF = TB == 1 ? RB_BT * RB_XC : TB * RB_BT * XS / 2;  // floats of the staging area
  __shared__ float sP[RB_BT][256];      // probabilities
  __shared__ float sRed[RB_BT][4];
  __shared__ float sMax[RB_BT], sSum[RB_BT];
  __shared__ __attribute__((aligned(16))) float sXf[SXF];  // token tile, one column chunk
  __shared__ int sId[TB * RB_BT][8];     // the tile's chosen experts (top_k <= 8) ...
  __shared__ float sDg[TB * RB_BT][8];   // ... and their gate gradients
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tw0 = blockIdx.x * RB_BT * TB, n = tid;
  for (int q = tid; q < TB * RB_BT * a.k; q += 256) {  // read before the first barrier below
    const int t = q / a.k, j = q % a.k;
    if (tw0 + t < a.T) {
      sId[t][j] = min(max(a.idx[size_t(tw0 + t) * a.k + j], 0), a.N - 1);
      sDg[t][j] = a.dgate[size_t(tw0 + t) * a.k + j];
    }
  }
  const bool live = n < a.N;
  float acc[RB_BT];
#pragma unroll
  for (int t = 0; t < RB_BT; ++t) acc[t] = 0.f;
  f32x4_t am[4][TB];
  const int l16 = lane & 15, g = lane >> 4, NB = (a.N + 15) >> 4;
  if (A == ACT_BF16 && a.d % 32 == 0) {  // uniform
    // bf16 rows: the logits on the matrix cores (exact products, fp32 sums).
    // The tile's columns in LDS as bf16 rows; wave w takes the 16-expert
    // blocks w, w+4, ... with its gate-row fragments straight from memory;
    // then the logits go through sP to the thread of each expert.
    uint16_t* sXb = reinterpret_cast<uint16_t*>(sXf);  // [TB RB_BT][XS] bf16
    const uint16_t* xg = static_cast<const uint16_t*>(a.x);
    const uint16_t* wgp = static_cast<const uint16_t*>(a.wg);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < TB; ++b) am[i][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < a.d; c0 += XC) {
      const int cw = min(XC, a.d - c0);
      for (int q = tid; q < TB * RB_BT * (cw / 8); q += 256) {
        const int t = q / (cw / 8), i = (q % (cw / 8)) * 8;
        const uint4 v = tw0 + t < a.T ? *reinterpret_cast<const uint4*>(xg + size_t(tw0 + t) * a.d + c0 + i)
                                      : make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(sXb + t * XS + i) = v;
      }
      __syncthreads();
      for (int st = 0; st < cw / 32; ++st) {
        bf16x8_t bx[TB];
#pragma unroll
        for (int b = 0; b < TB; ++b)
          bx[b] = *reinterpret_cast<const bf16x8_t*>(sXb + (RB_BT * b + l16) * XS + 32 * st + 8 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = wave + 4 * i, e = 16 * b + l16;
          if (b < NB) {  // uniform per wave
            const uint4 wv = e < a.N ? *reinterpret_cast<const uint4*>(wgp + size_t(e) * a.d + c0 + 32 * st + 8 * g)
                                     : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
              am[i][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv), bx[tb], am[i][tb], 0, 0, 0);
          }
        }
      }
      __syncthreads();  // the chunk is replaced next
    }
  } else if constexpr (TB == 1) {
    float (*sX)[RB_XC] = reinterpret_cast<float (*)[RB_XC]>(sXf);
    for (int c0 = 0; c0 < a.d; c0 += RB_XC) {
      const int cw = min(RB_XC, a.d - c0);
      // the tile's columns c0 .. c0+cw-1 (8 per thread and step, rows past T zero)
      for (int q = tid; q < RB_BT * cw / 8; q += 256) {
        const int t = q / (cw / 8), i = (q % (cw / 8)) * 8;
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (tw0 + t < a.T) load8<A>(a.x, size_t(tw0 + t) * a.d + c0 + i, v);
        *reinterpret_cast<float4*>(&sX[t][i]) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(&sX[t][i + 4]) = make_float4(v[4], v[5], v[6], v[7]);
      }
      __syncthreads();
      for (int i = 0; i < cw; i += 8) {
        float w[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (live) load8<A>(a.wg, size_t(n) * a.d + c0 + i, w);
#pragma unroll
        for (int t = 0; t < RB_BT; ++t) {
          const float4 x0 = *reinterpret_cast<const float4*>(&sX[t][i]);
          const float4 x1 = *reinterpret_cast<const float4*>(&sX[t][i + 4]);
          acc[t] = fmaf(w[0], x0.x, acc[t]);
          acc[t] = fmaf(w[1], x0.y, acc[t]);
          acc[t] = fmaf(w[2], x0.z, acc[t]);
          acc[t] = fmaf(w[3], x0.w, acc[t]);
          acc[t] = fmaf(w[4], x1.x, acc[t]);
          acc[t] = fmaf(w[5], x1.y, acc[t]);
          acc[t] = fmaf(w[6], x1.z, acc[t]);
          acc[t] = fmaf(w[7], x1.w, acc[t]);
        }
      }
      __syncthreads();  // the chunk is replaced next
    }
  }
  const bool mf = A == ACT_BF16 && a.d % 32 == 0;
#pragma unroll 1
  for (int tb = 0; tb < TB; ++tb) {
    const int t0 = tw0 + RB_BT * tb;
    if (mf) {
      // am[i][tb][v] = logit of expert 16 (w + 4 i) + 4 g + v for token t0 + l16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = wave + 4 * i;
        if (b < NB) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int e = 16 * b + 4 * g + v;
            f32x4_t m = am[i][0];
#pragma unroll
            for (int q = 1; q < TB; ++q)
              if (q == tb) m = am[i][q];
            if (e < a.N) sP[l16][e] = m[v];
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < RB_BT; ++t) acc[t] = live ? sP[t][n] : 0.f;
      __syncthreads();  // sP is rewritten with the probabilities below
    }
    // softmax over the experts, per token: max, then sum of exp
#pragma unroll
    for (int t = 0; t < RB_BT; ++t) {
      float m = live ? acc[t] : -INFINITY;
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      if (lane == 0) sRed[t][wave] = m;
    }
    __syncthreads();
    if (tid < RB_BT) sMax[tid] = fmaxf(fmaxf(sRed[tid][0], sRed[tid][1]), fmaxf(sRed[tid][2], sRed[tid][3]));
    __syncthreads();
    float ev[RB_BT];
#pragma unroll
    for (int t = 0; t < RB_BT; ++t) {
      ev[t] = live ? __expf(acc[t] - sMax[t]) : 0.f;
      float s = ev[t];
      for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
      if (lane == 0) sRed[t][wave] = s;
    }
    __syncthreads();
    if (tid < RB_BT) sSum[tid] = (sRed[tid][0] + sRed[tid][1]) + (sRed[tid][2] + sRed[tid][3]);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < RB_BT; ++t) sP[t][n] = live ? ev[t] / sSum[t] : 0.f;
    __syncthreads();
    // dl of this thread's expert for each token of the tile
#pragma unroll
    for (int t = 0; t < RB_BT; ++t) {
      const int tt = t0 + t;
      if (tt >= a.T || !live) continue;
      const int* id = sId[RB_BT * tb + t];
      const float* dg = sDg[RB_BT * tb + t];
      float v = 0.f;
      if (a.renorm) {
        float ps = 0.f, inner = 0.f, mine = 0.f;
        bool chosen = false;
        for (int j = 0; j < a.k; ++j) ps += sP[t][id[j]];
        for (int j = 0; j < a.k; ++j) {
          const int e = id[j];
          const float g = sP[t][e] / ps;
          inner = fmaf(dg[j], g, inner);
          if (e == n) {
            chosen = true;
            mine += dg[j];
          }
        }
        if (chosen) {
          const float g = sP[t][n] / ps;
          v = g * (mine - inner);
        }
      } else {
        float s = 0.f, an = 0.f;
        for (int j = 0; j < a.k; ++j) {
          const int e = id[j];
          s = fmaf(dg[j], sP[t][e], s);
          if (e == n) an += dg[j];
        }
        v = sP[t][n] * (an - s);
      }
      a.dl[size_t(tt) * a.N + n] = v;
    }
    if (TB > 1) __syncthreads();  // sP is rewritten for the next token block
  }
}

// dx[t][i] = sum_n dl[t][n] W_g[n][i] for BT tokens and 256 CW columns per
// workgroup (a thread per column, CW columns 256 apart); the tile's dl in LDS
// as [n][t] so that a thread reads four tokens' values in one 16-byte
// broadcast; four experts' gate rows loaded ahead.
template <int A, int BT, int CW>
__global__ __launch_bounds__(256) void router_dx_kernel(RouterBwdArgs a) {
  __shared__ __attribute__((aligned(16))) float sLT[256][BT];
  const int tid = threadIdx.x;
  const int ncb = (a.d + 256 * CW - 1) / (256 * CW);
  const int t0 = (blockIdx.x / ncb) * BT, c0 = (blockIdx.x % ncb) * 256 * CW;
  for (int q = tid; q < BT * a.N; q += 256) {
    const int t = q / a.N, n = q % a.N;
    sLT[n][t] = t0 + t < a.T ? a.dl[size_t(t0 + t) * a.N + n] : 0.f;
  }
  __syncthreads();
  float acc[BT][CW];
#pragma unroll
  for (int t = 0; t < BT; ++t)
#pragma unroll
    for (int c = 0; c < CW; ++c) acc[t][c] = 0.f;
  for (int n0 = 0; n0 < a.N; n0 += 4) {
    float w[4][CW];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        const int i = c0 + tid + 256 * c, n = n0 + u;
        w[u][c] = (i < a.d && n < a.N) ? load1<A>(a.wg, size_t(n) * a.d + i) : 0.f;
      }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = n0 + u < a.N ? n0 + u : a.N - 1;  // w is zero past N
#pragma unroll
      for (int t = 0; t < BT; t += 4) {
        const float4 l = *reinterpret_cast<const float4*>(&sLT[n][t]);
#pragma unroll
        for (int c = 0; c < CW; ++c) {
          acc[t][c] = fmaf(l.x, w[u][c], acc[t][c]);
          acc[t + 1][c] = fmaf(l.y, w[u][c], acc[t + 1][c]);
          acc[t + 2][c] = fmaf(l.z, w[u][c], acc[t + 2][c]);
          acc[t + 3][c] = fmaf(l.w, w[u][c], acc[t + 3][c]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < BT; ++t)
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int i = c0 + tid + 256 * c;
      if (t0 + t < a.T && i < a.d) a.dx[size_t(t0 + t) * a.d + i] = acc[t][c];
    }
}

// dx on the matrix cores (bf16 gate matrix, width a multiple of 256): a
// workgroup takes 64 tokens x 256 columns, wave w the columns 64 w .. 64 w + 63
// of all 64 tokens.  K runs over the experts 32 at a time: the gate matrix's
// 32 x 256 tile is loaded as 8 x 8 blocks, transposed in registers and
// stored with the experts innermost (so a fragment is one 16-byte LDS read);
// dl comes from the workspace as fp32, is split into two bf16 terms hi + lo
// (|dl - hi - lo| <= 2^-18 |dl|) once per workgroup and staged in LDS, and
// each term is multiplied exactly.
constexpr int RX_RS = 40;  // LDS row stride (bf16) of the transposed tile: 32 experts + 8

__device__ __forceinline__ void rx_split(const float (&v)[8], bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)v[j];
    hi[j] = h;
    lo[j] = (__bf16)(v[j] - (float)h);
  }
}

__global__ __launch_bounds__(256) void router_dx_mfma_kernel(RouterBwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sW[256 * RX_RS];  // [column][expert]
  __shared__ __attribute__((aligned(16))) uint16_t sLh[64 * RX_RS];  // [token][expert], dl hi
  __shared__ __attribute__((aligned(16))) uint16_t sLl[64 * RX_RS];  // [token][expert], dl lo
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int ncb = a.d / 256;
  const int t0 = (blockIdx.x / ncb) * 64, c0 = (blockIdx.x % ncb) * 256;
  const uint16_t* wg = static_cast<const uint16_t*>(a.wg);
  f32x4_t acc[4][4];  // [column block][token block]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // loader (threads 0..127): expert block rb (8 experts), column block cb (8 columns)
  const int rb = tid & 3, cbk = tid >> 2;
  // the next 32 experts' dl and gate rows are loaded into registers while the
  // current ones are multiplied from LDS
  float dv[8];
  uint4 blk[8];
  auto load_step = [&](int k0) {
    // dl: token tid / 4, experts 8 (tid % 4) .. + 7 (split once for all waves)
    const int t = t0 + (tid >> 2), ee = k0 + 8 * (tid & 3);
#pragma unroll
    for (int q = 0; q < 8; ++q) dv[q] = (t < a.T && ee + q < a.N) ? a.dl[size_t(t) * a.N + ee + q] : 0.f;
    if (tid < 128) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int e = k0 + 8 * rb + r;
        blk[r] = e < a.N ? *reinterpret_cast<const uint4*>(wg + size_t(e) * a.d + c0 + 8 * cbk)
                         : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  load_step(0);
  for (int k0 = 0; k0 < a.N; k0 += 32) {
    {
      bf16x8_t hi, lo;
      rx_split(dv, hi, lo);
      *reinterpret_cast<bf16x8_t*>(sLh + (tid >> 2) * RX_RS + 8 * (tid & 3)) = hi;
      *reinterpret_cast<bf16x8_t*>(sLl + (tid >> 2) * RX_RS + 8 * (tid & 3)) = lo;
    }
    if (tid < 128) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t w4[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint4& x0 = blk[2 * p];
          const uint4& x1 = blk[2 * p + 1];
          const uint32_t v0 = (c >> 1) == 0 ? x0.x : (c >> 1) == 1 ? x0.y : (c >> 1) == 2 ? x0.z : x0.w;
          const uint32_t v1 = (c >> 1) == 0 ? x1.x : (c >> 1) == 1 ? x1.y : (c >> 1) == 2 ? x1.z : x1.w;
          w4[p] = (c & 1) ? ((v0 >> 16) | (v1 & 0xFFFF0000u)) : ((v0 & 0xFFFFu) | (v1 << 16));
        }
        *reinterpret_cast<uint4*>(sW + (8 * cbk + c) * RX_RS + 8 * rb) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    }
    __syncthreads();
    if (k0 + 32 < a.N) load_step(k0 + 32);  // uniform
    bf16x8_t wf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wf[i] = *reinterpret_cast<const bf16x8_t*>(sW + (64 * wave + 16 * i + l16) * RX_RS + 8 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t hi = *reinterpret_cast<const bf16x8_t*>(sLh + (16 * j + l16) * RX_RS + 8 * g);
      const bf16x8_t lo = *reinterpret_cast<const bf16x8_t*>(sLl + (16 * j + l16) * RX_RS + 8 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i], hi, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i], lo, acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();  // sW is rewritten next
  }
  // acc[i][j][v] = dx[token t0 + 16 j + l16][column c0 + 64 wave + 16 i + 4 g + v]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + 16 * j + l16;
    if (t < a.T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = c0 + 64 * wave + 16 * i + 4 * g;
        float* o = a.dx + size_t(t) * a.d + c;  // dx is only 4-byte aligned
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = acc[i][j][v];
      }
    }
  }
}

// dW_g on the matrix cores (bf16 x, width a multiple of 256): a workgroup
// takes 64 experts x 256 columns over one token range, wave w the columns
// 64 w .. 64 w + 63 of all 64 experts; K runs over the range's tokens 32 at a
// time.  Both operands have the token outermost, so each step goes through
// LDS with the token innermost: dl (fp32) split into hi + lo bf16 terms, a
// thread writing 8 experts of one token; x as 8 x 8 blocks transposed in
// registers.  The ranges' partial sums are added in order by router_red_kernel.
constexpr int RW2_RS = 40;  // LDS row stride (bf16): 32 tokens + 8

__global__ __launch_bounds__(256) void router_dwg_mfma_kernel(RouterBwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sDh[64 * RW2_RS];   // [expert][token] hi
  __shared__ __attribute__((aligned(16))) uint16_t sDl[64 * RW2_RS];   // [expert][token] lo
  __shared__ __attribute__((aligned(16))) uint16_t sXt[256 * RW2_RS];  // [column][token]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int neb = (a.N + 63) / 64, ncb = a.d / 256, tiles = neb * ncb;
  const int b = blockIdx.x % tiles, split = blockIdx.x / tiles;
  const int e0 = (b % neb) * 64, c0 = (b / neb) * 256;
  const int ta = split * a.tchunk, tb = min(a.T, ta + a.tchunk);
  const uint16_t* xg = static_cast<const uint16_t*>(a.x);
  f32x4_t acc[4][4];  // [expert block][column block]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // dl loader: token tl = tid / 8, experts 8 (tid % 8) .. + 7;
  // x loader (threads 0..127): token block rb (8 tokens), column block cbk (8 columns)
  const int tl = tid >> 3, eg = tid & 7, rb = tid & 3, cbk = tid >> 2;
  // the next 32 tokens' dl and x are loaded into registers while the current
  // ones are multiplied from LDS
  float dv[8];
  uint4 blk[8];
  auto load_step = [&](int k0) {
    const int t = k0 + tl;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = e0 + 8 * eg + q;
      dv[q] = (t < tb && e < a.N) ? a.dl[size_t(t) * a.N + e] : 0.f;
    }
    if (tid < 128) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int tr = k0 + 8 * rb + r;
        blk[r] = tr < tb ? *reinterpret_cast<const uint4*>(xg + size_t(tr) * a.d + c0 + 8 * cbk)
                         : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  load_step(ta);
  for (int k0 = ta; k0 < tb; k0 += 32) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const __bf16 h = (__bf16)dv[q];
      const __bf16 l = (__bf16)(dv[q] - (float)h);
      sDh[(8 * eg + q) * RW2_RS + tl] = __builtin_bit_cast(uint16_t, h);
      sDl[(8 * eg + q) * RW2_RS + tl] = __builtin_bit_cast(uint16_t, l);
    }
    if (tid < 128) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t w4[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint4& x0 = blk[2 * p];
          const uint4& x1 = blk[2 * p + 1];
          const uint32_t v0 = (c >> 1) == 0 ? x0.x : (c >> 1) == 1 ? x0.y : (c >> 1) == 2 ? x0.z : x0.w;
          const uint32_t v1 = (c >> 1) == 0 ? x1.x : (c >> 1) == 1 ? x1.y : (c >> 1) == 2 ? x1.z : x1.w;
          w4[p] = (c & 1) ? ((v0 >> 16) | (v1 & 0xFFFF0000u)) : ((v0 & 0xFFFFu) | (v1 << 16));
        }
        *reinterpret_cast<uint4*>(sXt + (8 * cbk + c) * RW2_RS + 8 * rb) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    }
    __syncthreads();
    if (k0 + 32 < tb) load_step(k0 + 32);  // uniform
    bf16x8_t xf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xf[j] = *reinterpret_cast<const bf16x8_t*>(sXt + (64 * wave + 16 * j + l16) * RW2_RS + 8 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8_t hi = *reinterpret_cast<const bf16x8_t*>(sDh + (16 * i + l16) * RW2_RS + 8 * g);
      const bf16x8_t lo = *reinterpret_cast<const bf16x8_t*>(sDl + (16 * i + l16) * RW2_RS + 8 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, xf[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, xf[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();  // the tiles are rewritten next
  }
  // acc[i][j][v] = dW_g[e0 + 16 i + 4 g + v][c0 + 64 wave + 16 j + l16]
  float* dst = a.S > 1 ? a.part + size_t(split) * a.N * a.d : a.dwg;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = e0 + 16 * i + 4 * g + v;
      if (e < a.N) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[size_t(e) * a.d + c0 + 64 * wave + 16 * j + l16] = acc[i][j][v];
      }
    }
}

// dW_g (or the split's partial) for experts nb .. nb+15, columns cb .. cb+255
template <int A>
__global__ __launch_bounds__(256) void router_dwg_kernel(RouterBwdArgs a) {
  const int nblk = (a.N + RB_NB - 1) / RB_NB, cblk = (a.d + 255) / 256;
  const int b = blockIdx.x % (nblk * cblk), split = blockIdx.x / (nblk * cblk);
  const int n0 = (b % nblk) * RB_NB, i = (b / nblk) * 256 + threadIdx.x;
  const int ta = split * a.tchunk, tb = min(a.T, ta + a.tchunk);
  __shared__ __attribute__((aligned(16))) float sL[256][RB_NB];  // dl of 256 tokens for the block's experts
  float acc[RB_NB];
#pragma unroll
  for (int q = 0; q < RB_NB; ++q) acc[q] = 0.f;
  for (int tc = ta; tc < tb; tc += 256) {
    const int tn = min(256, tb - tc);
    for (int q = threadIdx.x; q < tn * RB_NB; q += 256) {
      const int t = q / RB_NB, e = q % RB_NB;
      sL[t][e] = n0 + e < a.N ? a.dl[size_t(tc + t) * a.N + n0 + e] : 0.f;
    }
    __syncthreads();
    if (i < a.d) {
      for (int t = 0; t < tn; ++t) {
        const float xv = load1<A>(a.x, size_t(tc + t) * a.d + i);
#pragma unroll
        for (int q = 0; q < RB_NB; q += 4) {
          const float4 l = *reinterpret_cast<const float4*>(&sL[t][q]);
          acc[q] = fmaf(l.x, xv, acc[q]);
          acc[q + 1] = fmaf(l.y, xv, acc[q + 1]);
          acc[q + 2] = fmaf(l.z, xv, acc[q + 2]);
          acc[q + 3] = fmaf(l.w, xv, acc[q + 3]);
        }
      }
    }
    __syncthreads();  // sL is replaced next
  }
  float* dst = a.S > 1 ? a.part + size_t(split) * a.N * a.d : a.dwg;
#pragma unroll
  for (int q = 0; q < RB_NB; ++q)
    if (n0 + q < a.N && i < a.d) dst[size_t(n0 + q) * a.d + i] = acc[q];
}

__global__ __launch_bounds__(256) void router_red_kernel(RouterBwdArgs a) {
  const size_t ND = size_t(a.N) * a.d, q = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (q >= ND) return;
  float s = a.part[q];
  for (int k = 1; k < a.S; ++k) s += a.part[size_t(k) * ND + q];
  a.dwg[q] = s;
}

__global__ __launch_bounds__(256) void router_zero_kernel(float* p, size_t n) {
  const size_t q = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (q < n) p[q] = 0.f;
}

// token ranges of the dW_g pass: none when its tiles reach 2048 workgroups
// (512 for the matrix-core pass), else up to that many with at least 256
// tokens each (64 for the matrix-core pass)
int router_bwd_splits(int T, int d, int N, int bf16, int* tchunk) {
  const bool mf = bf16 && d % 256 == 0;  // matrix-core pass: 64 x 256 tiles, about 512 workgroups
  const int tiles = mf ? ((N + 63) / 64) * (d / 256) : ((N + RB_NB - 1) / RB_NB) * ((d + 255) / 256);
  const int target = mf ? 512 : 2048, tmin = mf ? 64 : 256;  // workgroups, tokens per range
  int S = 1;
  if (tiles < target) {
    S = (target + tiles - 1) / tiles;
    const int smax = (T + tmin - 1) / tmin;
    S = S < smax ? S : smax;
    S = S < 1 ? 1 : S;
  }
  int tc = (T + S - 1) / S;
  if (tc < 1) tc = 1;
  S = (T + tc - 1) / tc;
  if (S < 1) S = 1;
  if (tchunk) *tchunk = tc;
  return S;
}

static size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

// the larger of the two dW_g passes' needs (the query does not know the dtype)
size_t router_bwd_workspace(int T, int d, int N) {
  if (T <= 0) return 0;
  const int S0 = router_bwd_splits(T, d, N, 0, nullptr), S1 = router_bwd_splits(T, d, N, 1, nullptr);
  const int S = S0 > S1 ? S0 : S1;
  return al256(size_t(T) * N * 4) + (S > 1 ? size_t(S) * N * d * 4 : 0);
}

hipError_t launch_router_bwd(const void* x, const void* wg, const int32_t* idx, const float* dgate, float* dx,
                             float* dwg, void* ws, int T, int d, int N, int k, int renorm, int act, hipStream_t s) {
  if (T <= 0) {
    const size_t n = size_t(N) * d;
    hipLaunchKernelGGL(router_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, dwg, n);
    return hipGetLastError();
  }
  RouterBwdArgs a{x, wg, idx, dgate, static_cast<float*>(ws), dx, dwg, nullptr, T, d, N, k, renorm, 1, 0};
  a.S = router_bwd_splits(T, d, N, act == ACT_BF16, &a.tchunk);
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + al256(size_t(T) * N * 4));
  const bool bf = act == ACT_BF16;
  // logits and dl: 16-token blocks, 4 or 2 per workgroup on the matrix cores
  // while that leaves at least 512 workgroups (the gate matrix is read once
  // per workgroup)
  const int tiles = (T + RB_BT - 1) / RB_BT;
  const int tb = bf && d % 32 == 0 ? (tiles / 4 >= 512 ? 4 : tiles / 2 >= 512 ? 2 : 1) : 1;
  const dim3 tgrid((tiles + tb - 1) / tb);
  if (tb == 4) hipLaunchKernelGGL((router_dl_kernel<ACT_BF16, 4>), tgrid, dim3(256), 0, s, a);
  else if (tb == 2) hipLaunchKernelGGL((router_dl_kernel<ACT_BF16, 2>), tgrid, dim3(256), 0, s, a);
  else if (bf) hipLaunchKernelGGL((router_dl_kernel<ACT_BF16, 1>), tgrid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((router_dl_kernel<ACT_F32, 1>), tgrid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dx: 64-token tiles of 512 columns when the tokens are many (the gate
  // matrix is read once per tile), else 16-token tiles of all columns
  const int cpt = (d + 255) / 256;
#define RB_DX(BT, C)                                                                                          \
  {                                                                                                            \
    const dim3 g(unsigned(((T + BT - 1) / BT) * ((d + 256 * C - 1) / (256 * C))));                             \
    if (bf) hipLaunchKernelGGL((router_dx_kernel<ACT_BF16, BT, C>), g, dim3(256), 0, s, a);                    \
    else hipLaunchKernelGGL((router_dx_kernel<ACT_F32, BT, C>), g, dim3(256), 0, s, a);                        \
  }
  if (bf && d % 256 == 0) {
    hipLaunchKernelGGL(router_dx_mfma_kernel, dim3(unsigned(((T + 63) / 64) * (d / 256))), dim3(256), 0, s, a);
  } else if (T >= 16384) RB_DX(64, 2)
  else if (cpt <= 1) RB_DX(16, 1)
  else if (cpt <= 2) RB_DX(16, 2)
  else if (cpt <= 4) RB_DX(16, 4)
  else RB_DX(16, 8)
#undef RB_DX
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (bf && d % 256 == 0) {
    const int tiles = ((N + 63) / 64) * (d / 256);
    hipLaunchKernelGGL(router_dwg_mfma_kernel, dim3(tiles * a.S), dim3(256), 0, s, a);
  } else {
    const int tiles = ((N + RB_NB - 1) / RB_NB) * ((d + 255) / 256);
    if (bf) hipLaunchKernelGGL(router_dwg_kernel<ACT_BF16>, dim3(tiles * a.S), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(router_dwg_kernel<ACT_F32>, dim3(tiles * a.S), dim3(256), 0, s, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess || a.S == 1) return e;
  hipLaunchKernelGGL(router_red_kernel, dim3((size_t(N) * d + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bmoe
