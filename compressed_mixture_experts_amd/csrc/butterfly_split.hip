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
#include "mfma_factors.hpp"

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

// ---------------------------------------------------------------- matrix-core low part
// Widths 4096 (S = 8) and 8192 (S = 9).  The low part of a chunk is G1 G0 with
//   G0 = stages 0 .. S-5: block-diagonal over runs of P0 = 2^(S-4) consecutive
//        indices (P0 x P0 blocks: 32 at S = 9, 16 at S = 8),
//   G1 = stages S-4 .. S-1: block-diagonal over the 16 indices u + P0 j (j < 16)
//        of each u < P0 (16 x 16 blocks),
// every block the product of its stages' rotations (the pair structure of each
// stage stays inside one block).  The blocks depend on the angles only, so they
// are built once per weight set, in bf16 and in the per-lane order of the MFMA
// operands; a workgroup then multiplies its 64-row tile (bf16, in LDS) by both
// factors: B x = G1 (G0 x), B^T x = G0^T (G1^T x).

template <int S>
struct LowMCfg {
  static constexpr int P0 = 1 << (S - 4);    // G0 block width = number of G1 blocks
  static constexpr int NB0 = (1 << S) / P0;  // G0 blocks per chunk (16)
  static constexpr int H0 = P0 / 16;         // 16-row halves of a G0 block
  static constexpr int RS = (1 << S) + 4;    // LDS row stride in bf16 (8-byte aligned rows)
  static constexpr int ROWS = SP_RB;
  static constexpr size_t g0_bytes = size_t(NB0) * P0 * P0 * 2;
  static constexpr size_t g1_bytes = size_t(P0) * 256 * 2;
  static constexpr size_t chunk_bytes = g0_bytes + g1_bytes;
  static constexpr size_t per_expert = 16 * chunk_bytes;
  static constexpr size_t lds_bytes = size_t(ROWS) * RS * 2;
  // G1 contraction slot 4g+i holds j = (g&1) DJ + (g>>1) (6-DJ) + (i&1) + 8 (i>>1):
  // lane groups 0 and 1 then read LDS words 32 banks apart
  static constexpr int DJ = S == 9 ? 2 : 4;
};

template <int S>
__host__ __device__ constexpr int g1_slot(int g, int i) {
  return (g & 1) * LowMCfg<S>::DJ + (g >> 1) * (6 - LowMCfg<S>::DJ) + (i & 1) + 8 * (i >> 1);
}

typedef short lm_s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t lm_mfma16(uint2 a, uint2 b) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(lm_s16x4_t, a),
                                                    __builtin_bit_cast(lm_s16x4_t, b),
                                                    f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t lm_mfma32(uint4 a, uint4 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}
__device__ __forceinline__ uint2 lm_pack4(const f32x4_t& d) {
  return make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
}
__device__ __forceinline__ uint2 lm_ld64(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ void lm_st64(uint16_t* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }

// Factor fragments one wave keeps: G0 blocks 4w .. 4w+3, G1 blocks (u) P0/4 w ..
template <int S> struct LowFrag;
template <> struct LowFrag<9> { uint4 g0[4][2]; uint2 g1[8]; };
template <> struct LowFrag<8> { uint4 g0_unused; uint2 g0[4][1]; uint2 g1[4]; };

// G0 on the tile: wave w owns blocks 4w .. 4w+3 in all 64 rows.  Operand B of
// row r: the block's contraction values held by lane group g (S = 9: inputs
// 8g .. 8g+7; S = 8: 4g .. 4g+3); the products overwrite the same elements.
template <int S>
__device__ __forceinline__ void lowm_g0(uint16_t* tile, const LowFrag<S>& F, int wave, int g, int l16) {
  using C = LowMCfg<S>;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const int b = 4 * wave + bb;
#pragma unroll
    for (int rg = 0; rg < C::ROWS / 16; ++rg) {
      uint16_t* rp = tile + (16 * rg + l16) * C::RS + C::P0 * b;
      if constexpr (S == 9) {
        const uint2 x0 = lm_ld64(rp + 8 * g), x1 = lm_ld64(rp + 8 * g + 4);
        const uint4 bx = make_uint4(x0.x, x0.y, x1.x, x1.y);
        const f32x4_t d0 = lm_mfma32(F.g0[bb][0], bx), d1 = lm_mfma32(F.g0[bb][1], bx);
        lm_st64(rp + 4 * g, lm_pack4(d0));
        lm_st64(rp + 16 + 4 * g, lm_pack4(d1));
      } else {
        const f32x4_t d = lm_mfma16(F.g0[bb][0], lm_ld64(rp + 4 * g));
        lm_st64(rp + 4 * g, lm_pack4(d));
      }
    }
  }
}

// G1 on the tile: wave w owns u = P0/4 w .. in groups of 4 consecutive u; lane
// group g reads, for each of its 4 slots, the 4 u's of one j at once (8 bytes)
// and regroups them per u.
template <int S>
__device__ __forceinline__ void lowm_g1(uint16_t* tile, const LowFrag<S>& F, int wave, int g, int l16) {
  using C = LowMCfg<S>;
  constexpr int UW = C::P0 / 4;  // u per wave
#pragma unroll
  for (int uq = 0; uq < UW / 4; ++uq) {
    const int u0 = UW * wave + 4 * uq;
#pragma unroll
    for (int rg = 0; rg < C::ROWS / 16; ++rg) {
      uint16_t* rp = tile + (16 * rg + l16) * C::RS + u0;
      uint2 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = lm_ld64(rp + C::P0 * g1_slot<S>(g, i));
      f32x4_t d[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
        const uint2 bq = (q < 2) ? make_uint2(__builtin_amdgcn_perm(r[1].x, r[0].x, sel), __builtin_amdgcn_perm(r[3].x, r[2].x, sel))
                                 : make_uint2(__builtin_amdgcn_perm(r[1].y, r[0].y, sel), __builtin_amdgcn_perm(r[3].y, r[2].y, sel));
        d[q] = lm_mfma16(F.g1[4 * uq + q], bq);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lm_st64(rp + C::P0 * g1_slot<S>(g, i),
                make_uint2(pack_bf16x2(d[0][i], d[1][i]), pack_bf16x2(d[2][i], d[3][i])));
    }
  }
}

// Low part on the matrix cores (in place allowed): WG = (tile of <= 64 rows of
// one expert, chunk).  Rows past the tile's last repeat it and are not stored.
template <int S, bool TRANS>
__global__ __launch_bounds__(BF_THREADS) void lowm_kernel(BflyArgs a) {
  using C = LowMCfg<S>;
  constexpr int L = S + 4, n = 1 << L;
  constexpr int PPR = (1 << S) / 8;                 // 16-byte pieces per row
  constexpr int PPT = C::ROWS * PPR / BF_THREADS;   // per thread
  constexpr int BATCH = PPT < 8 ? PPT : 8;
  extern __shared__ __attribute__((aligned(16))) uint16_t tile[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int t = blockIdx.x / 16, c = blockIdx.x % 16;
  int e, r0, nr;
  sp_find_tile(a.offsets, a.n_experts, t, e, r0, nr);
  if (e < 0) return;

  const unsigned char* fc = a.fac + (size_t(e) * 16 + c) * C::chunk_bytes;
  LowFrag<S> F;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    if constexpr (S == 9) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        F.g0[bb][h] = *reinterpret_cast<const uint4*>(fc + ((size_t(4 * wave + bb) * 2 + h) * 64 + lane) * 16);
    } else {
      F.g0[bb][0] = *reinterpret_cast<const uint2*>(fc + (size_t(4 * wave + bb) * 64 + lane) * 8);
    }
  }
#pragma unroll
  for (int q = 0; q < C::P0 / 4; ++q)
    F.g1[q] = *reinterpret_cast<const uint2*>(fc + C::g0_bytes + (size_t(C::P0 / 4 * wave + q) * 64 + lane) * 8);

  const uint16_t* in = reinterpret_cast<const uint16_t*>(a.in) + size_t(r0) * n + c * (1 << S);
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + size_t(r0) * n + c * (1 << S);
#pragma unroll
  for (int k0 = 0; k0 < PPT; k0 += BATCH) {
    uint4 v[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int q = (k0 + k) * BF_THREADS + tid, r = q / PPR, j = q % PPR;
      v[k] = *reinterpret_cast<const uint4*>(in + size_t(min(r, nr - 1)) * n + 8 * j);
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int q = (k0 + k) * BF_THREADS + tid, r = q / PPR, j = q % PPR;
      uint16_t* d = tile + r * C::RS + 8 * j;
      lm_st64(d, make_uint2(v[k].x, v[k].y));
      lm_st64(d + 4, make_uint2(v[k].z, v[k].w));
    }
  }
  __syncthreads();
  if constexpr (!TRANS) {
    lowm_g0<S>(tile, F, wave, g, l16);
    __syncthreads();
    lowm_g1<S>(tile, F, wave, g, l16);
  } else {
    lowm_g1<S>(tile, F, wave, g, l16);
    __syncthreads();
    lowm_g0<S>(tile, F, wave, g, l16);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int q = k * BF_THREADS + tid, r = q / PPR, j = q % PPR;
    if (r < nr) {
      const uint16_t* sp = tile + r * C::RS + 8 * j;
      const uint2 x0 = lm_ld64(sp), x1 = lm_ld64(sp + 4);
      *reinterpret_cast<uint4*>(out + size_t(r) * n + 8 * j) = make_uint4(x0.x, x0.y, x1.x, x1.y);
    }
  }
}

// Builder: one workgroup per (expert, chunk).  (cos, sin) of the chunk's S
// stages into LDS, then one job per operand row: G0 (block b, output o), G1
// (u, output slot).  Operand row o of M is M^T e_o (stages in decreasing order,
// transposed rotations); of M^T it is M e_o.
template <int S, bool TRANS>
__global__ __launch_bounds__(BF_THREADS) void lowfac_kernel(const float* __restrict__ ang, unsigned char* __restrict__ out) {
  using C = LowMCfg<S>;
  constexpr int L = S + 4, half = 1 << (L - 1), hc = 1 << (S - 1);
  constexpr int P0 = C::P0;
  __shared__ float2 cs[S * hc];
  const int tid = threadIdx.x;
  const int e = blockIdx.x / 16, c = blockIdx.x % 16;
  const float* ae = ang + size_t(e) * L * half + size_t(c) * hc;
  for (int idx = tid; idx < S * hc; idx += BF_THREADS) cs[idx] = sincos_rev(ae[(idx / hc) * half + idx % hc]);
  __syncthreads();
  unsigned char* fc = out + (size_t(e) * 16 + c) * C::chunk_bytes;
  constexpr int J0 = C::NB0 * P0, J1 = P0 * 16;
  for (int job = tid; job < J0 + J1; job += BF_THREADS) {
    if (job < J0) {
      const int b = job / P0, o = job % P0;
      float v[P0];
#pragma unroll
      for (int q = 0; q < P0; ++q) v[q] = q == o ? 1.0f : 0.0f;
      rotate_vec<P0, 0, S - 4, TRANS>(v, cs, hc, P0 * b, 1);
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        if constexpr (S == 9) {
          uint4 w;
          w.x = pack_bf16x2(v[8 * gq + 0], v[8 * gq + 1]);
          w.y = pack_bf16x2(v[8 * gq + 2], v[8 * gq + 3]);
          w.z = pack_bf16x2(v[8 * gq + 4], v[8 * gq + 5]);
          w.w = pack_bf16x2(v[8 * gq + 6], v[8 * gq + 7]);
          *reinterpret_cast<uint4*>(fc + ((size_t(b) * 2 + o / 16) * 64 + 16 * gq + o % 16) * 16) = w;
        } else {
          *reinterpret_cast<uint2*>(fc + (size_t(b) * 64 + 16 * gq + o) * 8) =
              make_uint2(pack_bf16x2(v[4 * gq], v[4 * gq + 1]), pack_bf16x2(v[4 * gq + 2], v[4 * gq + 3]));
        }
      }
    } else {
      const int jj = job - J0, u = jj / 16, l = jj % 16;
      const int jo = g1_slot<S>(l >> 2, l & 3);
      float v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = q == jo ? 1.0f : 0.0f;
      rotate_vec<16, S - 4, S, TRANS>(v, cs, hc, u, P0);
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        *reinterpret_cast<uint2*>(fc + C::g0_bytes + (size_t(u) * 64 + 16 * gq + l) * 8) =
            make_uint2(pack_bf16x2(v[g1_slot<S>(gq, 0)], v[g1_slot<S>(gq, 1)]),
                       pack_bf16x2(v[g1_slot<S>(gq, 2)], v[g1_slot<S>(gq, 3)]));
    }
  }
}

size_t low_factor_bytes(int log2n) {
  return log2n == 12 ? LowMCfg<8>::per_expert : log2n == 13 ? LowMCfg<9>::per_expert : 0;
}

hipError_t launch_low_factor_prep(const float* ang, unsigned char* out, int n_experts, int log2n, bool trans,
                                  hipStream_t s) {
  if (n_experts <= 0) return hipSuccess;
  const dim3 grid(n_experts * 16), block(BF_THREADS);
  switch (log2n) {
    case 12:
      if (trans) hipLaunchKernelGGL((lowfac_kernel<8, true>), grid, block, 0, s, ang, out);
      else hipLaunchKernelGGL((lowfac_kernel<8, false>), grid, block, 0, s, ang, out);
      break;
    case 13:
      if (trans) hipLaunchKernelGGL((lowfac_kernel<9, true>), grid, block, 0, s, ang, out);
      else hipLaunchKernelGGL((lowfac_kernel<9, false>), grid, block, 0, s, ang, out);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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

// ---------------------------------------------------------------- matrix-core high part
// The high part of column v is one 16 x 16 matrix H_v (stages S .. S+3 on the
// indices v + 2^S j), built once per weight set in bf16 and MFMA operand
// order: operand row l holds output j = (l >> 2) + 4 (l & 3), contraction slot
// 4g + i input j = g + 4i (so lane groups 0 and 1 read LDS words 32 banks
// apart).  The accumulator rows 4g + i then hold output j = g + 4i, the order
// of the next product's operand, so the FFN middle chains two products with
// the GELU in between without moving data.

template <int S>
struct HighMCfg {
  static constexpr int NV = 1 << S;                       // columns
  static constexpr size_t per_expert = size_t(NV) * 512;  // one 16 x 16 bf16 block per column
  static constexpr int RT = 16;                           // rows per sub-tile
  static constexpr int RSB = 16 * SP_VC * 2 + 8;          // LDS bytes per row: [16 j][64 v] bf16 + pad
  static constexpr size_t lds_bytes = size_t(RT) * RSB;
};

// Builder: one workgroup per (expert, 16 columns); thread = (column, output
// slot).  Operand row j of H is H^T e_j, of H^T it is H e_j.
template <int S, bool TRANS>
__global__ __launch_bounds__(BF_THREADS) void hfac_kernel(const float* __restrict__ ang, unsigned char* __restrict__ out) {
  constexpr int L = S + 4, half = 1 << (L - 1);
  constexpr int NB = HighMCfg<S>::NV / 16;
  __shared__ float2 cs[16][32];
  const int tid = threadIdx.x;
  const int e = blockIdx.x / NB, v0 = (blockIdx.x % NB) * 16;
  const float* ae = ang + size_t(e) * L * half;
  for (int idx = tid; idx < 16 * 32; idx += BF_THREADS) {
    const int c = idx / 32, t = (idx % 32) / 8, q = idx % 8;
    cs[c][idx % 32] = sincos_rev(ae[(S + t) * half + (q << S) + v0 + c]);
  }
  __syncthreads();
  const int c = tid / 16, l = tid % 16;
  const int jo = (l >> 2) + 4 * (l & 3);
  float x[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) x[q] = q == jo ? 1.0f : 0.0f;
  rotate_group<4, !TRANS>(x, cs[c]);
  unsigned char* dst = out + size_t(e) * HighMCfg<S>::per_expert + size_t(v0 + c) * 512;
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<uint2*>(dst + (16 * g + l) * 8) =
        make_uint2(pack_bf16x2(x[g], x[g + 4]), pack_bf16x2(x[g + 8], x[g + 12]));
}

// High part on the matrix cores.  WG = (tile of <= 64 rows of one expert, 64
// columns); sub-tiles of 16 rows go through LDS as [row][16 j][64 v] bf16
// (coalesced 16-byte loads and stores); wave w multiplies columns 16w .. 16w+15
// in groups of 4, reading each j's 4 columns with one 8-byte LDS read.
template <int S, int MODE>
__global__ __launch_bounds__(BF_THREADS, 4) void highm_kernel(BflyArgs a) {
  using C = HighMCfg<S>;
  constexpr int L = S + 4, n = 1 << L;
  constexpr int ncb = C::NV / SP_VC;
  constexpr int PPT = C::RT * 16 * (SP_VC / 8) / BF_THREADS;  // 16-byte pieces per thread (8)
  extern __shared__ __attribute__((aligned(16))) unsigned char hl[];
  __shared__ size_t s_row[SP_RB];
  __shared__ float s_g[SP_RB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int t = blockIdx.x / ncb, cb = blockIdx.x % ncb;
  int e, r0, nr;
  sp_find_tile(a.offsets, a.n_experts, t, e, r0, nr);
  if (e < 0) return;

  const int vw = cb * SP_VC + 16 * wave;  // this wave's first column
  uint2 fa0[16], fa1[MODE == SH_MID ? 16 : 1];
  const unsigned char* f0 = a.fac + size_t(e) * C::per_expert;
#pragma unroll
  for (int c = 0; c < 16; ++c) fa0[c] = *reinterpret_cast<const uint2*>(f0 + (size_t(vw + c) * 64 + lane) * 8);
  if constexpr (MODE == SH_MID) {
    const unsigned char* f1 = a.fac1 + size_t(e) * C::per_expert;
#pragma unroll
    for (int c = 0; c < 16; ++c) fa1[c] = *reinterpret_cast<const uint2*>(f1 + (size_t(vw + c) * 64 + lane) * 8);
  }
  const uint16_t* in = reinterpret_cast<const uint16_t*>(a.in);
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  // row tables of all the tile's rows (source or destination row, gate)
  if (tid < SP_RB) {
    const int q = r0 + min(tid, nr - 1);
    if constexpr (MODE == SH_IN) {
      s_row[tid] = size_t(a.perm[q] / a.top_k) * n;
    } else if constexpr (MODE == SH_OUT) {
      const int slot = a.perm[q];
      s_row[tid] = size_t(slot) * n;
      s_g[tid] = a.gate[slot];
    } else {
      s_row[tid] = size_t(q) * n;
    }
  }
  __syncthreads();
  // piece p = (row, j, 8 columns) of a sub-tile; rows past the tile's last repeat it
  auto load = [&](int rs, uint4 (&v)[PPT]) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = k * BF_THREADS + tid, row = min(rs + p / 128, nr - 1), j = (p / 8) % 16, vc = p % 8;
      const size_t src = MODE == SH_OUT ? size_t(r0 + row) * n : s_row[row];
      v[k] = *reinterpret_cast<const uint4*>(in + src + (size_t(j) << S) + cb * SP_VC + 8 * vc);
    }
  };
  for (int rs = 0; rs < nr; rs += C::RT) {
    const int m = min(C::RT, nr - rs);
    uint4 v[PPT];
    load(rs, v);
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = k * BF_THREADS + tid, row = p / 128, j = (p / 8) % 16, vc = p % 8;
      uint16_t* d = reinterpret_cast<uint16_t*>(hl + row * C::RSB) + j * SP_VC + 8 * vc;
      lm_st64(d, make_uint2(v[k].x, v[k].y));
      lm_st64(d + 4, make_uint2(v[k].z, v[k].w));
    }
    __syncthreads();
    const float gr = MODE == SH_OUT ? s_g[rs + min(l16, m - 1)] : 1.0f;
    uint16_t* rp = reinterpret_cast<uint16_t*>(hl + l16 * C::RSB) + 16 * wave;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      uint2 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = lm_ld64(rp + (g + 4 * i) * SP_VC + 4 * qd);
      f32x4_t d[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
        const uint2 bq = (q < 2) ? make_uint2(__builtin_amdgcn_perm(r[1].x, r[0].x, sel), __builtin_amdgcn_perm(r[3].x, r[2].x, sel))
                                 : make_uint2(__builtin_amdgcn_perm(r[1].y, r[0].y, sel), __builtin_amdgcn_perm(r[3].y, r[2].y, sel));
        d[q] = lm_mfma16(fa0[4 * qd + q], bq);
        if constexpr (MODE == SH_MID) {
          if (a.gelu) {
#pragma unroll
            for (int i = 0; i < 4; ++i) d[q][i] = gelu_erf(d[q][i]);
          }
          d[q] = lm_mfma16(fa1[4 * qd + q], lm_pack4(d[q]));
        }
        if constexpr (MODE == SH_OUT) {
#pragma unroll
          for (int i = 0; i < 4; ++i) d[q][i] *= gr;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lm_st64(rp + (g + 4 * i) * SP_VC + 4 * qd,
                make_uint2(pack_bf16x2(d[0][i], d[1][i]), pack_bf16x2(d[2][i], d[3][i])));
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = k * BF_THREADS + tid, row = p / 128, j = (p / 8) % 16, vc = p % 8;
      if (row < m) {
        const uint16_t* sp = reinterpret_cast<const uint16_t*>(hl + row * C::RSB) + j * SP_VC + 8 * vc;
        const uint2 x0 = lm_ld64(sp), x1 = lm_ld64(sp + 4);
        const size_t dst = MODE == SH_OUT ? s_row[rs + row] : size_t(r0 + rs + row) * n;
        *reinterpret_cast<uint4*>(out + dst + (size_t(j) << S) + cb * SP_VC + 8 * vc) = make_uint4(x0.x, x0.y, x1.x, x1.y);
      }
    }
    __syncthreads();  // stored before the next sub-tile is written
  }
}

size_t high_factor_bytes(int log2n) {
  switch (log2n) {
    case 10: return HighMCfg<6>::per_expert;
    case 11: return HighMCfg<7>::per_expert;
    case 12: return HighMCfg<8>::per_expert;
    case 13: return HighMCfg<9>::per_expert;
    default: return 0;
  }
}

template <int S>
static hipError_t launch_hfac_S(const float* ang, unsigned char* out, int n_experts, bool trans, hipStream_t s) {
  const dim3 grid(n_experts * (HighMCfg<S>::NV / 16)), block(BF_THREADS);
  if (trans) hipLaunchKernelGGL((hfac_kernel<S, true>), grid, block, 0, s, ang, out);
  else hipLaunchKernelGGL((hfac_kernel<S, false>), grid, block, 0, s, ang, out);
  return hipGetLastError();
}

hipError_t launch_high_factor_prep(const float* ang, unsigned char* out, int n_experts, int log2n, bool trans,
                                   hipStream_t s) {
  if (n_experts <= 0) return hipSuccess;
  switch (log2n) {
    case 10: return launch_hfac_S<6>(ang, out, n_experts, trans, s);
    case 11: return launch_hfac_S<7>(ang, out, n_experts, trans, s);
    case 12: return launch_hfac_S<8>(ang, out, n_experts, trans, s);
    case 13: return launch_hfac_S<9>(ang, out, n_experts, trans, s);
    default: return hipErrorInvalidValue;
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
  if constexpr (S == 8 || S == 9) {
    if (a.fac) {
      static int mdone[2][64] = {{0}};
      if (trans) return sp_launch(lowm_kernel<S, true>, grid, LowMCfg<S>::lds_bytes, a, s, mdone[1]);
      return sp_launch(lowm_kernel<S, false>, grid, LowMCfg<S>::lds_bytes, a, s, mdone[0]);
    }
  }
  if (trans) return sp_launch(bsplit_low_kernel<S, true>, grid, LowCfg<S>::lds_bytes, a, s, done[1]);
  return sp_launch(bsplit_low_kernel<S, false>, grid, LowCfg<S>::lds_bytes, a, s, done[0]);
}

template <int S>
static hipError_t launch_high_S(const BflyArgs& a, int mode, hipStream_t s) {
  static int done[64] = {0};
  const int grid = sp_tiles(a) * ((1 << S) / SP_VC);
  if (a.fac && (mode != SH_MID || a.fac1)) {
    const size_t lds = HighMCfg<S>::lds_bytes;
    switch (mode) {
      case SH_IN: return sp_launch(highm_kernel<S, SH_IN>, grid, lds, a, s, done);
      case SH_MID: return sp_launch(highm_kernel<S, SH_MID>, grid, lds, a, s, done);
      default: return sp_launch(highm_kernel<S, SH_OUT>, grid, lds, a, s, done);
    }
  }
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
