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
// Both parts are products with block-diagonal factors on the matrix cores,
// built from the angles once per weight set (bf16, MFMA operand order) by the
// builder kernels below.  Each workgroup owns up to SP_RB rows of ONE expert
// and a range of chunks (low) or 64 columns (high), so its factor fragments are
// loaded once and reused for all its rows; a width that has more angles than a
// row has elements would otherwise move more parameter bytes than activation
// bytes per row.  Rows are read and written as bf16, products accumulate in
// fp32.
#include "butterfly_impl.hpp"
#include "mfma_factors.hpp"

namespace bmoe {

constexpr int SP_RB = 64;  // rows per workgroup
constexpr int SP_VC = 64;  // high part: columns per workgroup

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

// ---------------------------------------------------------------- matrix-core low part
// Widths 1024 .. 8192 (S = 6 .. 9).  The low part of a chunk is G1 G0 with
//   G0 = stages 0 .. S-5: block-diagonal over runs of B0 = max(16, 2^(S-4))
//        consecutive indices (32 x 32 blocks at S = 9, 16 x 16 below; at
//        S < 8 a block only mixes its low S-4 bits),
//   G1 = stages S-4 .. S-1: block-diagonal over the 16 indices u + P0 j (j < 16)
//        of each u < P0 = 2^(S-4) (16 x 16 blocks),
// every block the product of its stages' rotations (the pair structure of each
// stage stays inside one block).  The blocks depend on the angles only, so they
// are built once per weight set, in bf16 and in the per-lane order of the MFMA
// operands; a workgroup then multiplies its 64-row tile (bf16, in LDS) by both
// factors: B x = G1 (G0 x), B^T x = G0^T (G1^T x).  A workgroup covers
// SC = max(1, 256 / 2^S) consecutive chunks, so each wave owns 4 blocks of G0
// and 4 (S = 9: 8) blocks of G1.

template <int S>
struct LowMCfg {
  static constexpr int P0 = 1 << (S - 4);        // G1 stride = number of G1 blocks per chunk
  static constexpr int B0 = P0 > 16 ? P0 : 16;   // G0 block width
  static constexpr int NB0 = (1 << S) / B0;      // G0 blocks per chunk
  static constexpr int SC = S >= 8 ? 1 : (256 >> S);   // chunks per workgroup
  static constexpr int W = SC << S;              // indices per workgroup row
  static constexpr int RS = W + 4;               // LDS row stride in bf16 (8-byte aligned rows)
  static constexpr int ROWS = SP_RB;
  static constexpr size_t g0_bytes = size_t(NB0) * B0 * B0 * 2;
  static constexpr size_t g1_bytes = size_t(P0) * 256 * 2;
  static constexpr size_t chunk_bytes = g0_bytes + g1_bytes;
  static constexpr size_t per_expert = 16 * chunk_bytes;
  static constexpr size_t lds_bytes = size_t(ROWS) * RS * 2;
  static constexpr int G0W = W / B0 / 4;         // G0 blocks per wave (4)
  static constexpr int UQW = W / 16 / 4 / 4;     // G1 groups of 4 blocks per wave (1, or 2 at S = 9)
  static_assert(G0W == 4 && UQW >= 1, "wave shape");
};

// G1 contraction slot 4g+i holds j = (g&1) A + (g>>1) B + (i&1) C + (i>>1) D, with
// A chosen so lane groups 0 and 1 read LDS words 32 banks apart where the
// stride allows it (any permutation of 0..15 is a valid slot order)
template <int S>
__host__ __device__ constexpr int g1_slot(int g, int i) {
  return S == 9   ? (g & 1) * 2 + (g >> 1) * 4 + (i & 1) + 8 * (i >> 1)
         : S == 8 ? (g & 1) * 4 + (g >> 1) * 2 + (i & 1) + 8 * (i >> 1)
                  : (g & 1) * 8 + (g >> 1) * 4 + (i & 1) + 2 * (i >> 1);
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

// Factor fragments one wave keeps: its 4 G0 blocks (two 16-row halves at
// S = 9) and its 4 UQW G1 blocks.
template <int S>
struct LowFrag {
  uint4 g0w[S == 9 ? 4 : 1][2];
  uint2 g0[4];
  uint2 g1[4 * LowMCfg<S>::UQW];
};

// G0 on the tile: wave w owns blocks 4w .. 4w+3 (of B0 consecutive indices) in
// all 64 rows.  Operand B of row r: the block's contraction values held by
// lane group g (B0 = 32: inputs 8g .. 8g+7; else 4g .. 4g+3); the products
// overwrite the same elements.
template <int S>
__device__ __forceinline__ void lowm_g0(uint16_t* tile, const LowFrag<S>& F, int wave, int g, int l16) {
  using C = LowMCfg<S>;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const int b = 4 * wave + bb;
#pragma unroll
    for (int rg = 0; rg < C::ROWS / 16; ++rg) {
      uint16_t* rp = tile + (16 * rg + l16) * C::RS + C::B0 * b;
      if constexpr (C::B0 == 32) {
        const uint2 x0 = lm_ld64(rp + 8 * g), x1 = lm_ld64(rp + 8 * g + 4);
        const uint4 bx = make_uint4(x0.x, x0.y, x1.x, x1.y);
        const f32x4_t d0 = lm_mfma32(F.g0w[bb][0], bx), d1 = lm_mfma32(F.g0w[bb][1], bx);
        lm_st64(rp + 4 * g, lm_pack4(d0));
        lm_st64(rp + 16 + 4 * g, lm_pack4(d1));
      } else {
        const f32x4_t d = lm_mfma16(F.g0[bb], lm_ld64(rp + 4 * g));
        lm_st64(rp + 4 * g, lm_pack4(d));
      }
    }
  }
}

// G1 on the tile: group k of 4 consecutive blocks (chunk 4k / P0, u0 = 4k % P0)
// belongs to wave k / UQW; lane group g reads, for each of its 4 slots, the 4
// u's of one j at once (8 bytes) and regroups them per u.
template <int S>
__device__ __forceinline__ void lowm_g1(uint16_t* tile, const LowFrag<S>& F, int wave, int g, int l16) {
  using C = LowMCfg<S>;
#pragma unroll
  for (int uq = 0; uq < C::UQW; ++uq) {
    const int k = C::UQW * wave + uq;
    const int base = ((4 * k) / C::P0 << S) + (4 * k) % C::P0;
#pragma unroll
    for (int rg = 0; rg < C::ROWS / 16; ++rg) {
      uint16_t* rp = tile + (16 * rg + l16) * C::RS + base;
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
// one expert, SC consecutive chunks).  Rows past the tile's last repeat it and
// are not stored.
template <int S, bool TRANS>
__global__ __launch_bounds__(BF_THREADS) void lowm_kernel(BflyArgs a) {
  using C = LowMCfg<S>;
  constexpr int L = S + 4, n = 1 << L;
  constexpr int NWG = 16 / C::SC;                   // workgroups per row
  constexpr int PPR = C::W / 8;                     // 16-byte pieces per row
  constexpr int PPT = C::ROWS * PPR / BF_THREADS;   // per thread
  constexpr int BATCH = PPT < 8 ? PPT : 8;
  extern __shared__ __attribute__((aligned(16))) uint16_t tile[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int t = blockIdx.x / NWG, c0 = (blockIdx.x % NWG) * C::SC;
  int e, r0, nr;
  sp_find_tile(a.offsets, a.n_experts, t, e, r0, nr);
  if (e < 0) return;

  // this wave's fragments; block b of the workgroup lies in chunk c0 + b / NB0
  const unsigned char* fe = a.fac + (size_t(e) * 16 + c0) * C::chunk_bytes;
  LowFrag<S> F;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const int b = 4 * wave + bb;
    const unsigned char* fc = fe + (b / C::NB0) * C::chunk_bytes + size_t(b % C::NB0) * C::B0 * C::B0 * 2;
    if constexpr (C::B0 == 32) {
#pragma unroll
      for (int h = 0; h < 2; ++h) F.g0w[bb][h] = *reinterpret_cast<const uint4*>(fc + (h * 64 + lane) * 16);
    } else {
      F.g0[bb] = *reinterpret_cast<const uint2*>(fc + lane * 8);
    }
  }
#pragma unroll
  for (int uq = 0; uq < C::UQW; ++uq) {
    const int k = C::UQW * wave + uq;
    const unsigned char* fc = fe + ((4 * k) / C::P0) * C::chunk_bytes + C::g0_bytes;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      F.g1[4 * uq + q] = *reinterpret_cast<const uint2*>(fc + (size_t((4 * k) % C::P0 + q) * 64 + lane) * 8);
  }

  const uint16_t* in = reinterpret_cast<const uint16_t*>(a.in) + size_t(r0) * n + (c0 << S);
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + size_t(r0) * n + (c0 << S);
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
  constexpr int P0 = C::P0, B0 = C::B0;
  __shared__ float2 cs[S * hc];
  const int tid = threadIdx.x;
  const int e = blockIdx.x / 16, c = blockIdx.x % 16;
  const float* ae = ang + size_t(e) * L * half + size_t(c) * hc;
  for (int idx = tid; idx < S * hc; idx += BF_THREADS) cs[idx] = sincos_rev(ae[(idx / hc) * half + idx % hc]);
  __syncthreads();
  unsigned char* fc = out + (size_t(e) * 16 + c) * C::chunk_bytes;
  constexpr int J0 = C::NB0 * B0, J1 = P0 * 16;
  for (int job = tid; job < J0 + J1; job += BF_THREADS) {
    if (job < J0) {
      const int b = job / B0, o = job % B0;
      float v[B0];
#pragma unroll
      for (int q = 0; q < B0; ++q) v[q] = q == o ? 1.0f : 0.0f;
      rotate_vec<B0, 0, S - 4, TRANS>(v, cs, hc, B0 * b, 1);
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        if constexpr (B0 == 32) {
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
  switch (log2n) {
    case 10: return LowMCfg<6>::per_expert;
    case 11: return LowMCfg<7>::per_expert;
    case 12: return LowMCfg<8>::per_expert;
    case 13: return LowMCfg<9>::per_expert;
    default: return 0;
  }
}

template <int S>
static hipError_t launch_lowfac_S(const float* ang, unsigned char* out, int n_experts, bool trans, hipStream_t s) {
  const dim3 grid(n_experts * 16), block(BF_THREADS);
  if (trans) hipLaunchKernelGGL((lowfac_kernel<S, true>), grid, block, 0, s, ang, out);
  else hipLaunchKernelGGL((lowfac_kernel<S, false>), grid, block, 0, s, ang, out);
  return hipGetLastError();
}

hipError_t launch_low_factor_prep(const float* ang, unsigned char* out, int n_experts, int log2n, bool trans,
                                  hipStream_t s) {
  if (n_experts <= 0) return hipSuccess;
  switch (log2n) {
    case 10: return launch_lowfac_S<6>(ang, out, n_experts, trans, s);
    case 11: return launch_lowfac_S<7>(ang, out, n_experts, trans, s);
    case 12: return launch_lowfac_S<8>(ang, out, n_experts, trans, s);
    case 13: return launch_lowfac_S<9>(ang, out, n_experts, trans, s);
    default: return hipErrorInvalidValue;
  }
}

enum SplitHigh { SH_IN = 0, SH_MID = 1, SH_OUT = 2 };

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

// Both parts need their prepared block factors (built with the layer's
// prepared data); a missing buffer is a caller error.
template <int S>
static hipError_t launch_low_S(const BflyArgs& a, bool trans, hipStream_t s) {
  static int done[2][64] = {{0}};
  if (!a.fac) return hipErrorInvalidValue;
  const int grid = sp_tiles(a) * (16 / LowMCfg<S>::SC);
  if (trans) return sp_launch(lowm_kernel<S, true>, grid, LowMCfg<S>::lds_bytes, a, s, done[1]);
  return sp_launch(lowm_kernel<S, false>, grid, LowMCfg<S>::lds_bytes, a, s, done[0]);
}

template <int S>
static hipError_t launch_high_S(const BflyArgs& a, int mode, hipStream_t s) {
  static int done[64] = {0};
  if (!a.fac || (mode == SH_MID && !a.fac1)) return hipErrorInvalidValue;
  const int grid = sp_tiles(a) * ((1 << S) / SP_VC);
  const size_t lds = HighMCfg<S>::lds_bytes;
  switch (mode) {
    case SH_IN: return sp_launch(highm_kernel<S, SH_IN>, grid, lds, a, s, done);
    case SH_MID: return sp_launch(highm_kernel<S, SH_MID>, grid, lds, a, s, done);
    default: return sp_launch(highm_kernel<S, SH_OUT>, grid, lds, a, s, done);
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
