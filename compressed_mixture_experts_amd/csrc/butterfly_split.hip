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
// and a range of chunks (low) or 64 / 128 columns (high), so its factor fragments are
// loaded once and reused for all its rows; a width that has more angles than a
// row has elements would otherwise move more parameter bytes than activation
// bytes per row.  Rows are read and written as bf16, products accumulate in
// fp32.
#include "butterfly_impl.hpp"
#include "mfma_factors.hpp"
#include "lowpart.hpp"

namespace bmoe {


// Tiles of RB rows per expert in expert order.  The workgroup's tile index
// is pick(total) for `total` real tiles; it is turned into (expert e, first
// bucket row r0, rows nr), e = -1 for an index outside [0, total).
template <int RB, typename Pick>
__device__ __forceinline__ void sp_lookup(const int32_t* offsets, int n_experts, Pick pick, int& e, int& r0,
                                          int& nr) {
  __shared__ int s_info[3];
  __shared__ int s_tmp[16];  // one entry per wave (up to 1024 threads); only experts < 256 count
  const int tid = threadIdx.x;
  if (tid == 0) s_info[0] = -1;
  int nt = 0, cnt = 0, off = 0;
  if (tid < n_experts) {
    off = offsets[tid];
    cnt = offsets[tid + 1] - off;
    nt = (cnt + RB - 1) / RB;
  }
  int total;
  const int excl = block_excl_scan(nt, s_tmp, total);
  const int t = pick(total);
  if (tid < n_experts && t >= excl && t < excl + nt) {
    const int j = t - excl;
    s_info[0] = tid;
    s_info[1] = off + j * RB;
    s_info[2] = min(RB, cnt - j * RB);
  }
  __syncthreads();
  e = s_info[0];
  r0 = s_info[1];
  nr = s_info[2];
}

// Workgroup tile t, in grid order.
template <int RB = SP_RB>
__device__ __forceinline__ void sp_find_tile(const int32_t* offsets, int n_experts, int t, int& e, int& r0,
                                             int& nr) {
  sp_lookup<RB>(offsets, n_experts, [=](int) { return t; }, e, r0, nr);
}

// Each tile split into `units` workgroups (sub = 0 .. units-1).  Workgroup b
// runs on XCD b mod 8 (round-robin dispatch); the mapping gives every XCD one
// contiguous run of the real units, the runs balanced to within one, so
// consecutive tiles of one expert share an XCD's L2 and the expert's factors
// are fetched from beyond it about once rather than once per XCD.  The grid
// must hold at least as many workgroups as real units.
template <int RB = SP_RB>
__device__ __forceinline__ void sp_find_tile_xcd(const int32_t* offsets, int n_experts, int units, int& e, int& r0,
                                                 int& nr, int& sub) {
  int u = -1;
  sp_lookup<RB>(offsets, n_experts, [&](int total) {
    const int b = blockIdx.x, x = b & 7, slot = b >> 3;
    const int nu = total * units, per = nu >> 3, rem = nu & 7;
    u = slot < per + (x < rem) ? x * per + min(x, rem) + slot : -1;
    return u < 0 ? -1 : u / units;
  }, e, r0, nr);
  sub = u < 0 ? 0 : u % units;
}

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
// transposed rotations); of M^T it is M e_o.  Width 2^L holds 2^(L-S) chunks:
// 16 for the split passes (L = S + 4), 32 for the low part of width 8192 that
// the up product's epilogue applies (S = 8).
template <int S, bool TRANS, int L = S + 4>
__global__ __launch_bounds__(BF_THREADS) void lowfac_kernel(const float* __restrict__ ang, unsigned char* __restrict__ out) {
  using C = LowMCfg<S>;
  constexpr int half = 1 << (L - 1), hc = 1 << (S - 1), NCH = 1 << (L - S);
  constexpr int P0 = C::P0, B0 = C::B0;
  __shared__ float2 cs[S * hc];
  const int tid = threadIdx.x;
  const int e = blockIdx.x / NCH, c = blockIdx.x % NCH;
  const float* ae = ang + size_t(e) * L * half + size_t(c) * hc;
  for (int idx = tid; idx < S * hc; idx += BF_THREADS) cs[idx] = sincos_rev(ae[(idx / hc) * half + idx % hc]);
  __syncthreads();
  unsigned char* fc = out + (size_t(e) * NCH + c) * C::chunk_bytes;
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

size_t low_factor_bytes(int log2n, bool chunks256) {
  if (chunks256) return log2n == 13 ? 32 * LowMCfg<8>::chunk_bytes : log2n == 12 ? LowMCfg<8>::per_expert : 0;
  switch (log2n) {
    case 10: return LowMCfg<6>::per_expert;
    case 11: return LowMCfg<7>::per_expert;
    case 12: return LowMCfg<8>::per_expert;
    case 13: return LowMCfg<9>::per_expert;
    default: return 0;
  }
}

template <int S, int L = S + 4>
static hipError_t launch_lowfac_S(const float* ang, unsigned char* out, int n_experts, bool trans, hipStream_t s) {
  const dim3 grid(n_experts << (L - S)), block(BF_THREADS);
  if (trans) hipLaunchKernelGGL((lowfac_kernel<S, true, L>), grid, block, 0, s, ang, out);
  else hipLaunchKernelGGL((lowfac_kernel<S, false, L>), grid, block, 0, s, ang, out);
  return hipGetLastError();
}

hipError_t launch_low_factor_prep(const float* ang, unsigned char* out, int n_experts, int log2n, bool trans,
                                  bool chunks256, hipStream_t s) {
  if (n_experts <= 0) return hipSuccess;
  if (chunks256 && log2n == 13) return launch_lowfac_S<8, 13>(ang, out, n_experts, trans, s);
  if (chunks256 && log2n != 12) return hipErrorInvalidValue;
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
  // columns per workgroup (16 per wave): 128 at width 8192, whose 16 indices
  // of a column lie 1 KiB apart, so that a workgroup reads 256-byte runs
  // (566 -> 533 us for the FFN middle's pass over 65536 rows of 8192); 64
  // below (128 columns at width 4096 gave half the workgroups and took 90
  // instead of 76 us over 16384 rows)
  static constexpr int VC = S == 9 ? 128 : 64;
  static constexpr int NTH = 4 * VC;                      // threads
  static constexpr int RSB = 16 * VC * 2 + 8;             // LDS bytes per row: [16 j][VC v] bf16 + pad
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

// High part on the matrix cores.  WG = (tile of <= 64 rows of one expert, VC
// columns, VC / 16 waves); sub-tiles of 16 rows go through LDS as
// [row][16 j][VC v] bf16 (coalesced 16-byte loads and stores); wave w
// multiplies columns 16w .. 16w+15 in groups of 4, reading each j's 4 columns
// with one 8-byte LDS read.
template <int S, int MODE>
__global__ __launch_bounds__(HighMCfg<S>::NTH, 1024 / HighMCfg<S>::NTH) void highm_kernel(BflyArgs a) {
  using C = HighMCfg<S>;
  constexpr int L = S + 4, n = 1 << L;
  constexpr int VC = C::VC, NTH = C::NTH;
  constexpr int VPC = VC / 8, PR = 16 * VPC;  // 16-byte pieces per (row, j) and per row
  constexpr int ncb = C::NV / VC;
  constexpr int PPT = C::RT * PR / NTH;  // 16-byte pieces per thread (8)
  extern __shared__ __attribute__((aligned(16))) unsigned char hl[];
  __shared__ size_t s_row[SP_RB];
  __shared__ float s_g[SP_RB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  int e, r0, nr, cb;
  sp_find_tile_xcd(a.offsets, a.n_experts, ncb, e, r0, nr, cb);
  if (e < 0) return;

  const int vw = cb * VC + 16 * wave;  // this wave's first column
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
      const int p = k * NTH + tid, row = min(rs + p / PR, nr - 1), j = (p / VPC) % 16, vc = p % VPC;
      const size_t src = MODE == SH_OUT ? size_t(r0 + row) * n : s_row[row];
      v[k] = *reinterpret_cast<const uint4*>(in + src + (size_t(j) << S) + cb * VC + 8 * vc);
    }
  };
  for (int rs = 0; rs < nr; rs += C::RT) {
    const int m = min(C::RT, nr - rs);
    uint4 v[PPT];
    load(rs, v);
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = k * NTH + tid, row = p / PR, j = (p / VPC) % 16, vc = p % VPC;
      uint16_t* d = reinterpret_cast<uint16_t*>(hl + row * C::RSB) + j * VC + 8 * vc;
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
      for (int i = 0; i < 4; ++i) r[i] = lm_ld64(rp + (g + 4 * i) * VC + 4 * qd);
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
        lm_st64(rp + (g + 4 * i) * VC + 4 * qd,
                make_uint2(pack_bf16x2(d[0][i], d[1][i]), pack_bf16x2(d[2][i], d[3][i])));
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = k * NTH + tid, row = p / PR, j = (p / VPC) % 16, vc = p % VPC;
      if (row < m) {
        const uint16_t* sp = reinterpret_cast<const uint16_t*>(hl + row * C::RSB) + j * VC + 8 * vc;
        const uint2 x0 = lm_ld64(sp), x1 = lm_ld64(sp + 4);
        const size_t dst = MODE == SH_OUT ? s_row[rs + row] : size_t(r0 + rs + row) * n;
        *reinterpret_cast<uint4*>(out + dst + (size_t(j) << S) + cb * VC + 8 * vc) = make_uint4(x0.x, x0.y, x1.x, x1.y);
      }
    }
    __syncthreads();  // stored before the next sub-tile is written
  }
}

// ---------------------------------------------------------------- FFN middle at width 8192, pair stage
// After the up product's epilogue has applied stages 0..7 of B(phi_up) (its
// 256-column tiles are the chunks of those stages), B(phi_up) still needs
// stage 8 and stages 9..12.  Stage 8 rotates the pairs (v + 512 j, v + 256 +
// 512 j) for v < 256, j < 16 (pair index 256 j + v), i.e. column v of the
// S = 9 high part against column v + 256 at the same j; stages 9..12 are the
// S = 9 high part's H_v' (v' < 512).  A workgroup takes 64 column pairs
// (v0 + p, p < 64, and their partners) and keeps them interleaved in LDS, tile
// column 2p + b holding column v' = 256 b + v0 + p, so a pair's stage-8
// rotation acts on two neighbouring bf16 values of one lane (fp32 cos and sin
// from a per-workgroup table).  The rest is the S = 9 middle: H(phi_up),
// GELU, H(theta_dn)^T; the low part of B(theta_dn)^T follows as its own pass.
struct HighPCfg {
  static constexpr int PW = 64;                                 // column pairs per workgroup
  static constexpr int VC = 2 * PW;                             // tile columns
  static constexpr int NTH = 4 * VC;                            // 16 tile columns per wave
  static constexpr int RT = 16;                                 // rows per sub-tile
  // LDS layout of a tile row: the 16 j's at a stride of JS bf16 (264 bytes,
  // two banks apart modulo 64 banks), rows RSB bytes apart (4 banks apart), so
  // that the 32 lanes of one pass of an 8-byte access (8 column groups x 4 j's
  // in the load and store phases, 16 rows x 2 j's in the product phase) fall
  // on distinct banks; with 256-byte j-runs they all shared one bank pair
  static constexpr int JS = VC + 4;
  static constexpr int RSB = 16 * JS * 2 + 144;
  static_assert(JS * 2 % 256 == 8 && RSB % 256 == 16, "bank spread");
  static constexpr int CSP = PW + 2;                            // cos/sin table row stride (float2)
  static constexpr size_t cs_off = size_t(RT) * RSB;            // table after the sub-tile (16-aligned)
  static constexpr size_t lds_bytes = cs_off + size_t(16) * CSP * sizeof(float2);
  static_assert(cs_off % 16 == 0, "table alignment");
};

__global__ __launch_bounds__(HighPCfg::NTH, 2) void highp_kernel(BflyArgs a) {
  using C = HighPCfg;
  constexpr int S = 9, L = 13, n = 1 << L, half = n / 2;
  constexpr int VC = C::VC, NTH = C::NTH;
  constexpr int ncb = 256 / C::PW;                 // workgroups per row tile
  constexpr int PGN = C::PW / 8;                    // groups of 8 pairs per (row, j)
  constexpr int JPR = 16 * PGN;                     // load jobs per row: (j, 8 pairs)
  constexpr int JPT = C::RT * JPR / NTH;           // per thread
  static_assert(C::RT * JPR % NTH == 0, "jobs per thread");
  extern __shared__ __attribute__((aligned(16))) unsigned char hl[];
  float2* cs = reinterpret_cast<float2*>(hl + C::cs_off);  // [16 j][CSP] stage-8 (cos, sin)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  int e, r0, nr, cb;
  sp_find_tile_xcd(a.offsets, a.n_experts, ncb, e, r0, nr, cb);
  if (e < 0) return;
  const int v0 = cb * C::PW;

  // factor fragments of tile column 16 w + c: v' = 256 (c & 1) + v0 + 8 w + (c >> 1)
  uint2 fa0[16], fa1[16];
  const unsigned char* f0 = a.fac + size_t(e) * HighMCfg<S>::per_expert;
  const unsigned char* f1 = a.fac1 + size_t(e) * HighMCfg<S>::per_expert;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const size_t vc = size_t(256 * (c & 1) + v0 + 8 * wave + (c >> 1));
    fa0[c] = *reinterpret_cast<const uint2*>(f0 + (vc * 64 + lane) * 8);
    fa1[c] = *reinterpret_cast<const uint2*>(f1 + (vc * 64 + lane) * 8);
  }
  {
    const float* a8 = a.ang0 + size_t(e) * L * half + size_t(8) * half;
    for (int idx = tid; idx < 16 * C::PW; idx += NTH) {
      const int j = idx / C::PW, p = idx % C::PW;
      cs[j * C::CSP + p] = sincos_rev(a8[256 * j + v0 + p]);
    }
  }
  const uint16_t* in = reinterpret_cast<const uint16_t*>(a.in);
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  for (int rs = 0; rs < nr; rs += C::RT) {
    const int m = min(C::RT, nr - rs);
    // job = (row, j, pairs 8 pg .. 8 pg + 7): the two 16-byte pieces of
    // columns v0 + 8 pg .. and their partners; rows past the tile's last repeat it
    uint4 v[2 * JPT];
#pragma unroll
    for (int k = 0; k < JPT; ++k) {
      const int q = k * NTH + tid, row = min(rs + q / JPR, nr - 1), j = (q / PGN) % 16, pg = q % PGN;
      const uint16_t* src = in + size_t(r0 + row) * n + (size_t(j) << S) + v0 + 8 * pg;
      v[2 * k] = *reinterpret_cast<const uint4*>(src);
      v[2 * k + 1] = *reinterpret_cast<const uint4*>(src + 256);
    }
    if (rs > 0) __syncthreads();  // the previous sub-tile has left LDS
#pragma unroll
    for (int k = 0; k < JPT; ++k) {
      const int q = k * NTH + tid, row = q / JPR, j = (q / PGN) % 16, pg = q % PGN;
      const uint4 x0 = v[2 * k], x1 = v[2 * k + 1];
      uint16_t* d = reinterpret_cast<uint16_t*>(hl + row * C::RSB) + j * C::JS + 16 * pg;
      lm_st64(d, make_uint2(__builtin_amdgcn_perm(x1.x, x0.x, 0x05040100u), __builtin_amdgcn_perm(x1.x, x0.x, 0x07060302u)));
      lm_st64(d + 4, make_uint2(__builtin_amdgcn_perm(x1.y, x0.y, 0x05040100u), __builtin_amdgcn_perm(x1.y, x0.y, 0x07060302u)));
      lm_st64(d + 8, make_uint2(__builtin_amdgcn_perm(x1.z, x0.z, 0x05040100u), __builtin_amdgcn_perm(x1.z, x0.z, 0x07060302u)));
      lm_st64(d + 12, make_uint2(__builtin_amdgcn_perm(x1.w, x0.w, 0x05040100u), __builtin_amdgcn_perm(x1.w, x0.w, 0x07060302u)));
    }
    __syncthreads();
    uint16_t* rp = reinterpret_cast<uint16_t*>(hl + l16 * C::RSB) + 16 * wave;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      // tile columns 16 w + 4 qd .. + 3: pairs 8 w + 2 qd and 8 w + 2 qd + 1, (b = 0, 1) each
      uint2 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = lm_ld64(rp + (g + 4 * i) * C::JS + 4 * qd);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // stage 8: (lo, hi) -> (c lo - s hi, s lo + c hi)
        const float4 t = *reinterpret_cast<const float4*>(cs + (g + 4 * i) * C::CSP + 8 * wave + 2 * qd);
        const float a0 = __uint_as_float(r[i].x << 16), b0 = __uint_as_float(r[i].x & 0xffff0000u);
        const float a1 = __uint_as_float(r[i].y << 16), b1 = __uint_as_float(r[i].y & 0xffff0000u);
        r[i] = make_uint2(pack_bf16x2(t.x * a0 - t.y * b0, t.y * a0 + t.x * b0),
                          pack_bf16x2(t.z * a1 - t.w * b1, t.w * a1 + t.z * b1));
      }
      f32x4_t d[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
        const uint2 bq = (q < 2) ? make_uint2(__builtin_amdgcn_perm(r[1].x, r[0].x, sel), __builtin_amdgcn_perm(r[3].x, r[2].x, sel))
                                 : make_uint2(__builtin_amdgcn_perm(r[1].y, r[0].y, sel), __builtin_amdgcn_perm(r[3].y, r[2].y, sel));
        d[q] = lm_mfma16(fa0[4 * qd + q], bq);
        if (a.gelu) {
#pragma unroll
          for (int i = 0; i < 4; ++i) d[q][i] = gelu_erf(d[q][i]);
        }
        d[q] = lm_mfma16(fa1[4 * qd + q], lm_pack4(d[q]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lm_st64(rp + (g + 4 * i) * C::JS + 4 * qd,
                make_uint2(pack_bf16x2(d[0][i], d[1][i]), pack_bf16x2(d[2][i], d[3][i])));
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < JPT; ++k) {
      const int q = k * NTH + tid, row = q / JPR, j = (q / PGN) % 16, pg = q % PGN;
      if (row < m) {
        const uint16_t* sp = reinterpret_cast<const uint16_t*>(hl + row * C::RSB) + j * C::JS + 16 * pg;
        const uint2 w0 = lm_ld64(sp), w1 = lm_ld64(sp + 4), w2 = lm_ld64(sp + 8), w3 = lm_ld64(sp + 12);
        uint16_t* dst = out + size_t(r0 + rs + row) * n + (size_t(j) << S) + v0 + 8 * pg;
        *reinterpret_cast<uint4*>(dst) =
            make_uint4(__builtin_amdgcn_perm(w0.y, w0.x, 0x05040100u), __builtin_amdgcn_perm(w1.y, w1.x, 0x05040100u),
                       __builtin_amdgcn_perm(w2.y, w2.x, 0x05040100u), __builtin_amdgcn_perm(w3.y, w3.x, 0x05040100u));
        *reinterpret_cast<uint4*>(dst + 256) =
            make_uint4(__builtin_amdgcn_perm(w0.y, w0.x, 0x07060302u), __builtin_amdgcn_perm(w1.y, w1.x, 0x07060302u),
                       __builtin_amdgcn_perm(w2.y, w2.x, 0x07060302u), __builtin_amdgcn_perm(w3.y, w3.x, 0x07060302u));
      }
    }
  }
}

// ---------------------------------------------------------------- whole butterfly, one pass
// Widths 1024 and 2048 (S = 6, 7): a row is 2 or 4 KiB, so a workgroup holds
// FM_RB = 16 whole rows of one expert in LDS (row-major, row stride n + 8)
// and applies both parts there, with the same prepared block factors as the
// split passes: input rotation B^T = low^T high^T (gather the token rows,
// high^T, then G1^T, G0^T), output rotation B = high low (G0, G1, then high,
// times the gate, scattered to the slot rows).  One read and one write of
// the rows instead of two of each.  In the row-major tile the high part's
// column v, index j is element j 2^S + v, and the low part's chunks are
// consecutive, so both parts use the split kernels' MFMA steps with those
// strides.  Each wave keeps one pass's factor fragments in registers and
// loads the next pass's before the barrier between them; with many rows a
// workgroup instead takes a tall tile of 64 rows of one expert, keeps all
// three passes' fragments and runs the rows as four 16-row sub-tiles.
constexpr int FM_RB = 16;      // rows per workgroup (per sub-tile of a tall tile)
constexpr int FM_TALL = 64;    // rows per tall tile
constexpr int FM_TALL_ROWS = 32768;  // tall tiles from this many rows: two 64-row workgroups per CU
constexpr int FM_THREADS = 256;

template <int S>
struct FullCfg {
  static constexpr int NV = 1 << S;          // high part: columns; low part: chunk width
  static constexpr int n = 16 * NV;
  static constexpr int RS = n + 8;           // LDS row stride (bf16)
  static constexpr int NB0 = NV / 16;        // G0 blocks (16 x 16) per chunk
  static constexpr int P0 = NV / 16;         // G1 blocks per chunk
  static constexpr int HC = NV / 4;          // high-part columns per wave
  static constexpr int G0W = 16 * NB0 / 4;   // G0 blocks per wave
  static constexpr int G1W = 16 * P0 / 16;   // G1 groups of 4 blocks per wave
  static constexpr int PPT = FM_RB * n / 8 / FM_THREADS;  // 16-byte pieces per thread
  static constexpr size_t lds_bytes = size_t(FM_RB) * RS * 2;
  static_assert(S == 6 || S == 7, "widths 1024 and 2048");
  static_assert(LowMCfg<S>::B0 == 16 && LowMCfg<S>::P0 == P0, "low factor layout");
};

enum FullMode { FM_IN = 0, FM_OUT = 1 };

template <int S, int MODE, int TR>
__global__ __launch_bounds__(FM_THREADS, 2) void fullm_kernel(BflyArgs a) {
  using C = FullCfg<S>;
  using LC = LowMCfg<S>;
  using HC = HighMCfg<S>;
  constexpr int n = C::n, NV = C::NV, RS = C::RS;
  extern __shared__ __attribute__((aligned(16))) uint16_t tile[];  // [FM_RB][RS]
  static_assert(TR % FM_RB == 0, "tile of whole sub-tiles");
  __shared__ size_t s_row[TR];
  __shared__ float s_g[TR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  int e, r0, nr, sub;
  sp_find_tile_xcd<TR>(a.offsets, a.n_experts, 1, e, r0, nr, sub);
  if (e < 0) return;
  const unsigned char* lowf = a.fac + size_t(e) * LC::per_expert;
  const unsigned char* highf = a.fac1 + size_t(e) * HC::per_expert;
  if (tid < TR) {
    const int q = r0 + min(tid, nr - 1);
    if constexpr (MODE == FM_IN) {
      s_row[tid] = size_t(a.perm[q] / a.top_k) * n;  // token row of x
    } else {
      const int slot = a.perm[q];
      s_row[tid] = size_t(slot) * n;                 // per-slot output row
      s_g[tid] = a.gate[slot];
    }
  }

  // factor fragments of one pass; a wave's blocks are w + 4 t
  uint2 fh[C::HC];          // high part: columns 16 (w + 4 gi) + c
  uint2 f0[C::G0W];         // G0: blocks w + 4 t (16 consecutive indices each)
  uint2 f1[4 * C::G1W];     // G1: groups k = w + 4 t of 4 blocks (u0 .. u0 + 3 of one chunk)
  auto load_high = [&]() {
#pragma unroll
    for (int gi = 0; gi < C::HC / 16; ++gi)
#pragma unroll
      for (int c = 0; c < 16; ++c)
        fh[16 * gi + c] = *reinterpret_cast<const uint2*>(highf + (size_t(16 * (wave + 4 * gi) + c) * 64 + lane) * 8);
  };
  auto load_g0 = [&]() {
#pragma unroll
    for (int t = 0; t < C::G0W; ++t) {
      const int b = wave + 4 * t;
      f0[t] = *reinterpret_cast<const uint2*>(lowf + size_t(b / C::NB0) * LC::chunk_bytes +
                                              size_t(b % C::NB0) * 512 + lane * 8);
    }
  };
  auto load_g1 = [&]() {
#pragma unroll
    for (int t = 0; t < C::G1W; ++t) {
      const int k = wave + 4 * t, ch = (4 * k) / C::P0, u0 = (4 * k) % C::P0;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        f1[4 * t + q] = *reinterpret_cast<const uint2*>(lowf + size_t(ch) * LC::chunk_bytes + LC::g0_bytes +
                                                        (size_t(u0 + q) * 64 + lane) * 8);
    }
  };
  uint16_t* rowp = tile + l16 * RS;  // this lane's row in the MFMA steps
  auto high_pass = [&](int rs, int m) {  // sub-tile rows rs .. rs + m - 1
    const float gr = MODE == FM_OUT ? s_g[rs + min(l16, m - 1)] : 1.0f;
#pragma unroll
    for (int gi = 0; gi < C::HC / 16; ++gi) {
      uint16_t* rp = rowp + 16 * (wave + 4 * gi);
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        uint2 r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = lm_ld64(rp + (g + 4 * i) * NV + 4 * qd);
        f32x4_t d[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
          const uint2 bq = (q < 2) ? make_uint2(__builtin_amdgcn_perm(r[1].x, r[0].x, sel), __builtin_amdgcn_perm(r[3].x, r[2].x, sel))
                                   : make_uint2(__builtin_amdgcn_perm(r[1].y, r[0].y, sel), __builtin_amdgcn_perm(r[3].y, r[2].y, sel));
          d[q] = lm_mfma16(fh[16 * gi + 4 * qd + q], bq);
          if constexpr (MODE == FM_OUT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) d[q][i] *= gr;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          lm_st64(rp + (g + 4 * i) * NV + 4 * qd,
                  make_uint2(pack_bf16x2(d[0][i], d[1][i]), pack_bf16x2(d[2][i], d[3][i])));
      }
    }
  };
  auto g0_pass = [&]() {
#pragma unroll
    for (int t = 0; t < C::G0W; ++t) {
      uint16_t* rp = rowp + 16 * (wave + 4 * t) + 4 * g;
      lm_st64(rp, lm_pack4(lm_mfma16(f0[t], lm_ld64(rp))));
    }
  };
  auto g1_pass = [&]() {
#pragma unroll
    for (int t = 0; t < C::G1W; ++t) {
      const int k = wave + 4 * t;
      uint16_t* rp = rowp + ((4 * k) / C::P0) * NV + (4 * k) % C::P0;
      uint2 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = lm_ld64(rp + C::P0 * g1_slot<S>(g, i));
      f32x4_t d[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
        const uint2 bq = (q < 2) ? make_uint2(__builtin_amdgcn_perm(r[1].x, r[0].x, sel), __builtin_amdgcn_perm(r[3].x, r[2].x, sel))
                                 : make_uint2(__builtin_amdgcn_perm(r[1].y, r[0].y, sel), __builtin_amdgcn_perm(r[3].y, r[2].y, sel));
        d[q] = lm_mfma16(f1[4 * t + q], bq);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lm_st64(rp + C::P0 * g1_slot<S>(g, i), make_uint2(pack_bf16x2(d[0][i], d[1][i]), pack_bf16x2(d[2][i], d[3][i])));
    }
  };

  if constexpr (TR == FM_RB) {
    // first pass's fragments, then the rows (rows past the tile's last repeat it)
    if constexpr (MODE == FM_IN) load_high(); else load_g0();
    __syncthreads();  // row table
    const uint16_t* in = reinterpret_cast<const uint16_t*>(a.in);
    {
      constexpr int CPR = n / 8;  // 16-byte pieces per row
  #pragma unroll
      for (int k0 = 0; k0 < C::PPT; k0 += 8) {
        uint4 v[8];
  #pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int p = (k0 + k) * FM_THREADS + tid, row = min(p / CPR, nr - 1), c = p % CPR;
          const size_t src = MODE == FM_IN ? s_row[row] : size_t(r0 + row) * n;
          v[k] = *reinterpret_cast<const uint4*>(in + src + 8 * c);
        }
  #pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int p = (k0 + k) * FM_THREADS + tid, row = p / CPR, c = p % CPR;
          uint16_t* d = tile + row * RS + 8 * c;
          lm_st64(d, make_uint2(v[k].x, v[k].y));
          lm_st64(d + 4, make_uint2(v[k].z, v[k].w));
        }
      }
    }
    if constexpr (MODE == FM_IN) load_g1(); else load_g1();
    __syncthreads();
    if constexpr (MODE == FM_IN) {
      high_pass(0, nr);   // high^T (transposed blocks)
      load_g0();
      __syncthreads();
      g1_pass();     // G1^T
      __syncthreads();
      g0_pass();     // G0^T
    } else {
      g0_pass();
      load_high();
      __syncthreads();
      g1_pass();
      __syncthreads();
      high_pass(0, nr);   // high, times the gate
    }
    __syncthreads();
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
    {
      constexpr int CPR = n / 8;
  #pragma unroll
      for (int k = 0; k < C::PPT; ++k) {
        const int p = k * FM_THREADS + tid, row = p / CPR, c = p % CPR;
        if (row < nr) {
          const uint16_t* sp = tile + row * RS + 8 * c;
          const uint2 x0 = lm_ld64(sp), x1 = lm_ld64(sp + 4);
          const size_t dst = MODE == FM_IN ? size_t(r0 + row) * n : s_row[row];
          *reinterpret_cast<uint4*>(out + dst + 8 * c) = make_uint4(x0.x, x0.y, x1.x, x1.y);
        }
      }
    }
  } else {
    // tall tiles (many rows): every pass's fragments stay in registers (192
    // per lane at width 2048) while the workgroup runs its TR rows as
    // sub-tiles of FM_RB, so each expert's factors cross from L2 once per TR
    // rows instead of once per FM_RB
    load_high();
    load_g0();
    load_g1();
    __syncthreads();  // row table
    const uint16_t* in = reinterpret_cast<const uint16_t*>(a.in);
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
    constexpr int CPR = n / 8;  // 16-byte pieces per row
    for (int rs = 0; rs < nr; rs += FM_RB) {
      const int m = min(FM_RB, nr - rs);
      // the sub-tile's rows (rows past the tile's last repeat it)
#pragma unroll
      for (int k0 = 0; k0 < C::PPT; k0 += 8) {
        uint4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int p = (k0 + k) * FM_THREADS + tid, row = min(rs + p / CPR, nr - 1), c = p % CPR;
          const size_t src = MODE == FM_IN ? s_row[row] : size_t(r0 + row) * n;
          v[k] = *reinterpret_cast<const uint4*>(in + src + 8 * c);
        }
        if (k0 == 0 && rs > 0) __syncthreads();  // the previous sub-tile has left LDS
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int p = (k0 + k) * FM_THREADS + tid, row = p / CPR, c = p % CPR;
          uint16_t* d = tile + row * RS + 8 * c;
          lm_st64(d, make_uint2(v[k].x, v[k].y));
          lm_st64(d + 4, make_uint2(v[k].z, v[k].w));
        }
      }
      __syncthreads();
      if constexpr (MODE == FM_IN) {
        high_pass(rs, m);  // high^T (transposed blocks)
        __syncthreads();
        g1_pass();         // G1^T
        __syncthreads();
        g0_pass();         // G0^T
      } else {
        g0_pass();
        __syncthreads();
        g1_pass();
        __syncthreads();
        high_pass(rs, m);  // high, times the gate
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < C::PPT; ++k) {
        const int p = k * FM_THREADS + tid, row = p / CPR, c = p % CPR;
        if (row < m) {
          const uint16_t* sp = tile + row * RS + 8 * c;
          const uint2 x0 = lm_ld64(sp), x1 = lm_ld64(sp + 4);
          const size_t dst = MODE == FM_IN ? size_t(r0 + rs + row) * n : s_row[rs + row];
          *reinterpret_cast<uint4*>(out + dst + 8 * c) = make_uint4(x0.x, x0.y, x1.x, x1.y);
        }
      }
    }
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
static hipError_t sp_launch(K k, int grid, size_t lds, const BflyArgs& a, hipStream_t s, int threads = BF_THREADS) {
  if (grid <= 0) return hipSuccess;
  const hipError_t err = allow_dynamic_lds((const void*)k, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k, dim3(grid), dim3(threads), lds, s, a);
  return hipGetLastError();
}

static int sp_tiles(const BflyArgs& a) { return (a.rows + SP_RB - 1) / SP_RB + a.n_experts; }

// Both parts need their prepared block factors (built with the layer's
// prepared data); a missing buffer is a caller error.
template <int S>
static hipError_t launch_low_S(const BflyArgs& a, bool trans, hipStream_t s) {
  if (!a.fac) return hipErrorInvalidValue;
  const int grid = sp_tiles(a) * (16 / LowMCfg<S>::SC);
  if (trans) return sp_launch(lowm_kernel<S, true>, grid, LowMCfg<S>::lds_bytes, a, s);
  return sp_launch(lowm_kernel<S, false>, grid, LowMCfg<S>::lds_bytes, a, s);
}

template <int S>
static hipError_t launch_high_S(const BflyArgs& a, int mode, hipStream_t s) {
  if (!a.fac || (mode == SH_MID && !a.fac1)) return hipErrorInvalidValue;
  using C = HighMCfg<S>;
  const int grid = sp_tiles(a) * (C::NV / C::VC);
  const size_t lds = C::lds_bytes;
  switch (mode) {
    case SH_IN: return sp_launch(highm_kernel<S, SH_IN>, grid, lds, a, s, C::NTH);
    case SH_MID: return sp_launch(highm_kernel<S, SH_MID>, grid, lds, a, s, C::NTH);
    default: return sp_launch(highm_kernel<S, SH_OUT>, grid, lds, a, s, C::NTH);
  }
}

template <int S, int TR>
static hipError_t launch_full_ST(const BflyArgs& a, bool out_mode, hipStream_t s) {
  const int grid = (a.rows + TR - 1) / TR + a.n_experts;
  const size_t lds = FullCfg<S>::lds_bytes;
  if (out_mode) return sp_launch(fullm_kernel<S, FM_OUT, TR>, grid, lds, a, s, FM_THREADS);
  return sp_launch(fullm_kernel<S, FM_IN, TR>, grid, lds, a, s, FM_THREADS);
}

// Fewer rows keep 16-row workgroups, which overlap each pass's factor loads
// with the previous pass (64-row tiles at 16384 rows of width 1024 leave too
// few workgroups: 21.6 -> 28-31 us); many rows take tall tiles (65536 rows of
// width 2048: 152-155 -> 141-143 us)
template <int S>
static hipError_t launch_full_S(const BflyArgs& a, bool out_mode, hipStream_t s) {
  if (!a.fac || !a.fac1) return hipErrorInvalidValue;
  if (a.rows >= FM_TALL_ROWS) return launch_full_ST<S, FM_TALL>(a, out_mode, s);
  return launch_full_ST<S, FM_RB>(a, out_mode, s);
}

bool bfly_full_supported(int log2n) { return log2n == 10 || log2n == 11; }

hipError_t launch_bfly_full(const BflyArgs& a, bool out_mode, int log2n, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  switch (log2n) {
    case 10: return launch_full_S<6>(a, out_mode, s);
    case 11: return launch_full_S<7>(a, out_mode, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bfly_mid_pair(const BflyArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (!a.fac || !a.fac1 || !a.ang0) return hipErrorInvalidValue;
  return sp_launch(highp_kernel, sp_tiles(a) * (256 / HighPCfg::PW), HighPCfg::lds_bytes, a, s, HighPCfg::NTH);
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
