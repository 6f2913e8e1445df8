// Shared ternary substrate product Z = alpha * U * W^T for wide layers, with the
// substrate prepared as paired 2-bit codes (ButterflyMoE, gist.science/zh/paper/2601.13563,
// technical summary §2.1-§2.2: one ternary substrate shared by every expert, so
// all routed rows form one dense contraction: M = rows, N = d_out, K = d_in).
//
// Workgroup tile: 128 rows x TN output columns, four waves; wave w owns output
// columns [w TN/4, (w+1) TN/4) for all 128 rows, so no two waves read the same
// substrate rows.  Its substrate fragments come straight from global memory
// (8 bytes = 32 weights per lane per 128-wide K step, two words of 16; four
// lanes fill 32 contiguous bytes of a row), each word becomes two words of
// fp4 nibbles by a mask (pair2_to_fp4) and exact bf16 +-1/0 with one
// v_cvt_scalef32_pk_bf16_fp4 per two weights.  The activation tile (128 rows x
// 128 K, bf16) goes through two LDS buffers and is read by all four waves.
// In a K step, lanes 16g .. 16g+15 supply contraction indices 32g .. 32g+31 of
// the step (8 per MFMA); the activation operand follows the same order.  The
// loads of step k+1 are issued before the products of step k, and within a
// step the LDS reads of each sub-step's operand fragments are interleaved with
// the first products of the sub-step before it (scheduling barriers and an
// explicit LDS wait at each sub-step boundary fix that order; left to itself
// the compiler issued each sub-step's reads just before their first use and
// waited for them there).
// TN = 256: 64 columns per wave, 128 accumulators per lane, two workgroups
// per CU (LDS 64 KiB each), so one workgroup's products cover the other's
// load waits.
//
// Tile order: groups of 4 row tiles sweep all column tiles, so a substrate
// slice is reused by 4 row tiles and an activation tile by every column tile
// while both sit in one XCD's L2 (contiguous logical tiles per XCD).
//
// The output tile leaves through LDS as whole 512-byte row runs.  With EPI
// (N = 4096 or 8192, rows bucketed by expert) it is first multiplied by
// stages 0..7 of each row's expert rotation: G0 on the accumulators, G1 on
// the staged tile; 256 columns are one chunk of them (ButterflyMoE zh,
// technical summary §2.2: the stages below bit 8 act within runs of 256
// consecutive indices).
#include "common.hpp"
#include "lowpart.hpp"

namespace bmoe {

constexpr int GF_THREADS = 256;
constexpr int GF_TM = 128;
constexpr int GF_KS = 128;          // K per step
constexpr int GF_GRP = 4;           // row tiles per group
constexpr int GF_TILE = GF_TM * GF_KS;  // bf16 elements of one activation tile

typedef __attribute__((address_space(3))) void gf_lds_t;
typedef __attribute__((address_space(1))) const void gf_glob_t;

__device__ __forceinline__ uint4 gf_fp4x8_to_bf16(uint32_t w) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
  return r;
}

// Activation tile in LDS: 128 rows of 128 bf16 (256 bytes, no padding); the
// 16-byte chunk ch of row r sits at position ch ^ gf_swz(r & 15) of the row,
// gf_swz swapping the two 2-bit halves of its argument.  With that map a
// wave's 16-byte operand read (lane l: row 16 j + l % 16, chunk 4 (l / 16) + s)
// has no LDS bank conflicts on gfx950 (measured: 0 conflict cycles per read;
// the plain map ch ^ (r & 15) took 4), as the linear read of a 1 KiB block
// does.  The tile is filled by direct global->LDS loads: one 16-byte load per
// lane, each wave-wide load filling 4 consecutive rows.
__device__ __forceinline__ int gf_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int TN, bool EPI>
__global__ __launch_bounds__(GF_THREADS, 2) void gemm_fp4_kernel(GemmFp4Args a) {
  constexpr int WN = TN / 4;                  // output columns per wave
  constexpr int OB = WN / 16;                 // 16-column blocks per wave
  constexpr int MB = GF_TM / 16;              // 16-row blocks
  constexpr int DPW = GF_TM / 4 / 4;          // direct loads per wave per tile (4 rows each)
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];  // [2][GF_TM][GF_KS]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int ntn = a.N / TN, ntm = (a.M + GF_TM - 1) / GF_TM;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = logical / (GF_GRP * ntn), r = logical % (GF_GRP * ntn);
  const int tn = r / GF_GRP, tm = grp * GF_GRP + r % GF_GRP;
  if (tm >= ntm) return;
  const int m0 = tm * GF_TM, n0 = tn * TN + wave * WN;
  const int K = a.K, nk = K / GF_KS;
  const uint16_t* U = reinterpret_cast<const uint16_t*>(a.a);
  // this lane's substrate rows n0 + 16 i + l16, bytes 8 g .. 8 g + 7 of each 32-byte step
  const unsigned char* wrow = a.w + size_t(n0 + l16) * (K / 4) + 8 * g;
  // this lane's source of direct load j: row 4 (DPW wave + j) + lane / 16 (clamped to
  // M - 1: rows past M are never stored), chunk (lane % 16) ^ gf_swz(row % 16)
  auto usrc = [&](int j) {
    const int row = 4 * (DPW * wave + j) + (lane >> 4);
    const int ch = (lane & 15) ^ gf_swz(row & 15);
    return U + size_t(min(m0 + row, a.M - 1)) * K + 8 * ch;
  };

  auto load_w = [&](int kt, uint2 (&w)[OB]) {
#pragma unroll
    for (int i = 0; i < OB; ++i)
      w[i] = *reinterpret_cast<const uint2*>(wrow + size_t(16 * i) * (K / 4) + 32 * kt);
  };
  auto load_u = [&](int kt, int buf) {
#pragma unroll
    for (int j = 0; j < DPW; ++j)
      __builtin_amdgcn_global_load_lds((gf_glob_t*)(usrc(j) + kt * GF_KS),
                                       (gf_lds_t*)(smem + buf * GF_TILE + (4 * (DPW * wave + j)) * GF_KS),
                                       16, 0, 0);
  };

  f32x4_t acc[OB][MB];
#pragma unroll
  for (int i = 0; i < OB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // operand reads: row 16 jb + l16, chunk 4 g + s at position (4 g + s) ^ gf_swz(l16)
  auto load_uf = [&](const uint16_t* ub, int s, bf16x8_t (&uf)[MB]) {
    const int p = (4 * g + s) ^ gf_swz(l16);
#pragma unroll
    for (int j = 0; j < MB; ++j)
      uf[j] = *reinterpret_cast<const bf16x8_t*>(ub + (16 * j + l16) * GF_KS + 8 * p);
  };
  // products of sub-step q (0 .. 3): weights 8 (q & 1) .. 8 (q & 1) + 7 of word
  // q >> 1 of each substrate fragment
  auto substep = [&](const bf16x8_t (&uf)[MB], const uint2 (&Wc)[OB], int q) {
#pragma unroll
    for (int i = 0; i < OB; ++i) {
      const bf16x8_t wf = __builtin_bit_cast(bf16x8_t, gf_fp4x8_to_bf16(pair2_to_fp4((q >> 1) ? Wc[i].y : Wc[i].x, q & 1)));
#pragma unroll
      for (int j = 0; j < MB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, uf[j], acc[i][j], 0, 0, 0);
    }
  };
  // step kt: start the loads of step kt + 1 (activation tile into the other LDS
  // buffer, substrate fragments into Wn), then four sub-steps, the operand
  // fragments of sub-step q + 1 read from LDS before the products of sub-step q
  // (scheduling barriers keep that order), then wait for the loads and for
  // every wave.
  auto step = [&](int kt, const uint2 (&Wc)[OB], uint2 (&Wn)[OB]) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      load_u(kt + 1, buf ^ 1);
      load_w(kt + 1, Wn);
    }
    const uint16_t* ub = smem + buf * GF_TILE;
    bf16x8_t ua[MB], ubf[MB];
    // each region: the LDS reads of sub-step q + 1 issued one per product at
    // the start of the products of sub-step q
    auto early_reads = [&]() {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, OB * MB - MB, 0);
    };
    load_uf(ub, 0, ua);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this sub-step's fragments are in
    load_uf(ub, 1, ubf);
    substep(ua, Wc, 0);
    early_reads();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    load_uf(ub, 2, ua);
    substep(ubf, Wc, 1);
    early_reads();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    load_uf(ub, 3, ubf);
    substep(ua, Wc, 2);
    early_reads();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    substep(ubf, Wc, 3);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // waits for this wave's loads, then for every wave
  };

  uint2 W0[OB], W1[OB];
  load_u(0, 0);
  load_w(0, W0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, W0, W1);
    if (kt + 1 < nk) step(kt + 1, W1, W0);
  }

  // Output tile through LDS (both activation buffers are free after the last
  // step's barrier): row r, 8-byte unit u (4 columns) at unit u ^ 2 (r mod 16)
  // of the row, so the 32 lanes of one write pass (16 rows, 2 units each) and
  // the 16 lanes of one 16-byte read (one row) hit distinct banks; each row's
  // TN columns then go out as whole 16-byte pieces, one row per 32 lanes.
  static_assert(TN == 256, "one 512-byte row of output per 32 lanes");
  // epilogue: bucket offsets of the experts (for each row's expert)
  __shared__ int s_off[EPI ? 257 : 1];
  __shared__ int s_exp[EPI ? GF_TM : 1];
  uint2* st = reinterpret_cast<uint2*>(smem);
  // the lane's 4 consecutive output columns of row 16 j + l16 in its column
  // block i, as bf16, and their place in the staged tile
  uint2 ob[OB][MB];
#pragma unroll
  for (int i = 0; i < OB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      ob[i][j].x = pack_bf16x2(a.alpha * acc[i][j][0], a.alpha * acc[i][j][1]);
      ob[i][j].y = pack_bf16x2(a.alpha * acc[i][j][2], a.alpha * acc[i][j][3]);
    }
  auto stage = [&](int i, int j, uint2 o) {
    const int r = 16 * j + l16, u = wave * (WN / 4) + 4 * i + g;
    st[r * (TN / 4) + (u ^ ((r & 15) << 1))] = o;
  };
  if constexpr (!EPI) {
#pragma unroll
    for (int i = 0; i < OB; ++i)
#pragma unroll
      for (int j = 0; j < MB; ++j) stage(i, j, ob[i][j]);
    __syncthreads();
  } else {
    // Stages 0..7 of each row's expert rotation on the tile: the tile's 256
    // columns are chunk tn of the width (4096 or 8192), so G0 (16 x 16 blocks of
    // consecutive columns) then G1 (16 x 16 blocks over u + 16 j) act inside
    // it, each product rounded to bf16 as the separate low-part pass does.
    // Wave w owns G0 blocks 4w .. 4w+3 and G1 blocks 4w .. 4w+3 for every
    // 16-row block; a row block spanning several experts is multiplied once
    // per expert and each row keeps its own expert's result.  G0 acts on the
    // accumulators before the tile is staged: a lane's 4 consecutive columns
    // of one row are the B operand of a 16 x 16 x 16 product over its block,
    // so only G1 makes a pass over the staged tile (the epilogue is bound by
    // those LDS passes); operands and roundings are those of a staged G0.
    using LC = LowMCfg<8>;
    static_assert(OB == 4, "a wave's four G0 blocks");
    for (int i = tid; i <= a.n_experts; i += GF_THREADS) s_off[i] = a.offsets[i];
    __syncthreads();
    if (tid < GF_TM) {
      // the expert of row m: s_off[e] <= m < s_off[e + 1] (s_off[n_experts] = M)
      const int m = min(m0 + tid, a.M - 1);
      int lo = 0, hi = a.n_experts;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= m) lo = mid; else hi = mid;
      }
      s_exp[tid] = lo;
    }
    __syncthreads();
    // 8-byte unit u (columns 4u .. 4u+3) of tile row r
    auto unit = [&](int r, int u) { return smem + r * TN + 4 * (u ^ ((r & 15) << 1)); };
    const unsigned char* lfc = a.lowfac + size_t(tn) * LC::chunk_bytes;
    const size_t lf_expert = size_t(a.N / TN) * LC::chunk_bytes;  // one expert's chunks
    uint2 f0[4], f1[4];
    int cur = -1;
    auto frags = [&](int e) {
      if (e == cur) return;
      const unsigned char* fc = lfc + size_t(e) * lf_expert;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) f0[bb] = *reinterpret_cast<const uint2*>(fc + (4 * wave + bb) * 512 + lane * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        f1[q] = *reinterpret_cast<const uint2*>(fc + LC::g0_bytes + (size_t(4 * wave + q) * 64 + lane) * 8);
      cur = e;
    };
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      uint2 y[OB];
#pragma unroll
      for (int i = 0; i < OB; ++i) y[i] = ob[i][j];
      const int er = s_exp[16 * j + l16];
      const int e1 = __builtin_amdgcn_readfirstlane(s_exp[16 * j + 15]);
      for (int e = __builtin_amdgcn_readfirstlane(s_exp[16 * j]); e <= e1; ++e) {
        frags(e);
#pragma unroll
        for (int i = 0; i < OB; ++i) {
          const f32x4_t d = lm_mfma16(f0[i], ob[i][j]);
          if (er == e) y[i] = lm_pack4(d);
        }
      }
#pragma unroll
      for (int i = 0; i < OB; ++i) stage(i, j, y[i]);
    }
    __syncthreads();
    for (int jb = 0; jb < MB; ++jb) {
      const int r = 16 * jb + l16, er = s_exp[r];
      const int e1 = __builtin_amdgcn_readfirstlane(s_exp[16 * jb + 15]);
      for (int e = __builtin_amdgcn_readfirstlane(s_exp[16 * jb]); e <= e1; ++e) {
        frags(e);
        uint2 x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = lm_ld64(unit(r, wave + 4 * g1_slot<8>(g, i)));
        f32x4_t d[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
          const uint2 bq = (q < 2) ? make_uint2(__builtin_amdgcn_perm(x[1].x, x[0].x, sel), __builtin_amdgcn_perm(x[3].x, x[2].x, sel))
                                   : make_uint2(__builtin_amdgcn_perm(x[1].y, x[0].y, sel), __builtin_amdgcn_perm(x[3].y, x[2].y, sel));
          d[q] = lm_mfma16(f1[q], bq);
        }
        if (er == e) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            lm_st64(unit(r, wave + 4 * g1_slot<8>(g, i)),
                    make_uint2(pack_bf16x2(d[0][i], d[1][i]), pack_bf16x2(d[2][i], d[3][i])));
        }
      }
    }
    __syncthreads();
  }
  uint16_t* Z = reinterpret_cast<uint16_t*>(a.z);
  constexpr int CPR = TN / 8;  // 16-byte pieces per output row
#pragma unroll
  for (int p = 0; p < GF_TM * CPR / GF_THREADS; ++p) {
    const int idx = p * GF_THREADS + tid, r = idx / CPR, c = idx % CPR;
    if (m0 + r < a.M)
      *reinterpret_cast<uint4*>(Z + size_t(m0 + r) * a.N + tn * TN + 8 * c) =
          *reinterpret_cast<const uint4*>(smem + r * TN + 8 * (c ^ (r & 15)));
  }
}

template <int TN, bool EPI>
static hipError_t launch_gemm_fp4_tn(const GemmFp4Args& a, hipStream_t s) {
  const int ntn = a.N / TN, ntm = (a.M + GF_TM - 1) / GF_TM;
  const int ngrp = (ntm + GF_GRP - 1) / GF_GRP;
  const size_t lds = size_t(2) * GF_TILE * sizeof(uint16_t);
  const hipError_t e = allow_dynamic_lds((const void*)gemm_fp4_kernel<TN, EPI>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_fp4_kernel<TN, EPI>), dim3(ngrp * GF_GRP * ntn), dim3(GF_THREADS), lds, s, a);
  return hipGetLastError();
}

bool gemm_fp4_supported(int N, int K) { return N % 256 == 0 && K % GF_KS == 0; }

// the epilogue's low part covers chunks of 256 = one column tile: stages 0..7
// of widths 4096 and 8192
bool gemm_fp4_low_epilogue_supported(int N) { return N == 4096 || N == 8192; }

hipError_t launch_gemm_fp4(const GemmFp4Args& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (!gemm_fp4_supported(a.N, a.K)) return hipErrorInvalidValue;
  if (a.lowfac) {
    if (!gemm_fp4_low_epilogue_supported(a.N) || !a.offsets || a.n_experts < 1 || a.n_experts > 256)
      return hipErrorInvalidValue;
    return launch_gemm_fp4_tn<256, true>(a, s);
  }
  return launch_gemm_fp4_tn<256, false>(a, s);
}

}  // namespace bmoe
