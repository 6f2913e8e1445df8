// Fused square-expert step: input rotation, shared-substrate product and output
// rotation of one tile of bucketed rows in a single workgroup (ButterflyMoE,
// gist.science/zh/paper/2601.13563, technical summary §2.1: inference rotates
// the input, multiplies by the ternary substrate and rotates the output; the
// expert matrix is never formed).  Rows U = B(theta_e)^T x and Z = U W^T stay
// in LDS; only x is read and the gated per-slot rows are written.
//
// Substrate operand: the caller provides W as one byte per weight holding the
// high byte of a bf16 (0x3F, 0xBF or 0x00, i.e. +-0.5 or 0); each 32-bit word of
// four weights becomes two bf16 pairs with two v_perm_b32 (low bytes zero),
// and the product is scaled by 2 alpha at the end (exact).
//
// LDS stays under 80 KiB at width <= 512 so that two workgroups share a CU and
// one's memory waits overlap the other's arithmetic.
#include "butterfly_impl.hpp"

namespace bmoe {

constexpr int FZ_RT = 32;  // rows per tile

// LDS: the fp32 tile, then one (cos, sin) table (the whole butterfly's up to
// width 256, one pass of three stages at width 512 so that two workgroups fit
// on a CU).  The bf16 operand U is written over the start of the tile.
template <int L>
struct FusedCfg {
  using C = BflyCfg<L>;
  static constexpr int n = C::n;
  static constexpr int TMODE = L <= 8 ? TAB_FULL : TAB_PASS;
  static constexpr int ust = n + 8;                                   // bf16 row stride of U
  static constexpr size_t tile_bytes = size_t(FZ_RT) * C::stride * 4;
  static constexpr size_t u_bytes = size_t(FZ_RT) * ust * 2;
  static constexpr size_t tab_bytes = size_t(TMODE == TAB_FULL ? L : 3) * C::half * 8;
  static constexpr size_t lds_bytes = tile_bytes + tab_bytes;
  static_assert(u_bytes <= tile_bytes, "U must fit over the tile");
};

// four substrate bytes (weights k..k+3) -> two bf16 pairs (low bytes zero)
__device__ __forceinline__ void wbytes_to_bf16(uint32_t w, uint32_t& p0, uint32_t& p1) {
  p0 = __builtin_amdgcn_perm(0u, w, 0x010C000Cu);
  p1 = __builtin_amdgcn_perm(0u, w, 0x030C020Cu);
}

// Substrate product Z = U W^T of the tile on MFMA (16x16x32 bf16).  Wave w owns
// output columns [w n/4, (w+1) n/4) (OB blocks of 16) for all 32 rows (RB = 2
// blocks of 16).  The contraction index is visited in double steps of 64: in
// double step u, lanes 16g .. 16g+15 hold the 16 weights k = 64u + 16g .. +15 of
// their output row (one 16-byte load; the four lane groups read 64 contiguous
// bytes of each row) and use the first 8 in the first MFMA of the step and the
// last 8 in the second; the U operand follows the same order.  The loads of
// the first PF double steps are issued by the caller before the input
// rotation so that they arrive while it runs.
template <int L>
struct WFrag {
  static constexpr int OB = (1 << L) / 64;
  static constexpr int DS = (1 << L) / 64;  // double steps
  static constexpr int PF = DS < 2 ? DS : 2;
  uint4 w[PF][OB];
};

template <int L>
__device__ __forceinline__ void load_wfrag(uint4 (&w)[WFrag<L>::OB], const unsigned char* wrow, int u) {
  constexpr int n = 1 << L;
#pragma unroll
  for (int i = 0; i < WFrag<L>::OB; ++i)
    w[i] = *reinterpret_cast<const uint4*>(wrow + size_t(16 * i) * n + 64 * u);
}

template <int L>
__global__ __launch_bounds__(BF_THREADS, 2) void fused_square_kernel(FusedArgs a) {
  using C = BflyCfg<L>;
  using F = FusedCfg<L>;
  using WF = WFrag<L>;
  constexpr int n = C::n;
  constexpr int angs = L * C::half;
  constexpr int TM = F::TMODE;
  constexpr int OB = WF::OB, DS = WF::DS, PF = WF::PF;
  constexpr int RB = FZ_RT / 16;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int s_info[3];
  __shared__ int s_tmp[4];
  __shared__ size_t s_src[FZ_RT], s_dst[FZ_RT];
  __shared__ float s_gate[FZ_RT];
  float* tile = smem;
  float2* tab = reinterpret_cast<float2*>(reinterpret_cast<unsigned char*>(smem) + F::tile_bytes);
  uint16_t* ub = reinterpret_cast<uint16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;

  // ---- tile of one expert
  if (tid == 0) s_info[0] = -1;
  {
    int nt = 0, cnt = 0, off = 0;
    if (tid < a.n_experts) {
      off = a.offsets[tid];
      cnt = a.offsets[tid + 1] - off;
      nt = (cnt + FZ_RT - 1) / FZ_RT;
    }
    int total;
    const int excl = block_excl_scan(nt, s_tmp, total);
    // tiles of one expert are consecutive: keep them on one XCD
    const int tl = t < total ? xcd_remap(t, total) : -1;
    if (tid < a.n_experts && tl >= excl && tl < excl + nt) {
      const int j = tl - excl;
      s_info[0] = tid;
      s_info[1] = off + j * FZ_RT;
      s_info[2] = min(FZ_RT, cnt - j * FZ_RT);
    }
  }
  __syncthreads();
  const int e = s_info[0];
  if (e < 0) return;
  const int r0 = s_info[1], nr = s_info[2];

  // angles of both rotations (registers in one-pass-table mode)
  AngleRegs<L, TM> Rth, Rph;
  if constexpr (TM == TAB_PASS) {
    load_angle_regs<L>(Rth, a.theta + size_t(e) * angs);
    load_angle_regs<L>(Rph, a.phi + size_t(e) * angs);
  }
  if (tid < nr) {
    const int slot = a.perm[r0 + tid];
    s_src[tid] = size_t(slot / a.top_k) * n;
    s_dst[tid] = size_t(slot) * n;
    s_gate[tid] = a.gate[slot];
  }
  if constexpr (TM == TAB_FULL) fill_full_table<L>(tab, a.theta + size_t(e) * angs);
  __syncthreads();

  // ---- gather x rows -> fp32 tile (loads of a batch issued together)
  constexpr int CPR = n / 8;
  constexpr int CPT = (FZ_RT * CPR + BF_THREADS - 1) / BF_THREADS;
  constexpr int BATCH = CPT < 8 ? CPT : 8;
  const int o_base = wave * (n / 4);
  const unsigned char* wrow = a.wb + size_t(o_base + (lane & 15)) * n + 16 * (lane >> 4);
  WF W;
  for (int c0 = 0; c0 < CPT; c0 += BATCH) {
    float v[BATCH][8];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int c = (c0 + b) * BF_THREADS + tid;
      const int r = c / CPR;
      if (r < nr) load8<ACT_BF16>(a.x, s_src[r] + (c % CPR) * 8, v[b]);
    }
    if (c0 == 0) {
      // substrate prefetch, issued after the first gather batch
#pragma unroll
      for (int u = 0; u < PF; ++u) load_wfrag<L>(W.w[u], wrow, u);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int c = (c0 + b) * BF_THREADS + tid;
      const int r = c / CPR;
      if (r < nr) {
        float* d = tile + r * C::stride + pos((c % CPR) * 8);
        reinterpret_cast<float4*>(d)[0] = make_float4(v[b][0], v[b][1], v[b][2], v[b][3]);
        reinterpret_cast<float4*>(d)[1] = make_float4(v[b][4], v[b][5], v[b][6], v[b][7]);
      }
    }
  }
  __syncthreads();

  // ---- U = B(theta_e)^T x
  run_passes<L, true, false, 0, TM>(tile, nr, tab, nullptr, Rth);

  // ---- U -> bf16 operand over the start of the tile (rows >= nr are zero)
  {
    uint4 uo[CPT];
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int c = cc * BF_THREADS + tid;
      const int r = c / CPR;
      uo[cc] = make_uint4(0, 0, 0, 0);
      if (r < nr) {
        const float* sp = tile + r * C::stride + pos((c % CPR) * 8);
        const float4 x0 = reinterpret_cast<const float4*>(sp)[0];
        const float4 x1 = reinterpret_cast<const float4*>(sp)[1];
        uo[cc].x = pack_bf16x2(x0.x, x0.y);
        uo[cc].y = pack_bf16x2(x0.z, x0.w);
        uo[cc].z = pack_bf16x2(x1.x, x1.y);
        uo[cc].w = pack_bf16x2(x1.z, x1.w);
      }
    }
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int c = cc * BF_THREADS + tid;
      const int r = c / CPR;
      if (r < FZ_RT) *reinterpret_cast<uint4*>(ub + r * F::ust + (c % CPR) * 8) = uo[cc];
    }
  }
  __syncthreads();

  // ---- Z = U W^T
  f32x4_t acc[OB][RB];
#pragma unroll
  for (int i = 0; i < OB; ++i)
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint16_t* urow = ub + (lane & 15) * F::ust + 16 * (lane >> 4);
  static_assert(DS % PF == 0, "double steps in whole prefetch rounds");
#pragma unroll 1
  for (int u0 = 0; u0 < DS; u0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int u = u0 + p;
      uint4 (&wc)[OB] = W.w[p];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8_t uf[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j)
          uf[j] = *reinterpret_cast<const bf16x8_t*>(urow + 16 * j * F::ust + 64 * u + 8 * h);
#pragma unroll
        for (int i = 0; i < OB; ++i) {
          uint4 wv;
          wbytes_to_bf16(h ? wc[i].z : wc[i].x, wv.x, wv.y);
          wbytes_to_bf16(h ? wc[i].w : wc[i].y, wv.z, wv.w);
          const bf16x8_t wf = __builtin_bit_cast(bf16x8_t, wv);
#pragma unroll
          for (int j = 0; j < RB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, uf[j], acc[i][j], 0, 0, 0);
        }
      }
      if (u + PF < DS) load_wfrag<L>(wc, wrow, u + PF);
    }
  }
  __syncthreads();  // every wave has read U

  // Z (fp32, 2 alpha scale) -> tile; lane holds 4 consecutive outputs of one row
  const float zs = 2.0f * a.alpha;
#pragma unroll
  for (int i = 0; i < OB; ++i) {
    const int o = o_base + 16 * i + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int r = 16 * j + (lane & 15);
      float* d = tile + r * C::stride + pos(o);
      *reinterpret_cast<float4*>(d) =
          make_float4(zs * acc[i][j][0], zs * acc[i][j][1], zs * acc[i][j][2], zs * acc[i][j][3]);
    }
  }
  if constexpr (TM == TAB_FULL) fill_full_table<L>(tab, a.phi + size_t(e) * angs);
  __syncthreads();

  // ---- y_slot = gate * B(phi_e) Z
  run_passes<L, false, false, 0, TM>(tile, nr, tab, nullptr, Rph);

#pragma unroll
  for (int cc = 0; cc < CPT; ++cc) {
    const int c = cc * BF_THREADS + tid;
    const int r = c / CPR;
    if (r < nr) {
      const int col = (c % CPR) * 8;
      const float* sp = tile + r * C::stride + pos(col);
      const float4 x0 = reinterpret_cast<const float4*>(sp)[0];
      const float4 x1 = reinterpret_cast<const float4*>(sp)[1];
      const float g = s_gate[r];
      const float v[8] = {g * x0.x, g * x0.y, g * x0.z, g * x0.w, g * x1.x, g * x1.y, g * x1.z, g * x1.w};
      store8<ACT_BF16>(a.out, s_dst[r] + col, v);
    }
  }
}

template <int L>
static hipError_t launch_fused_L(const FusedArgs& a, hipStream_t s) {
  using F = FusedCfg<L>;
  const int grid = (a.rows + FZ_RT - 1) / FZ_RT + a.n_experts;
  auto k = fused_square_kernel<L>;
  const hipError_t err = allow_dynamic_lds((const void*)k, F::lds_bytes);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k, dim3(grid), dim3(BF_THREADS), F::lds_bytes, s, a);
  return hipGetLastError();
}

bool fused_square_supported(int log2n) { return log2n >= 6 && log2n <= 9; }

hipError_t launch_fused_square(const FusedArgs& a, int log2n, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  switch (log2n) {
    case 6: return launch_fused_L<6>(a, s);
    case 7: return launch_fused_L<7>(a, s);
    case 8: return launch_fused_L<8>(a, s);
    case 9: return launch_fused_L<9>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bmoe
