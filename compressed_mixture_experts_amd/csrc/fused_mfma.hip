// Square-expert step with every product on the matrix cores (ButterflyMoE,
// gist.science/zh/paper/2601.13563, technical summary §2.1 and §2.2: the expert
// B(phi) W_base B(theta)^T is applied as input rotation, ternary substrate
// product and output rotation, never formed).
//
// Rotations as two block-diagonal factors.  For width n = 2^L write an index as
// i = p + P m with p < P = 2^LA (LA = 5 at width 512, 4 at width 256) and
// m < 16.  Stages 0 .. LA-1 only mix indices of equal m, stages LA .. L-1 only
// indices of equal p, so
//     B = G_B G_A,   G_A = diag over m of A_m (P x P),   G_B = diag over p of B_p (16 x 16),
// each block the product of its stages' Givens rotations.  A tile of 64 rows
// then needs 16 + P small dense products per rotation, done on MFMA in bf16
// with fp32 accumulation, instead of (n/2) L scalar rotations per row.
//
// The blocks are built once per weight set (mfma_factors.hpp), in the exact
// per-lane order of the MFMA operands (bf16): the transposed blocks of theta
// (input rotation B(theta)^T = G_A^T G_B^T) and the blocks of phi (output
// rotation G_B G_A).
//
// fused_mfma_kernel<L, RT>, one workgroup per tile of RT = 32, 48 or 64
// bucketed rows of one expert (4 waves at 32 rows, else 8), read from the tile
// record the bucketing kernel wrote (expert, rows, their slots and gates: one
// load round trip).  Two bf16 LDS buffers of RT rows alternate (wave = 2 tb +
// h, token block tb of 16 rows; NW waves; at 48 rows waves 6 and 7 sit out the
// rotations):
//   gather   x rows -> buf0 as [row][p][m]                 (transposed per row)
//   G_B^T    wave (tb, h): token block tb, classes p of half h   -> buf1 [row][m][p]
//   G_A^T    wave (tb, h): blocks m of half h                    -> buf0 [row][i]  (= U)
//   W        wave w: outputs [w n/NW, (w+1) n/NW) of all rows, accumulators kept
//            (substrate as paired 2-bit codes, expanded to exact bf16 in registers)
//   G_A      on the accumulators of the wave's own blocks        -> buf1 [row][p][m]
//   G_B      wave (tb, h): classes p of half h, * gate * alpha   -> buf0 [row][i]
//   store    buf0 rows -> per-slot rows; at top-2 they are added into y
//            instead (packed bf16 atomic adds into y, which the bucketing
//            kernel zeroed: 0 + a + b rounds the same in either order, so the
//            result is deterministic and equals a separate combine's)
// LDS is 2 x RT rows: two 32-row workgroups, or one taller one, per CU.  A
// CU's loads are bounded by its misses in flight and a tile reads ~224 KiB of
// substrate and factors at width 512, so while there are too few tiles to give
// every CU two, the shortest tiles that still fit one per CU finish first
// (fused_tile_rows); with more tiles, two 32-row workgroups per CU overlap
// each other's waits.  Every height gives every row the same arithmetic in
// the same order.
#include "mfma_factors.hpp"

namespace bmoe {

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t u4get(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

// eight fp4 (e2m1) substrate weights k..k+7 -> eight bf16 (exact: +-1 and 0)
__device__ __forceinline__ uint4 fp4x8_to_bf16(uint32_t w) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
  return r;
}

__device__ __forceinline__ f32x4_t mfma16(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                    __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int KA> struct AFragT { using type = uint2; };
template <> struct AFragT<8> { using type = uint4; };

template <int L, int RT>
__global__ __launch_bounds__(RT == 32 ? 256 : 512, RT == 32 ? 2 : 1) void fused_mfma_kernel(FusedArgs a) {
  using C = MfCfg<L>;
  using AF = typename AFragT<C::KA>::type;
  constexpr int n = C::n, PA = C::PA, NP = C::NP, HA = C::HA, TS = C::TS;
  constexpr int NT = RT == 32 ? 256 : 512;  // threads
  constexpr int NW = NT / 64;         // waves
  constexpr int MB = RT / 16;         // 16-row token blocks
  constexpr int OB = n / (16 * NW);   // substrate: 16-output blocks per wave
  constexpr int NU = n / 256;         // substrate: units of 256 contraction indices
  constexpr int NCW = NP / 2;         // G_B classes per wave
  constexpr int NBW = (n / NW) / PA;  // G_A blocks inside one wave's substrate outputs
  static_assert((RT == 32 || RT == 48 || RT == 64) && RT <= TILE_ROWS_MAX && NW >= 2 * MB, "tile rows");
  static_assert((NBW == 2 || NBW == 4) && NCW % 4 == 0 && (NU == 1 || NU == 2), "tile shape");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* buf0 = lds;
  unsigned char* buf1 = lds + size_t(RT) * TS;
  __shared__ size_t s_src[RT], s_dst[RT];
  __shared__ float s_gate[RT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int tb = wave >> 1, hh = wave & 1;
  const bool rot = tb < MB;  // wave takes part in the rotations

  // ---- this workgroup's tile record (one expert's consecutive records stay
  // on one XCD); the row entries are read with the header, before its test
  const TileRec* rec = a.rec + xcd_remap(blockIdx.x, gridDim.x);
  const int32_t rslot = rec->slot[tid < RT ? tid : 0];
  const float rgate = rec->gate[tid < RT ? tid : 0];
  const int e = rec->e;
  if (e < 0) return;
  const int nr = rec->nr;
  if (tid < nr) {
    s_src[tid] = size_t(rslot / a.top_k) * n;
    s_dst[tid] = size_t(rslot) * n;
    s_gate[tid] = rgate * a.alpha;
  }

  // ---- input-rotation factor fragments of this expert
  const unsigned char* fe = a.fac + size_t(e) * C::per_expert;
  uint2 fbt[NCW];
  if (rot) {
#pragma unroll
    for (int c = 0; c < NCW; ++c)
      fbt[c] = *reinterpret_cast<const uint2*>(fe + C::off_bt + (size_t(hh * NCW + c) * 64 + lane) * 8);
  }
  __syncthreads();

  // ---- gather x rows into buf0 as [row][p][m]: item (row, m-quad, 8 p's)
  constexpr int PG = PA / 8;
  constexpr int ITEMS = RT * 4 * PG;
  constexpr int IPT = (ITEMS + NT - 1) / NT;  // items past ITEMS have rows t >= RT >= nr
  // substrate rows: n/4 bytes of paired 2-bit codes (16 weights per word).
  // Unit v covers contraction indices [256v, 256v+256) = bytes [64v, 64v+64)
  // of a row; lane group g takes bytes 8g..8g+7 of each 32-byte half, the
  // words of indices 256v + 128h + 32g .. +31.
  const unsigned char* wrow = a.wb + size_t(wave * (n / NW) + l16) * (n / 4) + 8 * g;
  uint2 W0[OB][2];
  {
    uint4 ch[IPT][4];
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = it * NT + tid;
      const int pg = item % PG, mq = (item / PG) % 4, t = item / (PG * 4);
      if (t < nr) {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(a.x) + s_src[t] + 8 * pg;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          ch[it][mi] = *reinterpret_cast<const uint4*>(src + PA * (4 * mq + mi));
      }
    }
    // first substrate unit, after the gather loads
#pragma unroll
    for (int i = 0; i < OB; ++i)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        W0[i][hf] = *reinterpret_cast<const uint2*>(wrow + size_t(16 * i) * (n / 4) + 32 * hf);
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = it * NT + tid;
      const int pg = item % PG, mq = (item / PG) % 4, t = item / (PG * 4);
      if (t < nr) {
        unsigned char* dst = buf0 + t * TS + ((8 * pg) * 16 + 4 * mq) * 2;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t lo = __builtin_amdgcn_perm(u4get(ch[it][1], j >> 1), u4get(ch[it][0], j >> 1), sel);
          const uint32_t hi = __builtin_amdgcn_perm(u4get(ch[it][3], j >> 1), u4get(ch[it][2], j >> 1), sel);
          *reinterpret_cast<uint2*>(dst + j * 32) = make_uint2(lo, hi);
        }
      }
    }
  }
  AF fat[8][HA];  // second input-rotation factor, used after the next barrier
  if (rot) {
#pragma unroll
    for (int jb = 0; jb < 8; ++jb)
#pragma unroll
      for (int hq = 0; hq < HA; ++hq)
        fat[jb][hq] = *reinterpret_cast<const AF*>(
            fe + C::off_at + ((size_t(8 * hh + jb) * HA + hq) * 64 + lane) * sizeof(AF));
  }
  __syncthreads();

  const int trow = 16 * tb + l16;  // this lane's row in the butterfly phases
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  // ---- G_B^T (theta): classes hh*NCW .. +NCW of token block tb  -> buf1 [row][m][p]
  if (rot) {
    const unsigned char* xr = buf0 + trow * TS;
    unsigned char* yr = buf1 + trow * TS;
#pragma unroll
    for (int cg = 0; cg < NCW / 4; ++cg) {
      f32x4_t d[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int p = hh * NCW + 4 * cg + c;
        const uint2 b = *reinterpret_cast<const uint2*>(xr + (p * 16 + 4 * g) * 2);
        d[c] = mfma16(fbt[4 * cg + c], b, zero4);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint2*>(yr + ((4 * g + i) * PA + hh * NCW + 4 * cg) * 2) =
            make_uint2(pack_bf16x2(d[0][i], d[1][i]), pack_bf16x2(d[2][i], d[3][i]));
    }
  }
  __syncthreads();

  // ---- G_A^T (theta): blocks 8hh .. 8hh+7 of token block tb  -> buf0 [row][i] (U)
  if (rot) {
    const unsigned char* yr = buf1 + trow * TS;
    unsigned char* ur = buf0 + trow * TS;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      const int mb = 8 * hh + jb;
#pragma unroll
      for (int hq = 0; hq < HA; ++hq) {
        f32x4_t d;
        if constexpr (C::KA == 8) {
          const uint4 b = *reinterpret_cast<const uint4*>(yr + (mb * PA + 8 * g) * 2);
          d = mfma32(fat[jb][hq], b, zero4);
        } else {
          const uint2 b = *reinterpret_cast<const uint2*>(yr + (mb * PA + 4 * g) * 2);
          d = mfma16(fat[jb][hq], b, zero4);
        }
        *reinterpret_cast<uint2*>(ur + (PA * mb + 16 * hq + 4 * g) * 2) =
            make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
      }
    }
  }
  uint2 W1[OB][2];  // second substrate unit (width 512)
  if constexpr (NU == 2) {
#pragma unroll
    for (int i = 0; i < OB; ++i)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        W1[i][hf] = *reinterpret_cast<const uint2*>(wrow + size_t(16 * i) * (n / 4) + 64 + 32 * hf);
  }
  __syncthreads();

  // ---- Z = U W^T: wave owns outputs [wave n/NW, (wave+1) n/NW) of all RT rows.
  // In unit v, MFMA step s (8 contraction indices) of lane group g uses
  // indices 256v + 128(s/4) + 32g + 8(s%4) .. +7: word (s%4)/2 of half s/4,
  // its lower or upper eight weights; the U operand is read in the same order.
  f32x4_t acc[OB][MB];
#pragma unroll
  for (int i = 0; i < OB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = zero4;
  const uint16_t* urow = reinterpret_cast<const uint16_t*>(buf0) + l16 * (TS / 2) + 32 * g;
  auto unit = [&](const uint2 (&Wu)[OB][2], int v) {
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int kk = 256 * v + 128 * (st >> 2) + 8 * (st & 3);
      uint4 uf[MB];
#pragma unroll
      for (int j = 0; j < MB; ++j) uf[j] = *reinterpret_cast<const uint4*>(urow + 16 * j * (TS / 2) + kk);
#pragma unroll
      for (int i = 0; i < OB; ++i) {
        const uint2 wd = Wu[i][st >> 2];
        const uint4 wv = fp4x8_to_bf16(pair2_to_fp4((st & 2) ? wd.y : wd.x, st & 1));
#pragma unroll
        for (int j = 0; j < MB; ++j) acc[i][j] = mfma32(wv, uf[j], acc[i][j]);
      }
    }
  };
  // output-rotation factors, loaded once the first unit's substrate registers
  // are free so that the second unit's products cover their latency
  AF fa[NBW][HA];
  uint2 fb[NCW];  // last factor, used after the next barrier
  auto load_out_factors = [&]() {
#pragma unroll
    for (int jm = 0; jm < NBW; ++jm)
#pragma unroll
      for (int hq = 0; hq < HA; ++hq)
        fa[jm][hq] = *reinterpret_cast<const AF*>(
            fe + C::off_ap + ((size_t(NBW * wave + jm) * HA + hq) * 64 + lane) * sizeof(AF));
#pragma unroll
    for (int c = 0; c < NCW; ++c)
      fb[c] = *reinterpret_cast<const uint2*>(fe + C::off_bp + (size_t(hh * NCW + c) * 64 + lane) * 8);
  };
  unit(W0, 0);
  load_out_factors();
  if constexpr (NU == 2) unit(W1, 1);

  // ---- G_A (phi) on the accumulators: blocks NBW*wave .. +NBW-1  -> buf1 [row][p][m]
  // (buf1 was last read before the barrier above; buf0 still holds U for the
  // other waves, so it is not touched here)
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    f32x4_t d[NBW][HA];
#pragma unroll
    for (int jm = 0; jm < NBW; ++jm) {
      if constexpr (C::KA == 8) {
        const f32x4_t z0 = acc[2 * jm][rb], z1 = acc[2 * jm + 1][rb];
        const uint4 b = make_uint4(pack_bf16x2(z0[0], z0[1]), pack_bf16x2(z0[2], z0[3]),
                                   pack_bf16x2(z1[0], z1[1]), pack_bf16x2(z1[2], z1[3]));
#pragma unroll
        for (int hq = 0; hq < HA; ++hq) d[jm][hq] = mfma32(fa[jm][hq], b, zero4);
      } else {
        const f32x4_t z0 = acc[jm][rb];
        const uint2 b = make_uint2(pack_bf16x2(z0[0], z0[1]), pack_bf16x2(z0[2], z0[3]));
        d[jm][0] = mfma16(fa[jm][0], b, zero4);
      }
    }
    unsigned char* yr = buf1 + (16 * rb + l16) * TS;
#pragma unroll
    for (int hq = 0; hq < HA; ++hq)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = 16 * hq + 4 * g + i;
        if constexpr (NBW == 4)
          *reinterpret_cast<uint2*>(yr + (p * 16 + NBW * wave) * 2) =
              make_uint2(pack_bf16x2(d[0][hq][i], d[1][hq][i]), pack_bf16x2(d[2][hq][i], d[3][hq][i]));
        else
          *reinterpret_cast<uint32_t*>(yr + (p * 16 + NBW * wave) * 2) = pack_bf16x2(d[0][hq][i], d[1][hq][i]);
      }
  }
  __syncthreads();

  // ---- G_B (phi), * gate * alpha: classes hh*NCW .. of token block tb -> buf0 [row][i]
  if (rot) {
    const unsigned char* yr = buf1 + trow * TS;
    unsigned char* orow = buf0 + trow * TS;
    const float gs = s_gate[trow];
#pragma unroll
    for (int cg = 0; cg < NCW / 4; ++cg) {
      f32x4_t d[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int p = hh * NCW + 4 * cg + c;
        const uint2 b = *reinterpret_cast<const uint2*>(yr + (p * 16 + 4 * g) * 2);
        d[c] = mfma16(fb[4 * cg + c], b, zero4);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint2*>(orow + (hh * NCW + 4 * cg + PA * (4 * g + i)) * 2) =
            make_uint2(pack_bf16x2(gs * d[0][i], gs * d[1][i]), pack_bf16x2(gs * d[2][i], gs * d[3][i]));
    }
  }
  __syncthreads();

  // ---- per-slot rows
  constexpr int CPR = n / 8;
  if (a.yatom) {
    // each row's gated values added into its token's row of y, two bf16 per
    // lane, consecutive lanes on consecutive words
    typedef __bf16 bf2v_t __attribute__((ext_vector_type(2)));
    for (int w = tid; w < RT * (n / 2); w += NT) {
      const int r = w / (n / 2), c = w % (n / 2);
      if (r < nr)
        __builtin_amdgcn_global_atomic_fadd_v2bf16(
            (__attribute__((address_space(1))) bf2v_t*)(reinterpret_cast<uint16_t*>(a.yatom) + s_src[r] + 2 * c),
            __builtin_bit_cast(bf2v_t, *reinterpret_cast<const uint32_t*>(buf0 + r * TS + 4 * c)));
    }
    return;
  }
#pragma unroll
  for (int c = tid; c < RT * CPR; c += NT) {
    const int r = c / CPR;
    if (r < nr)
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + s_dst[r] + 8 * (c % CPR)) =
          *reinterpret_cast<const uint4*>(buf0 + r * TS + 16 * (c % CPR));
  }
}

template <int L, int RT>
static hipError_t launch_fused_mfma_L(const FusedArgs& a, hipStream_t s) {
  const size_t lds = size_t(2) * RT * MfCfg<L>::TS;
  const int grid = (a.rows + RT - 1) / RT + a.n_experts;
  auto k = fused_mfma_kernel<L, RT>;
  const hipError_t err = allow_dynamic_lds((const void*)k, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k, dim3(grid), dim3(RT == 32 ? 256 : 512), lds, s, a);
  return hipGetLastError();
}

int fused_tile_rows(int rows, int n_experts) {
  // compute units of the current device, asked on every call (no cached state)
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
    cu = 256;
  auto tiles = [&](int rt) { return (long(rows) + rt - 1) / rt + n_experts; };  // records, a bound on tiles
  if (tiles(32) > 2L * cu) return 32;
  return tiles(48) <= cu ? 48 : 64;
}

bool fused_mfma_supported(int log2n) { return log2n == 8 || log2n == 9; }

size_t factor_bytes_per_expert(int log2n) { return mf_factor_bytes(log2n); }

hipError_t launch_fused_mfma(const FusedArgs& a, int log2n, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (!a.rec) return hipErrorInvalidValue;
  const int rt = a.tile_rows;
  if (rt != 32 && rt != 48 && rt != 64) return hipErrorInvalidValue;
  switch (log2n) {
    case 8: return rt == 64 ? launch_fused_mfma_L<8, 64>(a, s)
                   : rt == 48 ? launch_fused_mfma_L<8, 48>(a, s) : launch_fused_mfma_L<8, 32>(a, s);
    case 9: return rt == 64 ? launch_fused_mfma_L<9, 64>(a, s)
                   : rt == 48 ? launch_fused_mfma_L<9, 48>(a, s) : launch_fused_mfma_L<9, 32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bmoe
