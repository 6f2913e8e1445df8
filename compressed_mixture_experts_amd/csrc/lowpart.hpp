// Low part of a wide butterfly on the matrix cores: the block structure, the
// prepared factor layout and the operand helpers shared by the split
// butterfly kernels and the substrate GEMM's epilogue (ButterflyMoE,
// gist.science/zh/paper/2601.13563, technical summary §2.2: stage s rotates
// the pairs of indices that differ in bit s).
#pragma once
#include "common.hpp"

namespace bmoe {

constexpr int SP_RB = 64;  // rows per workgroup of the split butterfly kernels

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

}  // namespace bmoe
