// Block factors of the butterfly rotations for the matrix-core expert kernel
// (ButterflyMoE, gist.science/zh/paper/2601.13563, technical summary §2.2:
// each expert's rotations are products of Givens stages).
//
// For width n = 2^L write an index as i = p + P m with p < P = 2^LA (LA = 5 at
// width 512, 4 at width 256) and m < 16.  Stages 0 .. LA-1 only mix indices of
// equal m and stages LA .. L-1 only indices of equal p, so
//     B = G_B G_A,  G_A = diag over m of A_m (P x P),  G_B = diag over p of B_p (16 x 16),
// each block the product of its stages' rotations.  The builder writes, per
// expert, the blocks in the per-lane order of the MFMA operands (bf16):
//   [G_B^T(theta) | G_A^T(theta) | G_A(phi) | G_B(phi)]
// (input rotation B(theta)^T = G_A^T G_B^T, output rotation B(phi) = G_B G_A).
#pragma once
#include "common.hpp"

namespace bmoe {


template <int L>
struct MfCfg {
  static constexpr int n = 1 << L;
  static constexpr int LA = L == 9 ? 5 : 4;    // stages in G_A
  static constexpr int PA = 1 << LA;           // G_A block width
  static constexpr int NM = n / PA;            // G_A blocks = G_B block width
  static constexpr int NP = PA;                // G_B blocks (classes)
  static constexpr int HA = PA / 16;           // 16-row halves of a G_A block
  static constexpr int KA = PA / 4;            // contraction values per lane in a G_A MFMA
  static constexpr int TS = 2 * n + 16;        // LDS row stride in bytes
  static constexpr size_t gb_bytes = size_t(NP) * 64 * 4 * 2;        // one G_B set
  static constexpr size_t ga_bytes = size_t(NM) * HA * 64 * KA * 2;  // one G_A set
  // per expert: [G_B^T(theta) | G_A^T(theta) | G_A(phi) | G_B(phi)]
  static constexpr size_t off_bt = 0, off_at = gb_bytes, off_ap = gb_bytes + ga_bytes,
                          off_bp = gb_bytes + 2 * ga_bytes;
  static constexpr size_t per_expert = 2 * (gb_bytes + ga_bytes);
  static_assert(NM == 16, "G_B blocks are 16 wide");
};

inline size_t mf_factor_bytes(int log2n) {
  return log2n == 8 ? MfCfg<8>::per_expert : log2n == 9 ? MfCfg<9>::per_expert : 0;
}

__device__ __forceinline__ int stage_pair_index(int i, int s) {
  return ((i >> (s + 1)) << s) | (i & ((1 << s) - 1));
}

// Apply stages [S_LO, S_HI) (local bit = s - S_LO) to a W-vector whose entry b
// sits at global index base + stride * b.  FWD: stages in increasing order with
// [[c, -s], [s, c]]; otherwise decreasing order with the transposed rotation.
template <int W, int S_LO, int S_HI, bool FWD>
__device__ __forceinline__ void rotate_vec(float (&v)[W], const float2* cs, int half, int base, int stride) {
#pragma unroll
  for (int k = 0; k < S_HI - S_LO; ++k) {
    const int s = FWD ? S_LO + k : S_HI - 1 - k;
    const int sl = s - S_LO;
#pragma unroll
    for (int q = 0; q < W / 2; ++q) {
      const int b = ((q >> sl) << (sl + 1)) | (q & ((1 << sl) - 1));
      const int i = base + stride * b;
      const float2 r = cs[s * half + stage_pair_index(i, s)];
      const float x = v[b], y = v[b + (1 << sl)];
      if (FWD) {
        v[b] = r.x * x - r.y * y;
        v[b + (1 << sl)] = r.y * x + r.x * y;
      } else {
        v[b] = r.x * x + r.y * y;
        v[b + (1 << sl)] = r.x * y - r.y * x;
      }
    }
  }
}

// (cos, sin) of every angle of one butterfly into cs (hardware transcendental
// unit: ~1e-6 error, far below the bf16 rounding of the factors).
template <int L>
__device__ __forceinline__ void mf_fill_cs(float2* cs, const float* __restrict__ ang, int tid, int nthreads) {
  constexpr float inv2pi = 0.15915494309189535f;
  for (int i = tid; i < L * (1 << (L - 1)); i += nthreads) {
    const float r = ang[i] * inv2pi;
    cs[i] = make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
  }
}

// Factor jobs of one expert: job j < 2 NM P builds a G_A vector (theta set
// first, then phi), the next 2 NP 16 a G_B vector.  theta: column j of the
// block (operand row j of its transpose); phi: row j of the block.
template <int L>
__device__ __forceinline__ void mf_factor_job(int job, const float2* cs_th, const float2* cs_ph,
                                              unsigned char* fe) {
  using C = MfCfg<L>;
  constexpr int half = C::n / 2, PA = C::PA, KA = C::KA, HA = C::HA;
  constexpr int NA = C::NM * PA;
  if (job < 2 * NA) {
    const bool th = job < NA;
    const int jj = th ? job : job - NA;
    const int m = jj / PA, j = jj % PA;
    float v[PA];
#pragma unroll
    for (int q = 0; q < PA; ++q) v[q] = q == j ? 1.0f : 0.0f;
    if (th) rotate_vec<PA, 0, C::LA, true>(v, cs_th, half, PA * m, 1);
    else rotate_vec<PA, 0, C::LA, false>(v, cs_ph, half, PA * m, 1);
    const int hq = j / 16, row = j % 16;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t h[KA / 2];
#pragma unroll
      for (int i = 0; i < KA; i += 2) {
        // contraction index held by lane group g, slot i: 4g+i (P = 16);
        // theta: 8g+i; phi (accumulator order of the substrate product): 4g+i, then 16+4g+i
        auto kidx = [&](int ii) { return KA == 4 ? 4 * g + ii : th ? 8 * g + ii : (ii < 4 ? 4 * g + ii : 12 + 4 * g + ii); };
        h[i / 2] = pack_bf16x2(v[kidx(i)], v[kidx(i + 1)]);
      }
      unsigned char* dst = fe + (th ? C::off_at : C::off_ap) + ((size_t(m) * HA + hq) * 64 + 16 * g + row) * KA * 2;
      if constexpr (KA == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(h[0], h[1], h[2], h[3]);
      else *reinterpret_cast<uint2*>(dst) = make_uint2(h[0], h[1]);
    }
  } else if (job < 2 * NA + 2 * C::NP * 16) {
    const int jb = job - 2 * NA;
    const bool th = jb < C::NP * 16;
    const int jj = th ? jb : jb - C::NP * 16;
    const int p = jj / 16, j = jj % 16;
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = q == j ? 1.0f : 0.0f;
    if (th) rotate_vec<16, C::LA, L, true>(v, cs_th, half, p, PA);
    else rotate_vec<16, C::LA, L, false>(v, cs_ph, half, p, PA);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<uint2*>(fe + (th ? C::off_bt : C::off_bp) + (size_t(p) * 64 + 16 * g + j) * 8) =
          make_uint2(pack_bf16x2(v[4 * g], v[4 * g + 1]), pack_bf16x2(v[4 * g + 2], v[4 * g + 3]));
  }
}

template <int L>
constexpr int mf_factor_jobs() {
  return 2 * MfCfg<L>::NM * MfCfg<L>::PA + 2 * MfCfg<L>::NP * 16;
}

}  // namespace bmoe
