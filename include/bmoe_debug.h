/*
 * bmoe_debug.h - single steps of the ButterflyMoE forward path, exported so
 * that each kernel can be checked on its own against a reference.  They run
 * the same kernels bmoe_forward runs, on caller-given device buffers, enqueued
 * on `stream`, with the same validation rules and error codes as bmoe.h.
 *
 * Test-only: these functions exist only in a library compiled with
 * -DBMOE_DEBUG_EXPORTS (libbmoe_debug.so, built beside libbmoe.so); the
 * product library libbmoe.so does not export them.
 */
#ifndef BMOE_DEBUG_H
#define BMOE_DEBUG_H

#include "bmoe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Apply one butterfly to every row: out[r] = B(angles) in[r], or
 * B(angles)^T in[r] when transpose is 1 (ButterflyMoE zh §2.2: hierarchical
 * Givens rotations; wiring as documented in bmoe.h).
 *   log2n in [1, 13]; rows >= 0; angles [log2n][2^log2n / 2] fp32 (device);
 *   in, out [rows][2^log2n] of dtype (bmoe_dtype), 16-byte aligned, may be
 *   the same buffer.  Rotations run in fp32. */
bmoe_status bmoe_dbg_butterfly(int32_t log2n, int32_t rows, const float* angles,
                               int32_t transpose, int32_t dtype,
                               const void* in, void* out, hipStream_t stream);

/* Ternary substrate product z = alpha * a * W^T (ButterflyMoE zh §2.2:
 * ternary substrate).
 *   a [M][K] of dtype; w_packed [N][K/16] words (bmoe_pack_ternary format);
 *   z [M][N] of dtype; fp32 accumulation.  K and N are multiples of 64
 *   (bf16) or 16 (fp32); M >= 0. */
bmoe_status bmoe_dbg_ternary_gemm(int32_t M, int32_t N, int32_t K, int32_t dtype,
                                  const void* a, const uint32_t* w_packed, float alpha,
                                  void* z, hipStream_t stream);

/* The same product on the matrix-core path of bf16 layers: W is re-encoded as
 * paired 2-bit codes into `w_fp4` (N * K / 4 bytes, device, 16-byte aligned,
 * caller-owned scratch, overwritten; each 32-bit word holds 16 consecutive
 * weights and masks turn it into fp4 e2m1 nibbles, in which +-1 and 0 are
 * exact), then multiplied with bf16 operands and fp32 accumulation
 * (ButterflyMoE zh §2.2: ternary substrate).  a [M][K] bf16, z [M][N] bf16; N
 * a multiple of 256, K a multiple of 128, M >= 0.  w_fp4 must overlap none of
 * a, w_packed, z. */
bmoe_status bmoe_dbg_ternary_gemm_fp4(int32_t M, int32_t N, int32_t K, const void* a,
                                      const uint32_t* w_packed, void* w_fp4, float alpha,
                                      void* z, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BMOE_DEBUG_H */
