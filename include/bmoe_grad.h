/*
 * bmoe_grad.h - gradients through the experts' butterfly rotations.
 *
 * Training a ButterflyMoE layer learns, per expert, the angles of its
 * butterflies (ButterflyMoE, gist.science/zh/paper/2601.13563, technical
 * summary §2.2: the experts are rotations of the shared substrate; their
 * parameters are the angles of hierarchical Givens rotations).  This header
 * gives the backward step of one bucketed rotation pass, the building block
 * of the layer's backward: for rows r of expert e (rows offsets[e] ..
 * offsets[e+1] - 1, as bmoe_route buckets them)
 *     forward   y_r = B(angles_e) x_r          (transpose 0)
 *           or  y_r = B(angles_e)^T x_r        (transpose 1)
 * and a given dy_r = dL/dy_r it returns dx_r = dL/dx_r and, per expert,
 *     dangles_e = sum over e's rows of dL/dangles_e.
 * Butterfly wiring as in bmoe.h.  The forward rotations are recomputed in
 * fp32 from x; angle gradients are fp32 sums, per expert in a fixed order
 * (the result does not depend on scheduling).
 */
#ifndef BMOE_GRAD_H
#define BMOE_GRAD_H

#include "bmoe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Device workspace bytes bmoe_butterfly_backward needs (per-chunk partial
 * angle gradients, and for log2n >= 12 two fp32 [rows][2^log2n] buffers
 * between its passes; 0 when rows is 0).  log2n in [1, 13], n_experts in
 * [1, 256], rows >= 0. */
bmoe_status bmoe_butterfly_backward_workspace(int32_t log2n, int32_t n_experts, int32_t rows,
                                              size_t* bytes);

/* Backward of the bucketed rotation pass described above.
 *   offsets  [n_experts + 1] int32 (device): expert e owns rows offsets[e] ..
 *            offsets[e+1] - 1; offsets[0] = 0, nondecreasing, offsets[N] =
 *            rows (values outside [0, rows] are clamped to it).
 *   angles   [n_experts][log2n][2^log2n / 2] fp32 (device), read only.
 *   x, dy    [rows][2^log2n] of dtype (bmoe_dtype, device), read only.
 *   dx       [rows][2^log2n] of dtype (device), written; may be the same
 *            buffer as x or dy, must not overlap them otherwise.
 *   dangles  [n_experts][log2n][2^log2n / 2] fp32 (device), overwritten for
 *            every expert (zero for an expert without rows).
 *   workspace at least bmoe_butterfly_backward_workspace bytes (device,
 *            16-byte aligned), caller-owned scratch, contents undefined after.
 * Enqueued on `stream`; nothing is allocated or synchronised.  Errors:
 * BMOE_ERR_SHAPE (sizes), BMOE_ERR_DTYPE, BMOE_ERR_NULL, BMOE_ERR_ALIGN
 * (x, dy, dx aligned to 16 bytes when 2^log2n >= 8, else to their
 * element size; angles, dangles, offsets to 4 bytes), BMOE_ERR_ALIAS (an output overlaps an input, the workspace or the
 * other output), BMOE_ERR_WORKSPACE, BMOE_ERR_HIP; all but the last are
 * detected before anything is enqueued. */
bmoe_status bmoe_butterfly_backward(int32_t log2n, int32_t n_experts, int32_t rows,
                                    const int32_t* offsets, const float* angles, int32_t transpose,
                                    int32_t dtype, const void* x, const void* dy, void* dx,
                                    float* dangles, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Gradient of the latent substrate weights through the straight-through
 * estimator (ButterflyMoE, gist.science/nl/paper/2601.13563, §2 "Drie
 * Fasen"; gist.science/zh/paper/2601.13563, technical summary §2.2): the
 * estimator passes the gradient of Z = alpha U W^T through the ternary
 * quantiser unchanged, and the substrate is shared by all experts, so
 *     dw[o][i] = alpha * sum over rows r of dz[r][o] * u[r][i].
 *   dz   [rows][d_out] bf16 (device, 16-byte aligned): gradient at the
 *        substrate product's output, read only.
 *   u    [rows][d_in] bf16 (device, 16-byte aligned): the product's input (rows after the
 *        input rotation), read only; rows in any order, the same for both.
 *   dw   [d_out][d_in] fp32 (device, 16-byte aligned), overwritten (zero for
 *        rows = 0).
 *   workspace at least bmoe_substrate_grad_workspace bytes (device, 16-byte
 *        aligned; 0 when the output tiles fill the GPU without splitting the
 *        rows), caller-owned scratch for per-split partial sums.
 * d_out and d_in are multiples of 128 in [128, 16384].  The result does not
 * depend on scheduling (splits are added in order).  Enqueued on `stream`;
 * nothing is allocated or synchronised.  Errors: BMOE_ERR_SHAPE,
 * BMOE_ERR_DTYPE (dtype other than BMOE_BF16), BMOE_ERR_NULL, BMOE_ERR_ALIGN,
 * BMOE_ERR_ALIAS (dw or the workspace overlaps an input, or each other),
 * BMOE_ERR_WORKSPACE, BMOE_ERR_HIP; all but the last are detected before
 * anything is enqueued. */
bmoe_status bmoe_substrate_grad_workspace(int32_t d_out, int32_t d_in, int32_t rows, size_t* bytes);
bmoe_status bmoe_substrate_grad(int32_t d_out, int32_t d_in, int32_t rows, int32_t dtype, const void* dz,
                                const void* u, float alpha, float* dw, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Backward of the gated combine y_t = sum_j gate_{t,j} o_{t,j} (ButterflyMoE,
 * gist.science/nl/paper/2601.13563, §2 "Gated Routing"; the forward's combine
 * in bmoe.h).  For the routed slot s = t*top_k + j at bucket position q
 * (bucket_slots[q] = s, as bmoe_route writes it):
 *     d_rows[q] = topk_gate[s] * dy[t]      (gradient at the expert's output)
 *     d_gate[s] = dy[t] . o[q]              (only when o is given)
 *   dy           [T][d] of dtype (device, 16-byte aligned), read only.
 *   bucket_slots [T*top_k] int32 (device): a permutation of the flat slots;
 *                values outside [0, T*top_k) are clamped to it.
 *   topk_gate    [T*top_k] fp32 (device), by flat slot, read only.
 *   o            [T*top_k][d] of dtype (device, 16-byte aligned) or NULL: the
 *                experts' outputs (before the gate) in bucket order.
 *   d_rows       [T*top_k][d] of dtype (device, 16-byte aligned), written.
 *   d_gate       [T*top_k] fp32 (device) by flat slot, written; NULL exactly
 *                when o is NULL.
 * d a multiple of 8 in [8, 16384], top_k in [1, 8].  fp32 arithmetic; every
 * output is written once (no dependence on scheduling).  Enqueued on
 * `stream`, nothing allocated or synchronised.  Errors: BMOE_ERR_SHAPE,
 * BMOE_ERR_DTYPE, BMOE_ERR_NULL, BMOE_ERR_ALIGN, BMOE_ERR_ALIAS (an output
 * overlaps an input or the other output), BMOE_ERR_HIP; all but the last are
 * detected before anything is enqueued. */
bmoe_status bmoe_combine_backward(int32_t T, int32_t top_k, int32_t d, int32_t dtype, const void* dy,
                                  const int32_t* bucket_slots, const float* topk_gate, const void* o,
                                  void* d_rows, float* d_gate, hipStream_t stream);

/* Backward of the gating network with the chosen experts held (ButterflyMoE,
 * gist.science/nl/paper/2601.13563, §2 "Gated Routing"; the router of
 * bmoe.h: logits l = W_g x_t, p = softmax(l) over all experts, gate_j =
 * p_{e_j}, renormalised over the k chosen when renorm_gates is 1).  Given the
 * gates' gradients it returns the router's part of the input gradient and
 * the gate matrix's gradient:
 *     without renormalisation  dl_n = p_n (a_n - s), a_n = sum_j d_gate_j [n = e_j],
 *                              s = sum_j d_gate_j p_{e_j}
 *     with renormalisation     dl_{e_j} = g_j (d_gate_j - sum_i d_gate_i g_i), else 0
 *     dx_t = W_g^T dl_t,   dw_gate = sum_t dl_t x_t^T.
 *   x         [T][d] of dtype (device, 16-byte aligned), read only.
 *   w_gate    [n_experts][d] of dtype (device, 16-byte aligned), read only.
 *   topk_idx  [T][top_k] int32 (device): the experts held (for example
 *             bmoe_route's output); values outside [0, n_experts) are clamped.
 *   d_gate    [T][top_k] fp32 (device): gradients of the gates.
 *   dx        [T][d] fp32 (device), written: add it to the input gradient of
 *             the experts' path.
 *   dw_gate   [n_experts][d] fp32 (device), written (zero for T = 0).
 *   workspace at least bmoe_router_backward_workspace bytes (device,
 *             16-byte aligned): the logits' gradients and per-range sums.
 * d a multiple of 8 in [8, 2048], n_experts in [1, 256], top_k in [1,
 * min(8, n_experts)].  The logits are recomputed; sums are fp32 throughout.
 * With bf16 rows the logits (d a multiple of 32), dx and dw_gate (d a
 * multiple of 256) run on the matrix cores: bf16 products are exact, and dl
 * enters as two bf16 terms whose sum is within 2^-18 of it; other shapes use
 * fp32 products.  Every output is written once and the token ranges are
 * added in order, so the result does not depend on scheduling.  Enqueued on `stream`, nothing
 * allocated or synchronised.  Errors: BMOE_ERR_SHAPE, BMOE_ERR_DTYPE,
 * BMOE_ERR_NULL, BMOE_ERR_ALIGN, BMOE_ERR_ALIAS, BMOE_ERR_WORKSPACE,
 * BMOE_ERR_HIP; all but the last are detected before anything is enqueued. */
bmoe_status bmoe_router_backward_workspace(int32_t T, int32_t d, int32_t n_experts, size_t* bytes);
bmoe_status bmoe_router_backward(int32_t T, int32_t d, int32_t n_experts, int32_t top_k, int32_t renorm_gates,
                                 int32_t dtype, const void* x, const void* w_gate, const int32_t* topk_idx,
                                 const float* d_gate, float* dx, float* dw_gate, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* Derivative of the FFN experts' activation (ButterflyViT,
 * gist.science/pt/paper/2603.06746, §2; the exact (erf) GELU of bmoe.h's FFN
 * layers, with the same erf approximation, |error| <= 1.5e-7):
 *     dh = da * (Phi(h) + h phi(h))  elementwise,
 * Phi / phi the standard normal distribution function / density.
 *   h   [rows][width] of dtype (device, 16-byte aligned): the activation's
 *       input (the FFN middle's first rotation output), read only.
 *   da  [rows][width] of dtype (device, 16-byte aligned): gradient at the
 *       activation's output, read only.
 *   dh  [rows][width] of dtype (device, 16-byte aligned), written; may be the
 *       same buffer as h or da, must not overlap them otherwise.
 * width a multiple of 8.  Enqueued on `stream`, nothing allocated or
 * synchronised.  Errors: BMOE_ERR_SHAPE, BMOE_ERR_DTYPE, BMOE_ERR_NULL,
 * BMOE_ERR_ALIGN, BMOE_ERR_ALIAS, BMOE_ERR_HIP; all but the last are detected
 * before anything is enqueued. */
bmoe_status bmoe_gelu_backward(int32_t rows, int32_t width, int32_t dtype, const void* h, const void* da, void* dh,
                               hipStream_t stream);

/* Input gradient of the substrate product Z = alpha U W_base^T through the
 * straight-through estimator (ButterflyMoE, gist.science/nl/paper/2601.13563,
 * §2 "Drie Fasen"; gist.science/zh/paper/2601.13563, technical summary §2.2):
 * the forward's ternary codes are used as values, so
 *     du = alpha * dz * W_base         ([rows][d_in] = [rows][d_out] x [d_out][d_in]).
 *   dz         [rows][d_out] of dtype (device, 16-byte aligned), read only.
 *   wt_packed  W_base^T packed: [d_in][d_out / 16] words (bmoe_pack_ternary of
 *              the transposed substrate, device, 16-byte aligned), read only.
 *   du         [rows][d_in] of dtype (device, 16-byte aligned), written; must
 *              not overlap dz or wt_packed.
 * d_out and d_in multiples of 64 (bf16) or 16 (fp32); fp32 accumulation; the
 * forward's substrate GEMM.  Enqueued on `stream`, nothing allocated or
 * synchronised.  Errors: BMOE_ERR_SHAPE, BMOE_ERR_DTYPE, BMOE_ERR_NULL,
 * BMOE_ERR_ALIGN, BMOE_ERR_ALIAS, BMOE_ERR_HIP; all but the last are detected
 * before anything is enqueued. */
bmoe_status bmoe_substrate_input_grad(int32_t rows, int32_t d_out, int32_t d_in, int32_t dtype, const void* dz,
                                      const uint32_t* wt_packed, float alpha, void* du, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BMOE_GRAD_H */
