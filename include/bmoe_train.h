/*
 * bmoe_train.h - training path of the ButterflyMoE layer (bmoe.h): a forward
 * that keeps what the backward needs, and the backward of the whole layer.
 *
 * The pages train the experts' rotation angles and a latent full-precision
 * substrate whose ternary codes the forward uses, through a straight-through
 * estimator (gist.science/nl/paper/2601.13563, §2 "Drie Fasen van de
 * Methode"; gist.science/zh/paper/2601.13563, technical summary §2.2).  For a
 * loss L with dL/dy = dy, bmoe_layer_backward returns the gradients of
 * L = sum(dy * y) in every parameter and in x:
 *   - the angles theta[m], phi[m] of every expert (plain chain rule through
 *     each Givens stage, summed over the expert's routed rows);
 *   - the latent substrates: dW_m = alpha_m * sum over all routed rows of
 *     dZ_r^T U_r, the gradient of the product with the codes taken as values
 *     (the estimator read as the identity through the quantiser);
 *   - the gate matrix, through the softmax at the chosen experts (routing held
 *     at the forward's choice, which is piecewise constant in the parameters);
 *   - x: the experts' part plus the router's part.
 *
 * Precision.  The training forward runs every rotation stage by stage in fp32
 * (the backward recomputes the stages the same way) and keeps its rows in the
 * activation dtype; its y equals bmoe_forward's bit for bit on fp32 layers.
 * Row gradients between the steps are kept in the activation dtype, parameter
 * and input gradients are fp32; the substrate gradient's product takes bf16
 * copies of its two row operands (fp32 accumulation).
 *
 * Limits: those of bmoe.h, and d_model (and d_ff when nonzero) at least 128.
 * Memory rules as in bmoe.h: every pointer is caller-owned device memory,
 * 16-byte aligned; nothing is allocated; all work is enqueued on `stream`.
 */
#ifndef BMOE_TRAIN_H
#define BMOE_TRAIN_H

#include "bmoe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the state bmoe_forward_train keeps for T tokens (R = T * top_k
 * routed rows): the routing (chosen experts and gates [T][top_k], bucket
 * offsets [n_experts+1], bucket order and its inverse [R]) and, in bucket
 * order and the activation dtype, the input of every rotation and substrate
 * product and the experts' outputs: square layers U, Z, O [R][d_model]; FFN
 * layers U [R][d_model], H1, H, V [R][d_ff], Z, O [R][d_model]. */
bmoe_status bmoe_train_state_size(const bmoe_layer* layer, int32_t T, size_t* bytes);

/* Workspace bytes of bmoe_forward_train for T tokens. */
bmoe_status bmoe_forward_train_workspace(const bmoe_layer* layer, int32_t T, size_t* bytes);

/* y[t] = layer(x[t]) as bmoe_forward, keeping the state above.  x, y
 * [T][d_model] (activation dtype); state and workspace of at least the sizes
 * above; y must not overlap x, the state or the workspace.  The layer's
 * prepared buffer is not used (the training rotations run in fp32). */
bmoe_status bmoe_forward_train(const bmoe_layer* layer, const void* x, int32_t T, void* y, void* state,
                               size_t state_bytes, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Gradient outputs of bmoe_layer_backward (device, fp32, overwritten):
 *   dx        [T][d_model]
 *   d_w_gate  [n_experts][d_model]
 *   d_theta[m], d_phi[m]  shaped like layer->theta[m], layer->phi[m]
 *   d_w_base[m]           [d_out][d_in] of substrate m
 * Entries m = 1 are used by FFN layers only. */
typedef struct bmoe_layer_grads {
  float* dx;
  float* d_w_gate;
  float* d_theta[2];
  float* d_phi[2];
  float* d_w_base[2];
} bmoe_layer_grads;

/* Workspace bytes of bmoe_layer_backward for T tokens. */
bmoe_status bmoe_layer_backward_workspace(const bmoe_layer* layer, int32_t T, size_t* bytes);

/* Backward of the layer for dy [T][d_model] (activation dtype) at the state a
 * bmoe_forward_train of the same layer, x and T left.  Row gathers and
 * scatters between token and bucket order run on the device; per-token sums
 * run in slot order, so the result is deterministic.  Errors: the layer and
 * shape checks, BMOE_ERR_NULL, BMOE_ERR_ALIGN, BMOE_ERR_WORKSPACE (state or
 * workspace too small), BMOE_ERR_ALIAS (an output overlaps an input, another
 * output, the state or the workspace), BMOE_ERR_DEVICE, BMOE_ERR_HIP. */
bmoe_status bmoe_layer_backward(const bmoe_layer* layer, const void* x, int32_t T, const void* dy,
                                const void* state, size_t state_bytes, const bmoe_layer_grads* grads,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BMOE_TRAIN_H */
