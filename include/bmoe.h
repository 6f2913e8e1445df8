/*
 * bmoe.h - ButterflyMoE expert-layer forward pass on AMD Instinct MI355X (gfx950).
 *
 * The layer (ButterflyMoE: Sub-Linear Ternary Experts via Structured Butterfly
 * Orbits; gist.science/zh/paper/2601.13563, technical summary §2.1 and §2.2):
 *   - N experts share one ternary substrate W_base with entries in {-1, 0, +1};
 *   - expert e is W_e = B(phi_e) * W_base * B(theta_e)^T, where each B is an
 *     orthogonal butterfly of log2(n) stages of Givens rotations, (n/2) angles
 *     per stage, n the width it acts on;
 *   - experts are never materialised: a routed token is rotated by
 *     B(theta_e)^T, multiplied by the ternary substrate, rotated by B(phi_e);
 *   - a standard top-k gating network picks the experts of each token
 *     (gist.science/nl/paper/2601.13563, §2 "Drie Fasen van de Methode").
 * The FFN form (ButterflyViT, gist.science/pt/paper/2603.06746, §2) has an up
 * substrate (d_ff x d_model) and a down substrate (d_model x d_ff), each with
 * its own pair of rotations, and an exact-erf GELU between them.
 *
 * Conventions fixed by this library where the pages are silent:
 *   Butterfly B(a) of width n = 2^L, angles a[L][n/2] (fp32, row-major):
 *     stage s rotates the pair (i, j = i + 2^s), bit s of i clear, by the angle
 *     a[s][p], p = i with bit s deleted:  v_i' = c v_i - s v_j,
 *     v_j' = s v_i + c v_j  (c = cos a, s = sin a);  B = S_{L-1} ... S_1 S_0.
 *   Router: logits l = W_g x (W_g row-major [n_experts][d_model], no bias);
 *     top-k by logit, larger first, equal logits to the lower expert index;
 *     gate = softmax(l) of the chosen expert over all N logits, divided by the
 *     sum of the k gates when renorm_gates is 1.
 *   Combine: y_t = sum_j gate_{t,j} * E_{e_{t,j}}(x_t); no capacity limit.
 *   Ternary storage: bmoe_pack_ternary's 2-bit format (see below).
 *
 * Memory and streams.  Every pointer argument of bmoe_route and bmoe_forward
 * is device memory owned by the caller; all arrays are row-major and dense.
 * x, y, w_gate, the workspace and the packed substrates must be 16-byte
 * aligned; angle arrays 4-byte aligned.  The library allocates and frees
 * nothing, never synchronises the device, and enqueues all work on the given
 * stream (0 = default stream).  Inputs must stay valid until the stream has
 * passed the call.  Calls on different streams must use different workspaces
 * and outputs.
 *
 * Errors.  Argument errors are detected on the host before anything is
 * enqueued (no partial launch); bmoe_last_error() then holds a description.
 * BMOE_ERR_HIP reports a failed HIP call or kernel launch.  bmoe_last_error()
 * is per host thread.
 *
 * Limits.  d_model and d_ff (when nonzero) are powers of two in [64, 8192];
 * 1 <= n_experts <= 256; 1 <= top_k <= min(8, n_experts); 0 <= T.
 *
 * Layout choices (the pages fix no interface; these are this library's):
 *   - The gate matrix is stored expert-major, [n_experts][d_model]: expert e's
 *     gate vector is one contiguous row, which is the operand layout the
 *     router's matrix-core tiles load (16 experts x 32 columns per fragment).
 *     A caller holding W_g as [d_model][n_experts] passes its transpose.
 *   - Angles come as one array per rotation (theta[m], phi[m]), each
 *     [n_experts][log2 n][n/2], rather than one array holding every rotation
 *     of an expert: a kernel applies one rotation to the rows of many
 *     experts, so each rotation's angles of all experts are one contiguous
 *     block.  The four rotations of an FFN expert are theta[0] (B(theta_up),
 *     width d_model), phi[0] (B(phi_up), d_ff), theta[1] (B(theta_dn), d_ff)
 *     and phi[1] (B(phi_dn), d_model).
 *   - The library keeps no state between calls except the per-thread error
 *     string; every call re-derives what it needs from its arguments.
 */
#ifndef BMOE_H
#define BMOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bmoe_status {
  BMOE_OK = 0,
  BMOE_ERR_NULL = 1,        /* a required pointer is NULL                      */
  BMOE_ERR_SHAPE = 2,       /* a size is outside the limits above              */
  BMOE_ERR_DTYPE = 3,       /* unknown dtype / activation code                 */
  BMOE_ERR_ALIGN = 4,       /* a pointer is not aligned as required            */
  BMOE_ERR_ALIAS = 5,       /* an output overlaps an input or the workspace    */
  BMOE_ERR_WORKSPACE = 6,   /* workspace / prepared buffer smaller than needed */
  BMOE_ERR_TERNARY = 7,     /* a substrate value is not in {-1, 0, +1}         */
  BMOE_ERR_HIP = 8,         /* a HIP runtime call or kernel launch failed      */
  BMOE_ERR_DEVICE = 9       /* the current device is not a gfx950 GPU          */
} bmoe_status;

typedef enum bmoe_dtype {
  BMOE_F32 = 0,             /* IEEE binary32                                   */
  BMOE_BF16 = 1             /* bfloat16 (upper half of binary32)               */
} bmoe_dtype;

typedef enum bmoe_act {
  BMOE_ACT_NONE = 0,
  BMOE_ACT_GELU_ERF = 1     /* h * (1 + erf(h / sqrt 2)) / 2                   */
} bmoe_act;

/* One ButterflyMoE layer.  Substrate m (m = 0, or m = 0 and 1 for the FFN
 * form) has shape d_out(m) x d_in(m):
 *   square layer (d_ff == 0): m=0 is d_model x d_model;
 *   FFN layer    (d_ff  > 0): m=0 (up) is d_ff x d_model, m=1 (down) is
 *                             d_model x d_ff.
 * All pointers are device memory. */
typedef struct bmoe_layer {
  int32_t d_model;          /* width of x and y                                 */
  int32_t d_ff;             /* 0: square experts; else FFN hidden width         */
  int32_t n_experts;        /* N                                                */
  int32_t top_k;            /* k                                                */
  int32_t act_dtype;        /* bmoe_dtype of x, y and w_gate                    */
  int32_t ffn_act;          /* bmoe_act between the FFN substrates (FFN only)   */
  int32_t renorm_gates;     /* 0: gate = softmax probability; 1: renormalised   */
  int32_t reserved;         /* must be 0                                        */
  const void* w_gate;       /* [n_experts][d_model], act_dtype                  */
  const uint32_t* w_base[2];/* packed substrate m: [d_out][d_in/16] words       */
  const float* theta[2];    /* input-side angles of substrate m:
                               [n_experts][log2 d_in][d_in/2]                   */
  const float* phi[2];      /* output-side angles of substrate m:
                               [n_experts][log2 d_out][d_out/2]                 */
  float w_scale[2];         /* scalar multiplying substrate m (normally 1.0)    */
  const void* prepared;     /* NULL, or a buffer filled by bmoe_prepare for these
                               weights (256-byte aligned, device memory)       */
  size_t prepared_bytes;    /* its size (ignored when prepared is NULL)         */
} bmoe_layer;

/* Number of 32-bit words bmoe_pack_ternary writes for a rows x cols matrix
 * (rows * cols / 16), or 0 when cols is not a positive multiple of 16. */
size_t bmoe_packed_words(int32_t rows, int32_t cols);

/* Pack a ternary matrix (HOST memory, int8 row-major [rows][cols], values in
 * {-1, 0, +1}) into the 2-bit substrate format, synchronously on the host.
 * Word w of row r holds columns 16w .. 16w+15.  For a column c = 16w + 2j + h
 * (j = 0..7, h = 0 or 1) the word holds a nonzero bit at position 16h + j and
 * a sign bit (1 = negative) at position 16h + 8 + j; a zero entry has both
 * bits clear.  Errors: BMOE_ERR_NULL, BMOE_ERR_SHAPE (cols not a multiple of
 * 16, rows < 1, out_words too small), BMOE_ERR_TERNARY (first bad index in
 * bmoe_last_error()).  ButterflyMoE zh §2.2: substrate values are ternary. */
bmoe_status bmoe_pack_ternary(const int8_t* w, int32_t rows, int32_t cols,
                              uint32_t* out, size_t out_words);

/* Bytes of device workspace bmoe_route / bmoe_forward need for T tokens.
 * Depends on the layer's sizes, T and whether layer->prepared is set. */
bmoe_status bmoe_workspace_size(const bmoe_layer* layer, int32_t T, size_t* bytes);

/* Size of the prepared-weights buffer of this layer, 0 when its forward path
 * uses none (or the layer is invalid).  Every bf16 layer uses one; fp32
 * layers use none.  Contents, all depending on the weights only
 * (ButterflyMoE zh §2.1-§2.2: ternary substrate, per-expert Givens angles;
 * nl §2: the gating network):
 *  - square layers of width 64..512: the substrate re-encoded for the expert
 *    kernel (one byte per weight at widths 64 and 128; at 256 and 512 two bits
 *    per weight, each 32-bit word holding 16 consecutive weights with the
 *    nonzero and sign bits of weight c < 8 at bits 4c+1 and 4c+3 and of
 *    weight 8+c at bits 4c and 4c+2, so that a mask gives fp4 e2m1 nibbles)
 *    and, at widths 256 and 512, every expert's
 *    rotations as block-diagonal factors in bf16 (stages below bit 5 at width
 *    512 / bit 4 at width 256 as one block per group of 32 / 16 consecutive
 *    indices, the stages above as 16 x 16 blocks);
 *  - other layers: each substrate whose product has an output width that is a
 *    multiple of 256 and a contraction that is a multiple of 128, in the same
 *    two-bit code; and
 *    for every rotation of width n = 2^L in 1024..8192, per expert, its stages
 *    0..L-5 as block factors per chunk of 2^(L-4) indices and its top four
 *    stages as one 16 x 16 block per column (bf16) -- except the FFN's
 *    phi_up of width 8192 when the up product runs on the two-bit code: its
 *    stages 0..7 per chunk of 256 indices (the up product applies them to
 *    its output; stage 8 is taken from the angles);
 *  - every bf16 layer, last: the gate matrix W_g reordered for the router's
 *    matrix-core products, ceil(n_experts / 16) * 16 * d_model * 2 bytes
 *    (per block of 16 experts and contraction step of 32, the 16-byte pieces
 *    in operand-lane order; experts past n_experts zero). */
size_t bmoe_prepared_bytes(const bmoe_layer* layer);

/* Fill `prepared` (device, 256-byte aligned, at least bmoe_prepared_bytes) for
 * the weights of `layer` (layer->prepared itself is ignored), enqueued on
 * `stream`.  Afterwards set layer->prepared / prepared_bytes to skip this work
 * in every bmoe_forward; it stays valid while the weights are unchanged.
 * A layer that uses no prepared buffer returns BMOE_OK and writes nothing.
 * Errors: those of the layer checks, BMOE_ERR_NULL, BMOE_ERR_ALIGN,
 * BMOE_ERR_WORKSPACE (buffer too small), BMOE_ERR_ALIAS (buffer overlaps a
 * weight array), BMOE_ERR_DEVICE, BMOE_ERR_HIP. */
bmoe_status bmoe_prepare(const bmoe_layer* layer, void* prepared, size_t bytes, hipStream_t stream);

/* Router and per-expert bucketing only.
 *   x              [T][d_model] act_dtype
 *   topk_idx       [T][top_k] int32 out: chosen experts, larger logit first
 *   topk_gate      [T][top_k] fp32  out: their gates
 *   expert_offsets [n_experts+1] int32 out (may be NULL): rows of expert e are
 *                  bucket positions offsets[e] .. offsets[e+1]-1
 *   bucket_slots   [T*top_k] int32 out (may be NULL): bucket position q holds
 *                  the flat slot t*top_k + j; within an expert, slots ascend
 * Expert indices equal those of an exact-arithmetic top-k: logits are computed
 * in fp32 and every token whose decisive gaps fall within the fp32 error bound
 * is recomputed in fp64. */
bmoe_status bmoe_route(const bmoe_layer* layer, const void* x, int32_t T,
                       int32_t* topk_idx, float* topk_gate,
                       int32_t* expert_offsets, int32_t* bucket_slots,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Full layer forward: y[t] = sum_j gate_{t,j} * E_{e_{t,j}}(x_t).
 *   x  [T][d_model] act_dtype;  y [T][d_model] act_dtype (must not overlap x,
 *   the workspace or the optional outputs);
 *   topk_idx / topk_gate: optional [T][top_k] outputs as in bmoe_route.
 * Intermediates between the steps are kept in act_dtype; GELU and
 * accumulation run in fp32.  Rotations run in fp32, except where they are
 * products with the bf16 block factors described at bmoe_prepared_bytes
 * (square bf16 layers of width 256 and 512; bf16 rotations of width
 * 1024..8192): fp32 accumulation, bf16 rounding between factors.  Square
 * bf16 layers of width 256 / 512 with top_k = 2 combine inside the expert
 * kernel: y is first zeroed, then each routed row is added into it with
 * packed bf16 atomic adds; two adds onto zero round the same in either order,
 * so y is deterministic and equal to a separate fp32 combine rounded once.
 * Without layer->prepared the call builds the prepared data in the
 * workspace first. */
bmoe_status bmoe_forward(const bmoe_layer* layer, const void* x, int32_t T, void* y,
                         int32_t* topk_idx, float* topk_gate,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the fixed device scratch that bmoe_forward_noalloc uses as its
 * workspace (64 MiB; one copy per GPU the library runs on, held until the
 * process ends). */
#define BMOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* bmoe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as bmoe_forward, but no workspace argument:
 * the library's own scratch array on the current device serves as the
 * workspace, so the call allocates nothing (no hipMalloc / hipFree; its first
 * call on a device looks up that device's scratch address once).
 *   - Layers and T whose bmoe_workspace_size exceeds
 *     BMOE_NOALLOC_SCRATCH_BYTES are rejected with BMOE_ERR_WORKSPACE before
 *     anything is enqueued (e.g. the d=512, 64-expert, top-2 layer fits up to
 *     about 30000 tokens with prepared weights).
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap in
 *     time on one device (different streams, or different host threads
 *     without ordering) race and give undefined results.  Calls ordered on
 *     one stream are safe; nothing in the scratch carries over between calls.
 *   - y must not overlap x or the optional routing outputs (BMOE_ERR_ALIAS). */
bmoe_status bmoe_forward_noalloc(const bmoe_layer* layer, const void* x, int32_t T, void* y,
                                 int32_t* topk_idx, float* topk_gate, hipStream_t stream);

/* Static description of a status code. */
const char* bmoe_status_string(bmoe_status status);

/* Detail of the last error on this host thread ("" if none). */
const char* bmoe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BMOE_H */
