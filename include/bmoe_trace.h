/*
 * bmoe_trace.h - timing hooks of the ButterflyMoE layer forward (bmoe.h):
 * the kernel launches one bmoe_forward makes, and a forward that records
 * caller-owned HIP events between them, so that single kernels of a live
 * forward can be timed on the stream they run on (also inside a captured
 * graph).  Same validation rules and error codes as bmoe.h.
 */
#ifndef BMOE_TRACE_H
#define BMOE_TRACE_H

#include "bmoe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Names of the kernel launches one bmoe_forward makes for this layer, in
 * launch order, comma-separated into `names` (truncated to names_len, always
 * NUL-terminated when names_len > 0; names may be NULL), and their number in
 * *n_kernels.  Errors: the layer checks of bmoe_forward, BMOE_ERR_NULL when
 * n_kernels is NULL. */
bmoe_status bmoe_forward_kernels(const bmoe_layer* layer, int32_t* n_kernels, char* names,
                                 size_t names_len);

/* bmoe_forward (without the optional routing outputs) that also records
 * marks[0] on `stream` before its first kernel launch and marks[i] after its
 * i-th launch (i = 1 .. n_kernels); NULL entries and entries at or beyond
 * n_marks are skipped.  The events are created and owned by the caller; the
 * call never synchronises.  Errors: those of bmoe_forward, BMOE_ERR_SHAPE
 * when n_marks is negative. */
bmoe_status bmoe_forward_marked(const bmoe_layer* layer, const void* x, int32_t T, void* y,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t* marks, int32_t n_marks);

#ifdef __cplusplus
}
#endif
#endif /* BMOE_TRACE_H */
