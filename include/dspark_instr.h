/*
 * dspark_instr.h -- instrumentation entry points of the dspark library.
 *
 * Not part of the draft -> schedule -> verify contract of dspark.h: these calls
 * exist so that a benchmark can time the library's kernels on the stream they
 * are launched on, and so that a test can read the device's random draws.  They
 * follow dspark.h's conventions (device pointers, caller-owned buffers, no
 * allocation, asynchronous on `stream`, validation before any launch).
 */
#ifndef DSPARK_INSTR_H
#define DSPARK_INSTR_H

#include "dspark.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * dspark_draft_timed -- dspark_draft, plus instrumentation: events[2i] and
 * events[2i+1] (caller-created HIP events, 2*K of them) are recorded on
 * `stream` immediately before and after the vocabulary-stream kernel of draft
 * step i+1, so that the caller can read that kernel's duration with
 * hipEventElapsedTime.  Same inputs, outputs and errors as dspark_draft;
 * DSPARK_E_POINTER if events is NULL.
 */
dspark_status dspark_draft_timed(const dspark_problem* P,
                                 const void* Z, const void* E, const void* Wt, const void* h,
                                 const float* w_conf, float b_conf, const float* tau,
                                 const int32_t* anchor,
                                 int32_t* draft_tok, float* draft_logq, float* draft_lse,
                                 float* conf, float* surv,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream,
                                 hipEvent_t* events);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_INSTR_H */
