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

/*
 * dspark_probe_draws -- the device's random draws on given inputs, for
 * checking them against their definition (Philox4x32-10 of Salmon et al.,
 * SC'11; the uniform ((w >> 8) | 1) * 2^-24; the Gumbel -ln(-ln u) with -ln u
 * taken as -log1p(-(1 - u)) for u >= 1/2), with the device functions the draft
 * and verification kernels use.
 *
 *   ctr       [n][4] uint32   Philox counters (16-byte aligned)
 *   out_words [n][4] uint32   out: Philox4x32-10 of ctr[i] under key (seed & 0xffffffff, seed >> 32)
 *   w         [m]    uint32   32-bit words
 *   uniform   [m]    float32  out: the uniform of w[i]
 *   gumbel    [m]    float32  out: the Gumbel of w[i]
 * n or m may be 0 (that part is skipped).  DSPARK_E_INVALID for n or m < 0;
 * DSPARK_E_POINTER for a NULL or misaligned array that is used.
 */
dspark_status dspark_probe_draws(uint64_t seed, const uint32_t* ctr, int32_t n, uint32_t* out_words,
                                 const uint32_t* w, int32_t m, float* uniform, float* gumbel, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_INSTR_H */
