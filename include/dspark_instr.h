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

/* The two schedules of the K-position draft phase (Method > Semi-autoregressive
 * generation: the same sequential computation either way, with identical
 * results up to floating-point summation order):
 *   DSPARK_DRAFT_PER_POSITION  one stream kernel and one selection kernel per
 *                              position, each re-reading Wt;
 *   DSPARK_DRAFT_PERSISTENT    one cooperative launch for all K positions, each
 *                              CU's slice of Wt held on chip for the cycle
 *                              (bf16 logits and factors, r = 256, B <= 256, a
 *                              device that launches cooperatively; not under
 *                              stream capture, not for the RNN head).
 * dspark_draft takes DSPARK_DRAFT_AUTO: the persistent schedule where it applies
 * and B <= 48, else the per-position one (the measured crossover). */
enum {
  DSPARK_DRAFT_AUTO = 0,
  DSPARK_DRAFT_PER_POSITION = 1,
  DSPARK_DRAFT_PERSISTENT = 2
};

/*
 * dspark_draft_timed -- dspark_draft with a chosen schedule and optional
 * timing.  `path` is one of the DSPARK_DRAFT_* values above.  If `events` is
 * not NULL, events[0] and events[1] (caller-created HIP events) are recorded on
 * `stream` immediately before the first and after the last kernel of the
 * K-position draft phase, before the confidence head, so that the caller can
 * read the phase's duration with hipEventElapsedTime.  Same inputs, outputs
 * and errors as dspark_draft, plus DSPARK_E_INVALID for an unknown `path` and
 * DSPARK_E_UNSUPPORTED for DSPARK_DRAFT_PERSISTENT where it does not apply.
 */
dspark_status dspark_draft_timed(const dspark_problem* P,
                                 const void* Z, const void* E, const void* Wt, const void* h,
                                 const float* w_conf, float b_conf, const float* tau,
                                 const int32_t* anchor,
                                 int32_t* draft_tok, float* draft_logq, float* draft_lse,
                                 float* conf, float* surv,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream,
                                 hipEvent_t* events, int32_t path);

/*
 * dspark_draft_path -- the schedule dspark_draft takes for problem P outside
 * stream capture: DSPARK_DRAFT_PERSISTENT or DSPARK_DRAFT_PER_POSITION, or a
 * negative dspark_status if P is invalid.  The first call may query the
 * device (cooperative launch support and occupancy).
 */
int32_t dspark_draft_path(const dspark_problem* P);

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
