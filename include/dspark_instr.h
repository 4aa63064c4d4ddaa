/*
 * dspark_instr.h -- instrumentation entry points of the dspark library.
 *
 * Not part of the draft -> schedule -> verify contract of dspark.h: these calls
 * exist so that a benchmark can time the library's kernels on the stream they
 * are launched on, so that a test can read the device's random draws, and for
 * the debug build's checks.  They follow dspark.h's conventions (device
 * pointers, caller-owned buffers, no allocation, asynchronous on `stream`,
 * validation before any launch), except where a call says it synchronises.
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
 *                              (bf16 or fp32 logits, bf16 factors, r = 256, B <= 256, a
 *                              device that launches cooperatively; not under
 *                              stream capture, not for the RNN head).
 * dspark_draft takes DSPARK_DRAFT_AUTO: the persistent schedule where it applies
 * and B <= 192 (bf16 logits) or B <= 256 (fp32 logits), else the per-position
 * one (the measured crossovers). */
enum {
  DSPARK_DRAFT_AUTO = 0,
  DSPARK_DRAFT_PER_POSITION = 1,
  DSPARK_DRAFT_PERSISTENT = 2
};

/*
 * dspark_draft_timed -- dspark_draft with a chosen schedule and optional
 * timing.  `path` is one of the DSPARK_DRAFT_* values above.  `events` holds
 * n_events caller-created HIP events, recorded on `stream`:
 *   n_events = 0 (events NULL): no timing;
 *   n_events = 2: events[0] / events[1] immediately before the first and after
 *     the last kernel of the K-position draft phase, before the confidence head;
 *   n_events = 2 + 2K: as for 2, and events[2 + 2i] / events[3 + 2i] around the
 *     i-th launch of the phase's stream kernel: on the per-position schedule
 *     position i + 1's (i = 0..K-1); on the persistent schedule its one launch
 *     (i = 0), the later ones recorded right after it.
 * The caller reads the intervals with hipEventElapsedTime.  Same inputs,
 * outputs and errors as dspark_draft, plus DSPARK_E_INVALID for an unknown
 * `path` or event count and DSPARK_E_UNSUPPORTED for DSPARK_DRAFT_PERSISTENT
 * where it does not apply.
 */
dspark_status dspark_draft_timed(const dspark_problem* P,
                                 const void* Z, const void* E, const void* Wt, const void* h,
                                 const float* w_conf, float b_conf, const float* tau,
                                 const int32_t* anchor,
                                 int32_t* draft_tok, float* draft_logq, float* draft_lse,
                                 float* conf, float* surv,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream,
                                 hipEvent_t* events, int32_t n_events, int32_t path);

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

/*
 * Debug checks.  The library built with DSPARK_DEBUG_CHECKS (libdspark_debug.so)
 * scans every call's inputs before its kernels and its outputs after them with
 * kernels of its own, on `stream`, and raises bits of a per-device flag word
 * (never a trap; the call's results are those of the ordinary library, which
 * these scans do not touch):
 *   DSPARK_DEBUG_LOGITS          a non-finite base or target logit (NaN or infinity)
 *   DSPARK_DEBUG_FACTORS         a non-finite entry of E, Wt, h or w_conf, or a tau
 *                                outside (0, FLT_MAX]
 *   DSPARK_DEBUG_IDS             an anchor or draft token outside [0, V)
 *   DSPARK_DEBUG_SCHEDULE_INPUT  a survival outside [0, 1], a step-time entry not
 *                                positive and finite, or an n_sched outside [0, K]
 *   DSPARK_DEBUG_OUTPUT          an output outside its documented range (a token
 *                                outside [0, V), log q > 0, a confidence or survival
 *                                outside [0, 1], an n_sched outside [0, K] or an
 *                                n_total other than B plus their sum, an accepted length above the
 *                                schedule, a residual mass outside [0, 1])
 *   DSPARK_DEBUG_BARRIER_TIMEOUT a grid-barrier wait of the persistent draft gave up
 *                                (its results are then unspecified)
 * dspark.h leaves calls on inputs that break its contract undefined; these flags
 * report them.  The ordinary library returns DSPARK_E_UNSUPPORTED from both calls.
 */
enum {
  DSPARK_DEBUG_LOGITS = 1,
  DSPARK_DEBUG_FACTORS = 2,
  DSPARK_DEBUG_IDS = 4,
  DSPARK_DEBUG_SCHEDULE_INPUT = 8,
  DSPARK_DEBUG_OUTPUT = 16,
  DSPARK_DEBUG_BARRIER_TIMEOUT = 32
};

/*
 * dspark_debug_flags -- synchronises the current device, stores its flag word in
 * *flags and, if `clear` is non-zero, resets it.  DSPARK_E_POINTER if flags is
 * NULL.
 */
dspark_status dspark_debug_flags(uint32_t* flags, int32_t clear);

/*
 * dspark_debug_check_inputs -- the input scans alone, no other kernel: Z
 * [B][K][V] and target [B][K+1][V] (logits dtype, 16-byte aligned) for
 * non-finite logits, anchor [B] for ids outside [0, V), T_table [B*(K+1)+1] for
 * entries not positive and finite.  Any of the four may be NULL (not scanned).
 * Problem errors as dspark_draft.
 */
dspark_status dspark_debug_check_inputs(const dspark_problem* P, const void* Z, const void* target,
                                        const int32_t* anchor, const float* T_table, hipStream_t stream);

/*
 * dspark_debug_force_barrier_timeout -- with on != 0, every later persistent
 * draft of this process makes its grid-barrier waits unreachable and bounded by
 * a few polls, so that each wait gives up, sets the time-out flag and every
 * workgroup still runs to the end (the draft's results are then unspecified and
 * DSPARK_DEBUG_BARRIER_TIMEOUT is raised); on == 0 restores normal waits.  A
 * test of the bounded-wait path; debug build only.
 */
dspark_status dspark_debug_force_barrier_timeout(int32_t on);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_INSTR_H */
