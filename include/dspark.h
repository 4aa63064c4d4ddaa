/*
 * dspark.h -- C ABI of the per-cycle draft -> schedule -> verify step of
 * confidence-scheduled speculative decoding with a Markov draft head, for
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one of the DSpark summary page ("DSpark: semi-autoregressive
 * generation and confidence-scheduled verification", juhoplayground.github.io):
 *
 *   dspark_draft    -- Method > Semi-autoregressive generation (Markov head:
 *                      rank-r transition bias added to the backbone's base
 *                      logits, tokens sampled position after position) and
 *                      Method > Confidence-scheduled verification (confidence
 *                      head, Sequential Temperature Scaling, prefix survival);
 *   dspark_schedule_fixed, dspark_schedule_threshold -- Main results (the
 *                     fixed-length and static-threshold baselines)
 *   dspark_draft_rnn, dspark_verify_rnn -- Method > Semi-autoregressive
 *                      generation (the RNN head as the sequential block)
 *   dspark_sts_fit  -- Method > Confidence-scheduled verification (fitting the
 *                      STS temperatures left to right by grid search on ECE)
 *   dspark_schedule_async -- Production deployment results (asynchronous
 *                     dynamic top-k budget)
 *   dspark_schedule -- Method > Confidence-scheduled verification (hardware-aware
 *                      prefix scheduler against a step-time table profiled once
 *                      at start-up; greedy in survival order, stopping at the
 *                      first drop in throughput so that it never looks ahead);
 *   dspark_verify   -- Overview / Background (lossless rejection-sampling
 *                      verification of the scheduled prefix, left to right).
 *
 * Notation: B requests, K draft positions (k = 1..K, 1-based in the text,
 * 0-based in memory), V vocabulary entries, r Markov rank, d hidden size,
 * T_s the sampling temperature.  Token x_0 of request b is anchor[b]; row k of
 * Z predicts x_k.
 *
 * Conventions common to every entry point
 * ---------------------------------------
 * - All array arguments are DEVICE pointers on the current HIP device, dense
 *   and row-major as documented per argument; the problem struct is a HOST
 *   pointer.  The caller owns every buffer (inputs, outputs, workspace); the
 *   library allocates, frees and synchronises nothing and keeps no state
 *   between calls, so calls can be captured in a HIP graph.  Work is enqueued
 *   on `stream` (NULL = the default stream) and is asynchronous.
 * - dspark_draft runs one of two schedules of the same computation
 *   (dspark_instr.h): outside capture, for small batches, one cooperative
 *   launch over all K positions; under capture, and otherwise, a launch per
 *   position.  Tokens agree between them except at near-ties; log q and the
 *   log-partitions agree up to fp32 summation order (a few ulps).  Results are
 *   bit-reproducible for a given schedule.
 * - Logit, weight and hidden arrays must be 16-byte aligned; int32/float
 *   arrays 4-byte aligned.
 * - Validation runs on the host before anything is enqueued and returns a
 *   non-OK status without touching any buffer.  DSPARK_E_LAUNCH means a kernel
 *   launch was rejected by the runtime; faults inside kernels surface at the
 *   caller's next synchronisation.  Outputs are unspecified after a non-OK
 *   status.
 * - Randomness: Philox4x32-10 (Salmon et al., SC'11) with key
 *   (seed & 0xffffffff, seed >> 32) and counter (idx >> 2, b, k, purpose),
 *   taking output word idx & 3, where b is the 0-based request, k the 1-based
 *   position and idx a chunk id, a vocabulary id, or 0.  A word w becomes the
 *   uniform ((w >> 8) | 1) * 2^-24 and the Gumbel -ln(-ln u).  Purposes:
 *   1/2 draft chunk/element, 3 accept, 4/5 residual chunk/element, 6/7 bonus
 *   chunk/element.  Tokens are drawn by two-level Gumbel-max over chunks of
 *   128 vocabulary entries: the chunk maximising (log chunk mass + chunk
 *   Gumbel), then the entry of that chunk maximising (log weight + entry
 *   Gumbel); ties go to the smallest id.  Results are therefore a pure
 *   function of (inputs, seed).
 * - Workspace: one buffer of at least dspark_workspace_bytes(P) bytes,
 *   256-byte aligned, shared by the three calls of a cycle (its contents need
 *   not be initialised and carry nothing between calls).
 *
 * Supported shapes: 1 <= B <= 65536, 1 <= K <= 64, 8 <= V < 2^31 with
 * V % 8 == 0, d >= 1 with d % 8 == 0, r in {16, 32, 64, 128, 256} for bf16
 * weights and {16, 32, 64} for fp32 weights; B*K <= 2^20.  Logits (Z and the
 * target) and h may be fp32 or bf16, independently; weights (E, Wt) fp32 or
 * bf16.  0 < T_s finite.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_E_INVALID = -1,      /* a size or scalar is out of range (B, K, V, d, T_s, ...) */
  DSPARK_E_DTYPE = -2,        /* a dtype code is not a dspark_dtype */
  DSPARK_E_UNSUPPORTED = -3,  /* valid, but no kernel is built for it (e.g. r = 48) */
  DSPARK_E_WORKSPACE = -4,    /* workspace null, misaligned or smaller than required */
  DSPARK_E_LAUNCH = -5,       /* the runtime rejected a kernel launch */
  DSPARK_E_POINTER = -6       /* a required pointer is null or misaligned (appended after the five codes above) */
} dspark_status;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

typedef struct {
  int32_t B, K, V, r, d;
  int32_t logits_dtype;   /* dspark_dtype of Z and of the target logits */
  int32_t weight_dtype;   /* dspark_dtype of E and Wt */
  int32_t hidden_dtype;   /* dspark_dtype of h */
  float sampling_temp;    /* T_s: q = softmax((Z + bias) / T_s), p = softmax(target / T_s) */
  uint64_t seed;          /* Philox key */
} dspark_problem;

/* Bytes of workspace the three calls need for problem P; 0 if P is invalid.
 * Host-only: makes no HIP call. */
size_t dspark_workspace_bytes(const dspark_problem* P);

/* Static, NUL-terminated description of a status code.  Takes an int so that a
 * code read back as an integer (from another language, or out of range) is
 * accepted; values that are not a dspark_status give "unknown status". */
const char* dspark_status_string(int status);

/*
 * dspark_draft -- sequential Markov-head sampling of K draft tokens per
 * request, then the confidence head and prefix survival.
 *
 * For k = 1..K, with prev = x_{k-1} (the anchor for k = 1):
 *   ell_v  = (Z[b][k-1][v] + sum_j E[prev][j] * Wt[v][j]) / T_s
 *   x_k    = two-level Gumbel-max draw from softmax(ell) (purposes 1/2)
 *   lse    = log sum_v exp(ell_v);  logq = ell_{x_k} - lse
 * then z = w_conf[0:d] . h[b][k-1] + w_conf[d:d+r] . E[x_{k-1}] + b_conf,
 *   conf = sigmoid(z / tau[k-1]),  surv[b][k-1] = prod_{j<=k} conf[b][j-1].
 *
 * Inputs:  Z [B][K][V] (logits_dtype); E [V][r], Wt [V][r] (weight_dtype;
 *          Wt is the logit projection stored vocabulary-major);
 *          h [B][K][d] (hidden_dtype); w_conf [d + r] fp32; tau [K] fp32 (> 0);
 *          anchor [B] int32 in [0, V).
 * Outputs: draft_tok [B][K] int32; draft_logq, draft_lse, conf, surv [B][K] fp32
 *          (logq and lse in nats of ell).
 * Token ids outside [0, V) in anchor are undefined behaviour.
 */
dspark_status dspark_draft(const dspark_problem* P,
                           const void* Z, const void* E, const void* Wt, const void* h,
                           const float* w_conf, float b_conf, const float* tau,
                           const int32_t* anchor,
                           int32_t* draft_tok, float* draft_logq, float* draft_lse,
                           float* conf, float* surv,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_schedule -- choose n_b, the number of draft positions of request b to
 * verify.  Candidates (s = surv[b][k-1], b, k) are taken in the order (s
 * descending, b ascending, k ascending) starting from A = B expected tokens at
 * N = B verified positions; a candidate is taken iff
 *   (A + s) * T_table[N] >= A * T_table[N + 1]   (then A += s, N += 1),
 * and the pass stops at the first candidate refused.
 *
 * Inputs:  surv [B][K] fp32, each row non-increasing (as written by
 *          dspark_draft; other rows give unspecified but in-bounds results);
 *          T_table [B*(K+1) + 1] fp32, the step time with N verified positions
 *          (any positive unit; only ratios matter).
 * Outputs: n_sched [B] int32 in [0, K]; n_total [1] int32 = B + sum_b n_sched[b].
 */
dspark_status dspark_schedule(const dspark_problem* P,
                              const float* surv, const float* T_table,
                              int32_t* n_sched, int32_t* n_total,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_schedule_noalloc -- dspark_schedule for callers that cannot allocate
 * (code under HIP graph capture that may not call hipMalloc, tight serving
 * loops, harnesses that forbid allocation): the same schedule, bit for bit,
 * with no workspace argument.  Its scratch (partial ranks and the candidates in
 * schedule order) is a static device array inside the library, 2.25 MiB per
 * GPU, held until the process ends; the call itself allocates nothing.
 *
 * Limit: B * K <= 32768 candidates; larger problems return DSPARK_E_WORKSPACE
 * (use dspark_schedule with a workspace).  Every call on one GPU shares that
 * GPU's scratch, so calls that overlap on one GPU (concurrent streams, or
 * threads issuing to different streams) race and give unspecified results;
 * calls ordered on one stream, or separated by synchronisation, do not.
 * Other arguments, outputs and errors as for dspark_schedule; DSPARK_E_LAUNCH
 * also when the scratch's device address cannot be obtained.
 */
dspark_status dspark_schedule_noalloc(const dspark_problem* P,
                                      const float* surv, const float* T_table,
                                      int32_t* n_sched, int32_t* n_total, hipStream_t stream);

/*
 * dspark_schedule_async -- the asynchronous "dynamic top-k" form of the
 * scheduler (DSpark page, Production deployment results): the verification
 * budget is sized from the confidence-head outputs of two steps earlier and
 * filled with the current step's candidates in order of their latest
 * cumulative confidence, so that the budget can be fixed ahead of the step
 * (graph replay, overlapped scheduling).
 *
 * M = the number of candidates dspark_schedule would take on surv_lag (same
 * table, same rule); then the first M current candidates in the order (surv
 * descending, b ascending, k ascending) are taken.  Within a request a later
 * position never precedes an earlier one, so each n_b is a prefix length and
 * does not depend on the request's confidences beyond it.
 *
 * Inputs:  surv_lag [B][K] fp32, the survivals of two steps earlier (rows
 *          non-increasing); surv [B][K] fp32, the current survivals (rows
 *          non-increasing); T_table as for dspark_schedule.
 * Outputs: n_sched [B] int32; n_total [1] int32 = B + M.
 * Same errors as dspark_schedule; the workspace is used as scratch.
 */
dspark_status dspark_schedule_async(const dspark_problem* P,
                                    const float* surv_lag, const float* surv, const float* T_table,
                                    int32_t* n_sched, int32_t* n_total,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_schedule_fixed / dspark_schedule_threshold -- the verification
 * baselines the scheduler is compared against (DSpark page, Main results:
 * offline benchmark with fixed-length blocks; static threshold sweep over the
 * confidence head).
 *
 * fixed:     n_b = gamma for every request (0 <= gamma <= K).
 * threshold: n_b = the longest prefix of positions with surv[b][k-1] >= theta
 *            (theta finite; fp32 comparison).
 * Outputs:   n_sched [B] int32; n_total [1] int32 = B + sum_b n_b.
 * No workspace.  DSPARK_E_INVALID for gamma outside [0, K] or a non-finite theta;
 * DSPARK_E_POINTER for NULL or misaligned (4-byte) pointers.
 */
dspark_status dspark_schedule_fixed(const dspark_problem* P, int32_t gamma,
                                    int32_t* n_sched, int32_t* n_total, hipStream_t stream);
dspark_status dspark_schedule_threshold(const dspark_problem* P, const float* surv, float theta,
                                        int32_t* n_sched, int32_t* n_total, hipStream_t stream);

/*
 * dspark_rnn_workspace_bytes / dspark_draft_rnn / dspark_verify_rnn -- the RNN
 * head as the sequential block (Method > Semi-autoregressive generation: the
 * second sequential block keeps a recurrent state over the whole drafted prefix
 * and applies a gated update from the current state, the previous token's
 * embedding and the backbone hidden state; Main results: small gains over the
 * Markov head at long draft lengths).
 *
 * The gated update is a GRU cell (gate order reset, update, new; the reset gate
 * scales the recurrent product of the new gate), with input u_k = [h_k; E[x_{k-1}]]:
 *   a = W_ih u_k + b_ih,  c = W_hh s_{k-1} + b_hh,  s_0 = 0,
 *   rho = sigmoid(a_r + c_r), z = sigmoid(a_z + c_z), n = tanh(a_n + rho * c_n),
 *   s_k = (1 - z) * n + z * s_{k-1};
 * bf16(s_k) (round to nearest even) replaces E[x_{k-1}] as the operand of the
 * logit projection at position k, in the draft and in the resample of the
 * verification.  Everything else is dspark_draft / dspark_verify: the same
 * sampling, randomness, confidence head (inputs [h_k; E[x_{k-1}]]), outputs
 * and errors.
 *
 *   W_ih  [3r][d + r] bf16   input weights (columns 0..d-1 act on h_k, d.. on E[x_{k-1}])
 *   b_ih  [3r] float32
 *   W_hh  [3r][r] bf16        recurrent weights
 *   b_hh  [3r] float32
 *   state [B][K][r] float32   draft: out, s_k of every position; verify: in (the draft's)
 * Supported for bf16 logits, factors and hidden states with r a multiple of 32,
 * within the sizes the fragment-fed kernels address (DSPARK_E_UNSUPPORTED
 * otherwise).  Workspace: at least dspark_rnn_workspace_bytes(P) for the draft
 * (the draft's regions plus the hidden-state part of the input gates for all
 * B*K positions); the verification needs dspark_workspace_bytes(P).
 */
size_t dspark_rnn_workspace_bytes(const dspark_problem* P);
dspark_status dspark_draft_rnn(const dspark_problem* P, const void* Z, const void* E, const void* Wt, const void* h,
                               const void* W_ih, const float* b_ih, const void* W_hh, const float* b_hh,
                               const float* w_conf, float b_conf, const float* tau, const int32_t* anchor,
                               int32_t* draft_tok, float* draft_logq, float* draft_lse, float* conf, float* surv,
                               float* state, void* workspace, size_t workspace_bytes, hipStream_t stream);
dspark_status dspark_verify_rnn(const dspark_problem* P, const void* target, const void* Z, const void* E,
                                const void* Wt, const int32_t* anchor, const int32_t* draft_tok,
                                const float* draft_logq, const float* draft_lse, const float* state,
                                const int32_t* n_sched, int32_t* out_tok, int32_t* n_accepted, int32_t* next_anchor,
                                float* logp, float* resid_mass, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * dspark_sts_workspace_bytes / dspark_sts_fit -- fitting the Sequential
 * Temperature Scaling temperatures (Method > Confidence-scheduled verification,
 * the STS paragraph; Main results for the calibration it reaches).
 *
 * Left to right over the K positions, with the temperatures of earlier
 * positions fixed, a one-dimensional search over the caller's grid picks the
 * temperature tau_k that minimises the Expected Calibration Error of the
 * survival S_k = S_{k-1} * sigmoid(logit(c_k) / tau_k) (logit(c) = ln c - ln(1-c),
 * S_0 = 1) against the label "accepted length >= k", over the samples that
 * verified position k (k <= n_verified[m]).  ECE uses n_bins equal-width bins
 * on [0, 1] (bin = min(floor(p * n_bins), n_bins - 1)):
 *   ECE = sum over bins |sum of predictions - accepted count| / observed count.
 * Arithmetic is float64.  Grid entries that are not finite and positive are
 * never chosen; ties go to the smallest index.  A position with no observed
 * sample, or no usable grid entry, keeps tau = 1 with tau_idx = -1 and a NaN
 * ece_fit (ece_raw is NaN only when nothing is observed).
 *
 *   conf_raw   [M][K] float32  raw confidences (the head at temperature 1), in [0, 1]
 *   acc_len    [M] int32       accepted drafts of each sample (0..n_verified)
 *   n_verified [M] int32       drafts each sample verified (0..K)
 *   tau_grid   [G] float64     candidate temperatures
 *   tau        [K] float64     out: fitted temperatures
 *   tau_idx    [K] int32       out: their grid indices (-1: kept at 1)
 *   ece_fit    [K] float64     out: ECE of the fitted survival
 *   ece_raw    [K] float64     out: ECE of the raw survival (every tau = 1)
 * Limits: 0 <= M <= 2^24, 1 <= K <= 1024, 1 <= G <= 4096, 1 <= n_bins <= 16
 * (DSPARK_E_INVALID otherwise; the workspace size is then 0).  Float64 arrays
 * 8-byte aligned, the others 4-byte (DSPARK_E_POINTER).  Workspace as for the
 * other entry points, at least dspark_sts_workspace_bytes(M, K, G, n_bins).
 */
size_t dspark_sts_workspace_bytes(int32_t M, int32_t K, int32_t G, int32_t n_bins);
dspark_status dspark_sts_fit(int32_t M, int32_t K, const float* conf_raw, const int32_t* acc_len,
                             const int32_t* n_verified, const double* tau_grid, int32_t G, int32_t n_bins,
                             double* tau, int32_t* tau_idx, double* ece_fit, double* ece_raw,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_verify -- lossless rejection-sampling verification.
 *
 * With p_k = softmax(target[b][k-1] / T_s) and q_k the draft distribution of
 * position k (recomputed from Z, E, Wt and draft_lse), for k = 1..n_b in order:
 * accept x_k iff u <= min(1, p_k(x_k) / q_k(x_k)) with u the accept draw
 * (purpose 3).  At the first rejection k*, emit y drawn from max(0, p_k* - q_k*)
 * (purposes 4/5 at position k*; from p_k* if that mass is exactly 0) and keep
 * x_1..x_{k*-1}; if all n_b are accepted, emit y drawn from p_{n_b+1}
 * (purposes 6/7 at position n_b + 1) and keep x_1..x_{n_b}.
 *
 * Inputs:  target [B][K+1][V] (logits_dtype); Z, E, Wt, anchor as for
 *          dspark_draft; draft_tok, draft_logq, draft_lse [B][K] as written by
 *          dspark_draft; n_sched [B] in [0, K].
 * Outputs: out_tok [B][K+1] int32: x_1..x_a, y, then -1;
 *          n_accepted [B] int32 (a); next_anchor [B] int32 (y);
 *          logp [B][K] fp32: log p_k(x_k) for k <= n_b, NaN beyond;
 *          resid_mass [B] fp32: sum_v max(0, p_k* - q_k*) at a rejection, NaN
 *          when the bonus path was taken.
 */
dspark_status dspark_verify(const dspark_problem* P,
                            const void* target, const void* Z, const void* E, const void* Wt,
                            const int32_t* anchor, const int32_t* draft_tok,
                            const float* draft_logq, const float* draft_lse,
                            const int32_t* n_sched,
                            int32_t* out_tok, int32_t* n_accepted, int32_t* next_anchor,
                            float* logp, float* resid_mass,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
