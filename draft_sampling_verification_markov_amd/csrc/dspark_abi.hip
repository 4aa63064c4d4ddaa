// C ABI of the dspark library: argument validation, workspace layout and the
// kernel sequence of each call.  See include/dspark.h for the contract.
#include <math.h>

#include <float.h>

#include <mutex>

#include "dspark_internal.hpp"

namespace dspark {

// The library built with DSPARK_DEBUG_CHECKS scans every call's inputs before
// its kernels and its outputs after them (k_debug.hip); the scans raise bits of
// the flag word that dspark_debug_flags reads.  Compiled in both builds, run
// only in that one.
#ifdef DSPARK_DEBUG_CHECKS
constexpr bool kDebugChecks = true;
#else
constexpr bool kDebugChecks = false;
#endif
// debug build: the persistent draft's barrier waits are made to time out
// (dspark_debug_force_barrier_timeout), to exercise the bounded-wait path
static bool g_debug_force_timeout = false;

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

Layout make_layout(const dspark_problem& P) {
  Layout L{};
  const size_t B = (size_t)P.B, K = (size_t)P.K;
  L.G = stream_grid(P.V);
  L.nseg = vlse_segments(P.V);
  size_t off = 0;
  // per-(row, workgroup) partials of the per-position launches or of the persistent one
  const size_t gmax = (size_t)(L.G > persist_grid(P.V) ? L.G : persist_grid(P.V));
  L.part = off;   off = align_up(off + B * gmax * sizeof(float4));
  L.zpart = off;  off = align_up(off + B * L.G * sizeof(float2));
  L.vlse = off;   off = align_up(off + B * K * L.nseg * sizeof(float2));
  L.lsep = off;   off = align_up(off + B * K * sizeof(float));
  L.job = off;    off = align_up(off + B * sizeof(int32_t));
  L.rows = off;   off = align_up(off + B * K * sizeof(int32_t));
  L.nrows = off;  off = align_up(off + sizeof(int32_t));
  L.rpart = off;  off = align_up(off + (size_t)sched_segments((int)(B * K)) * B * K * sizeof(int32_t));
  L.sorts = off;  off = align_up(off + B * K * sizeof(float));
  L.sorti = off;  off = align_up(off + B * K * sizeof(int32_t));
  L.lagn = off;   off = align_up(off + (B + 1) * sizeof(int32_t));
  L.efrag = off;  off = align_up(off + (size_t)((B + 31) / 32) * 32 * (size_t)P.r * 2);
  L.prec = off;   off = align_up(off + (B <= (size_t)kPersistMaxB ? B * (size_t)persist_grid(P.V) * 32 : 0));
  L.ptok = off;   off = align_up(off + (size_t)kSyncGroups * kTokRepSlots * sizeof(unsigned long long));
  L.psync = off;  off = align_up(off + kPersistSyncWords * sizeof(uint32_t));
  L.total = off;
  return L;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static dspark_status check_problem(const dspark_problem* P) {
  if (!P) return DSPARK_E_POINTER;
  if (P->B < 1 || P->B > 65536 || P->K < 1 || P->K > 64) return DSPARK_E_INVALID;
  if (P->V < 8 || P->V % 8 != 0) return DSPARK_E_INVALID;
  if (P->d < 1 || P->d % 8 != 0 || P->r < 1) return DSPARK_E_INVALID;
  if ((long long)P->B * P->K > (1LL << 20)) return DSPARK_E_INVALID;
  if (!(P->sampling_temp > 0.0f) || !isfinite(P->sampling_temp)) return DSPARK_E_INVALID;
  for (int32_t t : {P->logits_dtype, P->weight_dtype, P->hidden_dtype})
    if (t != DSPARK_F32 && t != DSPARK_BF16) return DSPARK_E_DTYPE;
  const int r = P->r;
  if (P->weight_dtype == DSPARK_BF16) {
    if (r != 16 && r != 32 && r != 64 && r != 128 && r != 256) return DSPARK_E_UNSUPPORTED;
  } else {
    if (r != 16 && r != 32 && r != 64) return DSPARK_E_UNSUPPORTED;
  }
  return DSPARK_OK;
}

static dspark_status check_workspace(const dspark_problem& P, void* ws, size_t bytes) {
  if (!ws || !aligned(ws, 256)) return DSPARK_E_WORKSPACE;
  if (bytes < make_layout(P).total) return DSPARK_E_WORKSPACE;
  return DSPARK_OK;
}

template <typename T>
static T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

static Key host_key(uint64_t seed) { return Key{(uint32_t)seed, (uint32_t)(seed >> 32)}; }

}  // namespace dspark

using namespace dspark;

extern "C" size_t dspark_workspace_bytes(const dspark_problem* P) {
  if (check_problem(P) != DSPARK_OK) return 0;
  return make_layout(*P).total;
}

extern "C" const char* dspark_status_string(int status) {
  switch (status) {
    case DSPARK_OK: return "ok";
    case DSPARK_E_INVALID: return "invalid problem size or scalar argument";
    case DSPARK_E_DTYPE: return "unknown dtype code";
    case DSPARK_E_UNSUPPORTED: return "unsupported configuration (no kernel built for it)";
    case DSPARK_E_WORKSPACE: return "workspace null, misaligned or too small";
    case DSPARK_E_POINTER: return "null or misaligned pointer argument";
    case DSPARK_E_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

// The RNN head's weights and its state output (absent for the Markov head).
struct RnnDraft {
  const void* W_ih;
  const float* b_ih;
  const void* W_hh;
  const float* b_hh;
  float* state;
};

// Debug scans (run only with kDebugChecks): false if a scan could not be launched.
static bool debug_draft_inputs(const dspark_problem& p, const void* Z, const void* E, const void* Wt, const void* h,
                               const float* w_conf, const float* tau, const int32_t* anchor, hipStream_t s) {
  const bool zb = p.logits_dtype == DSPARK_BF16, wb = p.weight_dtype == DSPARK_BF16, hb = p.hidden_dtype == DSPARK_BF16;
  return debug_scan_nonfinite(Z, (size_t)p.B * p.K * p.V, zb, DSPARK_DEBUG_LOGITS, s) == hipSuccess &&
         debug_scan_nonfinite(E, (size_t)p.V * p.r, wb, DSPARK_DEBUG_FACTORS, s) == hipSuccess &&
         debug_scan_nonfinite(Wt, (size_t)p.V * p.r, wb, DSPARK_DEBUG_FACTORS, s) == hipSuccess &&
         debug_scan_nonfinite(h, (size_t)p.B * p.K * p.d, hb, DSPARK_DEBUG_FACTORS, s) == hipSuccess &&
         debug_scan_nonfinite(w_conf, (size_t)(p.d + p.r), false, DSPARK_DEBUG_FACTORS, s) == hipSuccess &&
         debug_scan_range_f32(tau, (size_t)p.K, FLT_MIN, FLT_MAX, DSPARK_DEBUG_FACTORS, s) == hipSuccess &&
         debug_scan_range_i32(anchor, (size_t)p.B, 0, p.V - 1, DSPARK_DEBUG_IDS, s) == hipSuccess;
}
static bool debug_draft_outputs(const dspark_problem& p, const int32_t* tok, const float* logq, const float* conf,
                                const float* surv, hipStream_t s) {
  const size_t n = (size_t)p.B * p.K;
  return debug_scan_range_i32(tok, n, 0, p.V - 1, DSPARK_DEBUG_OUTPUT, s) == hipSuccess &&
         debug_scan_range_f32(logq, n, -FLT_MAX, 1e-5f, DSPARK_DEBUG_OUTPUT, s) == hipSuccess &&
         debug_scan_range_f32(conf, n, 0.f, 1.f, DSPARK_DEBUG_OUTPUT, s) == hipSuccess &&
         debug_scan_range_f32(surv, n, 0.f, 1.f, DSPARK_DEBUG_OUTPUT, s) == hipSuccess;
}
static bool debug_schedule_inputs(const dspark_problem& p, const float* surv, const float* T_table, hipStream_t s) {
  const size_t n = (size_t)p.B * p.K;
  return (!surv || debug_scan_range_f32(surv, n, 0.f, 1.f, DSPARK_DEBUG_SCHEDULE_INPUT, s) == hipSuccess) &&
         (!T_table ||
          debug_scan_range_f32(T_table, n + (size_t)p.B + 1, FLT_MIN, FLT_MAX, DSPARK_DEBUG_SCHEDULE_INPUT, s) ==
              hipSuccess);
}
static bool debug_verify_inputs(const dspark_problem& p, const void* target, const void* Z, const void* E,
                                const void* Wt, const int32_t* anchor, const int32_t* tok, const int32_t* n_sched,
                                hipStream_t s) {
  const bool zb = p.logits_dtype == DSPARK_BF16, wb = p.weight_dtype == DSPARK_BF16;
  return debug_scan_nonfinite(target, (size_t)p.B * (p.K + 1) * p.V, zb, DSPARK_DEBUG_LOGITS, s) == hipSuccess &&
         debug_scan_nonfinite(Z, (size_t)p.B * p.K * p.V, zb, DSPARK_DEBUG_LOGITS, s) == hipSuccess &&
         debug_scan_nonfinite(E, (size_t)p.V * p.r, wb, DSPARK_DEBUG_FACTORS, s) == hipSuccess &&
         debug_scan_nonfinite(Wt, (size_t)p.V * p.r, wb, DSPARK_DEBUG_FACTORS, s) == hipSuccess &&
         debug_scan_range_i32(anchor, (size_t)p.B, 0, p.V - 1, DSPARK_DEBUG_IDS, s) == hipSuccess &&
         debug_scan_range_i32(tok, (size_t)p.B * p.K, 0, p.V - 1, DSPARK_DEBUG_IDS, s) == hipSuccess &&
         debug_scan_range_i32(n_sched, (size_t)p.B, 0, p.K, DSPARK_DEBUG_SCHEDULE_INPUT, s) == hipSuccess;
}

static dspark_status draft_impl(const dspark_problem* P, const void* Z, const void* E, const void* Wt,
                                const void* h, const float* w_conf, float b_conf, const float* tau,
                                const int32_t* anchor, int32_t* draft_tok, float* draft_logq, float* draft_lse,
                                float* conf, float* surv, void* workspace, size_t workspace_bytes,
                                hipStream_t stream, hipEvent_t* events, const RnnDraft* rnn = nullptr,
                                int32_t path = DSPARK_DRAFT_AUTO, int32_t n_events = 0) {
  // timing events: events[0] / events[1] around the draft phase; with 2 + 2K,
  // events[2 + 2i] / events[3 + 2i] around the i-th launch of its stream kernel
  const bool per_launch = events && n_events >= 2 + 2 * (P ? P->K : 0);
  dspark_status st = check_problem(P);
  if (st != DSPARK_OK) return st;
  const dspark_problem& p = *P;
  if (rnn) {
    if (!rnn_supported(p)) return DSPARK_E_UNSUPPORTED;
    if (!rnn->W_ih || !rnn->b_ih || !rnn->W_hh || !rnn->b_hh || !rnn->state) return DSPARK_E_POINTER;
    if (!aligned(rnn->W_ih, 16) || !aligned(rnn->W_hh, 16) || !aligned(rnn->state, 16) || !aligned(rnn->b_ih, 4) ||
        !aligned(rnn->b_hh, 4))
      return DSPARK_E_POINTER;
  }
  if (!Z || !E || !Wt || !h || !w_conf || !tau || !anchor || !draft_tok || !draft_logq || !draft_lse || !conf ||
      !surv)
    return DSPARK_E_POINTER;
  for (const void* q : {Z, E, Wt, h, (const void*)w_conf})
    if (!aligned(q, 16)) return DSPARK_E_POINTER;
  for (const void* q : {(const void*)tau, (const void*)anchor, (const void*)draft_tok, (const void*)draft_logq,
                        (const void*)draft_lse, (const void*)conf, (const void*)surv})
    if (!aligned(q, 4)) return DSPARK_E_POINTER;
  st = check_workspace(p, workspace, workspace_bytes);
  if (st != DSPARK_OK) return st;
  if (rnn && workspace_bytes < make_layout(p).total + rnn_extra_bytes(p)) return DSPARK_E_WORKSPACE;
  (void)hipGetLastError();
  if (kDebugChecks && !debug_draft_inputs(p, Z, E, Wt, h, w_conf, tau, anchor, stream)) return DSPARK_E_LAUNCH;

  const Layout L = make_layout(p);
  float4* part = at<float4>(workspace, L.part);
  StreamArgs sa{};
  sa.Z = Z;
  sa.E = E;
  sa.Wt = Wt;
  sa.anchor = anchor;
  sa.tok = draft_tok;
  sa.part = part;
  sa.B = p.B;
  sa.K = p.K;
  sa.V = p.V;
  sa.nchunks = n_chunks(p.V);
  sa.scale2 = kLog2e / p.sampling_temp;
  sa.key = host_key(p.seed);
  uint4* const efrag = at<uint4>(workspace, L.efrag);
  const bool use_efrag = draft_uses_efrag(p);
  sa.efrag = efrag;

  SelectArgs se{};
  se.Z = Z;
  se.E = E;
  se.Wt = Wt;
  se.anchor = anchor;
  se.tok = draft_tok;
  se.logq = draft_logq;
  se.lse = draft_lse;
  se.part = part;
  se.B = p.B;
  se.K = p.K;
  se.V = p.V;
  se.r = p.r;
  se.G = L.G;
  se.inv_T = 1.0f / p.sampling_temp;
  se.key = sa.key;

  // the persistent kernel is a cooperative launch; under stream capture the
  // per-position kernels are recorded instead
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &capture) != hipSuccess) capture = hipStreamCaptureStatusActive;
  (void)hipGetLastError();
  const bool persist_ok = !rnn && capture == hipStreamCaptureStatusNone && draft_persistent_supported(p);
  if (path == DSPARK_DRAFT_PERSISTENT && !persist_ok) return DSPARK_E_UNSUPPORTED;
  if (path == DSPARK_DRAFT_PERSISTENT || (path == DSPARK_DRAFT_AUTO && persist_ok && p.B <= persist_max_b(p))) {
    // every position in one cooperative launch, Wt slices held on chip
    PersistArgs pa{};
    pa.Z = Z;
    pa.E = E;
    pa.Wt = Wt;
    pa.anchor = anchor;
    pa.tok = draft_tok;
    pa.logq = draft_logq;
    pa.lse = draft_lse;
    pa.rec = at<unsigned long long>(workspace, L.prec);
    pa.tokrep = at<unsigned long long>(workspace, L.ptok);
    pa.sync = at<unsigned>(workspace, L.psync);
    pa.B = p.B;
    pa.K = p.K;
    pa.V = p.V;
    pa.nchunks = n_chunks(p.V);
    pa.z_bytes = (uint32_t)((size_t)p.B * p.K * p.V * (p.logits_dtype == DSPARK_F32 ? 4 : 2));
    pa.spin_limit = kPersistSpinLimit;
    pa.unreachable = 0;
    if (kDebugChecks && g_debug_force_timeout) {  // every barrier wait times out after a few polls
      pa.spin_limit = 64;
      pa.unreachable = 1;
    }
    pa.scale2 = sa.scale2;
    pa.inv_T = se.inv_T;
    pa.key = sa.key;
    if (events && hipEventRecord(events[0], stream) != hipSuccess) return DSPARK_E_LAUNCH;
    if (per_launch && hipEventRecord(events[2], stream) != hipSuccess) return DSPARK_E_LAUNCH;
    if (launch_draft_persistent(p, pa, stream) != hipSuccess) return DSPARK_E_LAUNCH;
    // one launch: the other per-launch events all right after it
    if (per_launch)
      for (int i = 3; i < 2 + 2 * p.K; ++i)
        if (hipEventRecord(events[i], stream) != hipSuccess) return DSPARK_E_LAUNCH;
    // a barrier time-out (the flag word the kernel sets) raises its debug bit
    if (kDebugChecks && debug_scan_range_i32(reinterpret_cast<const int32_t*>(pa.sync) + (size_t)kSyncFlag * kSyncStride, 1, 0, 0,
                                             DSPARK_DEBUG_BARRIER_TIMEOUT, stream) != hipSuccess)
      return DSPARK_E_LAUNCH;
    if (events && hipEventRecord(events[1], stream) != hipSuccess) return DSPARK_E_LAUNCH;
  } else {
  float* Gh = rnn ? at<float>(workspace, L.total) : nullptr;
  if (rnn) {
    se.state = rnn->state;
    if (launch_rnn_gemm(p, h, rnn->W_ih, rnn->b_ih, Gh, stream) != hipSuccess) return DSPARK_E_LAUNCH;
  }
  for (int k = 1; k <= p.K; ++k) {
    sa.k = k;
    se.k = k;
    // Markov head: step 1 gathers the anchors' E rows itself
    sa.first_from_anchor = !rnn && use_efrag && k == 1;
    // Markov head: the select kernel stores the fragments of position k for step k + 1;
    // RNN head: the step kernel stores those of the state of position k before step k
    se.efrag = !rnn && use_efrag && k < p.K ? efrag : nullptr;
    if (rnn && launch_rnn_step(p, Gh, rnn->W_ih, rnn->W_hh, rnn->b_hh, E, anchor, draft_tok, rnn->state, efrag, k,
                               stream) != hipSuccess)
      return DSPARK_E_LAUNCH;
    if (events && k == 1 && hipEventRecord(events[0], stream) != hipSuccess) return DSPARK_E_LAUNCH;
    if (per_launch && hipEventRecord(events[2 * k], stream) != hipSuccess) return DSPARK_E_LAUNCH;
    if (launch_stream_draft(p, sa, L.G, stream) != hipSuccess) return DSPARK_E_LAUNCH;
    if (per_launch && hipEventRecord(events[2 * k + 1], stream) != hipSuccess) return DSPARK_E_LAUNCH;
    if (launch_select(p, se, stream) != hipSuccess) return DSPARK_E_LAUNCH;
    if (events && k == p.K && hipEventRecord(events[1], stream) != hipSuccess) return DSPARK_E_LAUNCH;
  }
  }

  ConfArgs ca{};
  ca.h = h;
  ca.E = E;
  ca.w_c = w_conf;
  ca.b_c = b_conf;
  ca.tau = tau;
  ca.anchor = anchor;
  ca.tok = draft_tok;
  ca.conf = conf;
  ca.surv = surv;
  ca.B = p.B;
  ca.K = p.K;
  ca.V = p.V;
  ca.d = p.d;
  ca.r = p.r;
  if (launch_conf(p, ca, stream) != hipSuccess) return DSPARK_E_LAUNCH;
  if (kDebugChecks && !debug_draft_outputs(p, draft_tok, draft_logq, conf, surv, stream)) return DSPARK_E_LAUNCH;
  return DSPARK_OK;
}

extern "C" dspark_status dspark_draft(const dspark_problem* P, const void* Z, const void* E, const void* Wt,
                                      const void* h, const float* w_conf, float b_conf, const float* tau,
                                      const int32_t* anchor, int32_t* draft_tok, float* draft_logq,
                                      float* draft_lse, float* conf, float* surv, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  const AbiRange range("dspark_draft");
  return draft_impl(P, Z, E, Wt, h, w_conf, b_conf, tau, anchor, draft_tok, draft_logq, draft_lse, conf, surv,
                    workspace, workspace_bytes, stream, nullptr);
}

extern "C" dspark_status dspark_draft_timed(const dspark_problem* P, const void* Z, const void* E, const void* Wt,
                                            const void* h, const float* w_conf, float b_conf, const float* tau,
                                            const int32_t* anchor, int32_t* draft_tok, float* draft_logq,
                                            float* draft_lse, float* conf, float* surv, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                                            int32_t n_events, int32_t path) {
  const AbiRange range("dspark_draft_timed");
  if (path != DSPARK_DRAFT_AUTO && path != DSPARK_DRAFT_PER_POSITION && path != DSPARK_DRAFT_PERSISTENT)
    return DSPARK_E_INVALID;
  if (!events ? n_events != 0 : (n_events != 2 && (!P || n_events != 2 + 2 * P->K))) return DSPARK_E_INVALID;
  return draft_impl(P, Z, E, Wt, h, w_conf, b_conf, tau, anchor, draft_tok, draft_logq, draft_lse, conf, surv,
                    workspace, workspace_bytes, stream, events, nullptr, path, n_events);
}

extern "C" int32_t dspark_draft_path(const dspark_problem* P) {
  const dspark_status st = check_problem(P);
  if (st != DSPARK_OK) return st;
  return draft_persistent_supported(*P) && P->B <= persist_max_b(*P) ? DSPARK_DRAFT_PERSISTENT : DSPARK_DRAFT_PER_POSITION;
}

extern "C" size_t dspark_rnn_workspace_bytes(const dspark_problem* P) {
  if (check_problem(P) != DSPARK_OK) return 0;
  return make_layout(*P).total + rnn_extra_bytes(*P);
}

extern "C" dspark_status dspark_draft_rnn(const dspark_problem* P, const void* Z, const void* E, const void* Wt,
                                          const void* h, const void* W_ih, const float* b_ih, const void* W_hh,
                                          const float* b_hh, const float* w_conf, float b_conf, const float* tau,
                                          const int32_t* anchor, int32_t* draft_tok, float* draft_logq,
                                          float* draft_lse, float* conf, float* surv, float* state, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  const AbiRange range("dspark_draft_rnn");
  const RnnDraft rnn{W_ih, b_ih, W_hh, b_hh, state};
  return draft_impl(P, Z, E, Wt, h, w_conf, b_conf, tau, anchor, draft_tok, draft_logq, draft_lse, conf, surv,
                    workspace, workspace_bytes, stream, nullptr, &rnn);
}

extern "C" dspark_status dspark_schedule(const dspark_problem* P, const float* surv, const float* T_table,
                                         int32_t* n_sched, int32_t* n_total, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  const AbiRange range("dspark_schedule");
  dspark_status st = check_problem(P);
  if (st != DSPARK_OK) return st;
  if (!surv || !T_table || !n_sched || !n_total) return DSPARK_E_POINTER;
  for (const void* q : {(const void*)surv, (const void*)T_table, (const void*)n_sched, (const void*)n_total})
    if (!aligned(q, 4)) return DSPARK_E_POINTER;
  st = check_workspace(*P, workspace, workspace_bytes);
  if (st != DSPARK_OK) return st;
  (void)hipGetLastError();
  if (kDebugChecks && !debug_schedule_inputs(*P, surv, T_table, stream)) return DSPARK_E_LAUNCH;
  const Layout L = make_layout(*P);
  if (launch_schedule(*P, surv, T_table, n_sched, n_total, at<int32_t>(workspace, L.rpart),
                      at<float>(workspace, L.sorts), at<int32_t>(workspace, L.sorti), stream) != hipSuccess)
    return DSPARK_E_LAUNCH;
  if (kDebugChecks && debug_check_schedule(n_sched, n_total, P->B, P->K, DSPARK_DEBUG_OUTPUT, stream) != hipSuccess)
    return DSPARK_E_LAUNCH;
  return DSPARK_OK;
}

// ---------------------------------------------------------------- schedule without allocation
// The scheduler's scratch for callers that cannot allocate: a file-scope device
// array, one copy per GPU for the life of the process, holding the partial
// ranks (int32 [S][n], S <= 16 segments), the survivals in schedule order
// (float [n]) and their candidate indices (int32 [n]) for up to
// kNoAllocCandidates = 32,768 candidates (2.25 MiB).  Its device address is
// taken once per device with hipGetSymbolAddress (host code never passes the
// symbol itself to a kernel) and kept per device.  Nothing in it needs
// clearing: the rank kernel writes every partial and the ordering writes
// every slot before any read.
namespace dspark {
constexpr int kNoAllocCandidates = 32768;
constexpr size_t kNoAllocRankBytes = (size_t)kSchedSegMax * kNoAllocCandidates * sizeof(int32_t);
constexpr size_t kNoAllocScratchBytes = kNoAllocRankBytes + (size_t)kNoAllocCandidates * (sizeof(float) + sizeof(int32_t));
constexpr int kNoAllocMaxDevices = 64;
}  // namespace dspark

static __device__ __align__(256) unsigned char scratch[dspark::kNoAllocScratchBytes];

static std::mutex g_scratch_mutex;
static unsigned char* g_scratch_ptr[dspark::kNoAllocMaxDevices];

// Device address of this device's scratch (the current device), looked up once.
static hipError_t scratch_for_current_device(unsigned char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= dspark::kNoAllocMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<unsigned char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

extern "C" dspark_status dspark_schedule_noalloc(const dspark_problem* P, const float* surv, const float* T_table,
                                                 int32_t* n_sched, int32_t* n_total, hipStream_t stream) {
  const AbiRange range("dspark_schedule_noalloc");
  dspark_status st = check_problem(P);
  if (st != DSPARK_OK) return st;
  if ((long long)P->B * P->K > kNoAllocCandidates) return DSPARK_E_WORKSPACE;
  if (!surv || !T_table || !n_sched || !n_total) return DSPARK_E_POINTER;
  for (const void* q : {(const void*)surv, (const void*)T_table, (const void*)n_sched, (const void*)n_total})
    if (!aligned(q, 4)) return DSPARK_E_POINTER;
  (void)hipGetLastError();
  unsigned char* ws = nullptr;
  if (scratch_for_current_device(&ws) != hipSuccess) return DSPARK_E_LAUNCH;
  int32_t* rpart = reinterpret_cast<int32_t*>(ws);
  float* sorted_s = reinterpret_cast<float*>(ws + kNoAllocRankBytes);
  int32_t* sorted_i = reinterpret_cast<int32_t*>(ws + kNoAllocRankBytes + (size_t)kNoAllocCandidates * sizeof(float));
  if (kDebugChecks && !debug_schedule_inputs(*P, surv, T_table, stream)) return DSPARK_E_LAUNCH;
  if (launch_schedule(*P, surv, T_table, n_sched, n_total, rpart, sorted_s, sorted_i, stream) != hipSuccess)
    return DSPARK_E_LAUNCH;
  if (kDebugChecks && debug_check_schedule(n_sched, n_total, P->B, P->K, DSPARK_DEBUG_OUTPUT, stream) != hipSuccess)
    return DSPARK_E_LAUNCH;
  return DSPARK_OK;
}

extern "C" dspark_status dspark_schedule_fixed(const dspark_problem* P, int32_t gamma, int32_t* n_sched,
                                               int32_t* n_total, hipStream_t stream) {
  const AbiRange range("dspark_schedule_fixed");
  dspark_status st = check_problem(P);
  if (st != DSPARK_OK) return st;
  if (gamma < 0 || gamma > P->K) return DSPARK_E_INVALID;
  if (!n_sched || !n_total) return DSPARK_E_POINTER;
  if (!aligned(n_sched, 4) || !aligned(n_total, 4)) return DSPARK_E_POINTER;
  (void)hipGetLastError();
  if (launch_schedule_static(*P, nullptr, 0, gamma, 0.f, n_sched, n_total, stream) != hipSuccess)
    return DSPARK_E_LAUNCH;
  if (kDebugChecks && debug_check_schedule(n_sched, n_total, P->B, P->K, DSPARK_DEBUG_OUTPUT, stream) != hipSuccess)
    return DSPARK_E_LAUNCH;
  return DSPARK_OK;
}

extern "C" dspark_status dspark_schedule_threshold(const dspark_problem* P, const float* surv, float theta,
                                                   int32_t* n_sched, int32_t* n_total, hipStream_t stream) {
  const AbiRange range("dspark_schedule_threshold");
  dspark_status st = check_problem(P);
  if (st != DSPARK_OK) return st;
  if (!isfinite(theta)) return DSPARK_E_INVALID;
  if (!surv || !n_sched || !n_total) return DSPARK_E_POINTER;
  for (const void* q : {(const void*)surv, (const void*)n_sched, (const void*)n_total})
    if (!aligned(q, 4)) return DSPARK_E_POINTER;
  (void)hipGetLastError();
  if (kDebugChecks && !debug_schedule_inputs(*P, surv, nullptr, stream)) return DSPARK_E_LAUNCH;
  if (launch_schedule_static(*P, surv, 1, 0, theta, n_sched, n_total, stream) != hipSuccess) return DSPARK_E_LAUNCH;
  if (kDebugChecks && debug_check_schedule(n_sched, n_total, P->B, P->K, DSPARK_DEBUG_OUTPUT, stream) != hipSuccess)
    return DSPARK_E_LAUNCH;
  return DSPARK_OK;
}

static bool sts_sizes_ok(int32_t M, int32_t K, int32_t G, int32_t n_bins) {
  return M >= 0 && M <= (1 << 24) && K >= 1 && K <= 1024 && G >= 1 && G <= 4096 && n_bins >= 1 &&
         n_bins <= kStsBinsMax;
}

extern "C" size_t dspark_sts_workspace_bytes(int32_t M, int32_t K, int32_t G, int32_t n_bins) {
  if (!sts_sizes_ok(M, K, G, n_bins)) return 0;
  return make_sts_layout(M, K, G, n_bins).total;
}

extern "C" dspark_status dspark_sts_fit(int32_t M, int32_t K, const float* conf_raw, const int32_t* acc_len,
                                        const int32_t* n_verified, const double* tau_grid, int32_t G,
                                        int32_t n_bins, double* tau, int32_t* tau_idx, double* ece_fit,
                                        double* ece_raw, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  const AbiRange range("dspark_sts_fit");
  if (!sts_sizes_ok(M, K, G, n_bins)) return DSPARK_E_INVALID;
  if (!tau_grid || !tau || !tau_idx || !ece_fit || !ece_raw) return DSPARK_E_POINTER;
  if (M > 0 && (!conf_raw || !acc_len || !n_verified)) return DSPARK_E_POINTER;
  for (const void* q : {(const void*)conf_raw, (const void*)acc_len, (const void*)n_verified, (const void*)tau_idx})
    if (!aligned(q, 4)) return DSPARK_E_POINTER;
  for (const void* q : {(const void*)tau_grid, (const void*)tau, (const void*)ece_fit, (const void*)ece_raw})
    if (!aligned(q, 8)) return DSPARK_E_POINTER;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < make_sts_layout(M, K, G, n_bins).total)
    return DSPARK_E_WORKSPACE;
  (void)hipGetLastError();
  if (launch_sts_fit(M, K, conf_raw, acc_len, n_verified, tau_grid, G, n_bins, tau, tau_idx, ece_fit, ece_raw,
                     workspace, stream) != hipSuccess)
    return DSPARK_E_LAUNCH;
  return DSPARK_OK;
}

extern "C" dspark_status dspark_schedule_async(const dspark_problem* P, const float* surv_lag, const float* surv,
                                               const float* T_table, int32_t* n_sched, int32_t* n_total,
                                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const AbiRange range("dspark_schedule_async");
  dspark_status st = check_problem(P);
  if (st != DSPARK_OK) return st;
  if (!surv_lag || !surv || !T_table || !n_sched || !n_total) return DSPARK_E_POINTER;
  for (const void* q : {(const void*)surv_lag, (const void*)surv, (const void*)T_table, (const void*)n_sched,
                        (const void*)n_total})
    if (!aligned(q, 4)) return DSPARK_E_POINTER;
  st = check_workspace(*P, workspace, workspace_bytes);
  if (st != DSPARK_OK) return st;
  (void)hipGetLastError();
  const Layout L = make_layout(*P);
  int32_t* lag = at<int32_t>(workspace, L.lagn);
  if (kDebugChecks && !(debug_schedule_inputs(*P, surv_lag, T_table, stream) &&
                        debug_schedule_inputs(*P, surv, nullptr, stream)))
    return DSPARK_E_LAUNCH;
  if (launch_schedule_async(*P, surv_lag, surv, T_table, n_sched, n_total, at<int32_t>(workspace, L.rpart),
                            at<float>(workspace, L.sorts), at<int32_t>(workspace, L.sorti), lag, lag + P->B,
                            stream) != hipSuccess)
    return DSPARK_E_LAUNCH;
  if (kDebugChecks && debug_check_schedule(n_sched, n_total, P->B, P->K, DSPARK_DEBUG_OUTPUT, stream) != hipSuccess)
    return DSPARK_E_LAUNCH;
  return DSPARK_OK;
}

static dspark_status verify_impl(const dspark_problem* P, const void* target, const void* Z, const void* E,
                                 const void* Wt, const int32_t* anchor, const int32_t* draft_tok,
                                 const float* draft_logq, const float* draft_lse, const int32_t* n_sched,
                                 int32_t* out_tok, int32_t* n_accepted, int32_t* next_anchor, float* logp,
                                 float* resid_mass, void* workspace, size_t workspace_bytes, hipStream_t stream,
                                 const float* state) {
  dspark_status st = check_problem(P);
  if (st != DSPARK_OK) return st;
  const dspark_problem& p = *P;
  if (state) {
    if (!rnn_supported(p)) return DSPARK_E_UNSUPPORTED;
    if (!aligned(state, 16)) return DSPARK_E_POINTER;
  }
  if (!target || !Z || !E || !Wt || !anchor || !draft_tok || !draft_logq || !draft_lse || !n_sched || !out_tok ||
      !n_accepted || !next_anchor || !logp || !resid_mass)
    return DSPARK_E_POINTER;
  for (const void* q : {target, Z, E, Wt})
    if (!aligned(q, 16)) return DSPARK_E_POINTER;
  for (const void* q : {(const void*)anchor, (const void*)draft_tok, (const void*)draft_logq,
                        (const void*)draft_lse, (const void*)n_sched, (const void*)out_tok,
                        (const void*)n_accepted, (const void*)next_anchor, (const void*)logp,
                        (const void*)resid_mass})
    if (!aligned(q, 4)) return DSPARK_E_POINTER;
  st = check_workspace(p, workspace, workspace_bytes);
  if (st != DSPARK_OK) return st;
  (void)hipGetLastError();
  if (kDebugChecks && !debug_verify_inputs(p, target, Z, E, Wt, anchor, draft_tok, n_sched, stream))
    return DSPARK_E_LAUNCH;

  const Layout L = make_layout(p);
  VerifyArgs va{};
  va.Zt = target;
  va.Z = Z;
  va.E = E;
  va.Wt = Wt;
  va.anchor = anchor;
  va.tok = draft_tok;
  va.logq = draft_logq;
  va.lse_q = draft_lse;
  va.n_sched = n_sched;
  va.out_tok = out_tok;
  va.n_acc = n_accepted;
  va.next_anchor = next_anchor;
  va.logp = logp;
  va.resid_mass = resid_mass;
  va.vlse = at<float2>(workspace, L.vlse);
  va.lse_p = at<float>(workspace, L.lsep);
  va.job = at<int32_t>(workspace, L.job);
  va.rows = at<int32_t>(workspace, L.rows);
  va.nrows = at<int32_t>(workspace, L.nrows);
  va.part = at<float4>(workspace, L.part);
  va.zpart = at<float2>(workspace, L.zpart);
  va.B = p.B;
  va.K = p.K;
  va.V = p.V;
  va.r = p.r;
  va.G = L.G;
  va.nseg = L.nseg;
  va.inv_T = 1.0f / p.sampling_temp;
  va.scale2 = kLog2e / p.sampling_temp;
  va.key = host_key(p.seed);
  va.efrag = verify_uses_efrag(p) ? at<uint4>(workspace, L.efrag) : nullptr;
  va.state = state;
  if (launch_verify_pre(p, va, stream) != hipSuccess) return DSPARK_E_LAUNCH;

  StreamArgs sa{};
  sa.Z = Z;
  sa.Zt = target;
  sa.E = E;
  sa.Wt = Wt;
  sa.anchor = anchor;
  sa.tok = draft_tok;
  sa.lse_q = draft_lse;
  sa.lse_p = va.lse_p;
  sa.job = va.job;
  sa.n_sched = n_sched;
  sa.part = at<float4>(workspace, L.part);
  sa.zpart = at<float2>(workspace, L.zpart);
  sa.efrag = va.efrag;
  sa.B = p.B;
  sa.K = p.K;
  sa.V = p.V;
  sa.k = 0;
  sa.nchunks = n_chunks(p.V);
  sa.scale2 = va.scale2;
  sa.key = va.key;
  if (launch_stream_verify(p, sa, L.G, stream) != hipSuccess) return DSPARK_E_LAUNCH;
  if (launch_verify_finish(p, va, stream) != hipSuccess) return DSPARK_E_LAUNCH;
  if (kDebugChecks && debug_check_verify(n_sched, out_tok, n_accepted, next_anchor, resid_mass, p.B, p.K, p.V,
                                         DSPARK_DEBUG_OUTPUT, stream) != hipSuccess)
    return DSPARK_E_LAUNCH;
  return DSPARK_OK;
}

extern "C" dspark_status dspark_verify(const dspark_problem* P, const void* target, const void* Z, const void* E,
                                       const void* Wt, const int32_t* anchor, const int32_t* draft_tok,
                                       const float* draft_logq, const float* draft_lse, const int32_t* n_sched,
                                       int32_t* out_tok, int32_t* n_accepted, int32_t* next_anchor, float* logp,
                                       float* resid_mass, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  const AbiRange range("dspark_verify");
  return verify_impl(P, target, Z, E, Wt, anchor, draft_tok, draft_logq, draft_lse, n_sched, out_tok, n_accepted,
                     next_anchor, logp, resid_mass, workspace, workspace_bytes, stream, nullptr);
}

extern "C" dspark_status dspark_verify_rnn(const dspark_problem* P, const void* target, const void* Z,
                                           const void* E, const void* Wt, const int32_t* anchor,
                                           const int32_t* draft_tok, const float* draft_logq, const float* draft_lse,
                                           const float* state, const int32_t* n_sched, int32_t* out_tok,
                                           int32_t* n_accepted, int32_t* next_anchor, float* logp, float* resid_mass,
                                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const AbiRange range("dspark_verify_rnn");
  if (!state) return DSPARK_E_POINTER;
  return verify_impl(P, target, Z, E, Wt, anchor, draft_tok, draft_logq, draft_lse, n_sched, out_tok, n_accepted,
                     next_anchor, logp, resid_mass, workspace, workspace_bytes, stream, state);
}

extern "C" dspark_status dspark_debug_flags(uint32_t* flags, int32_t clear) {
  if (!kDebugChecks) return DSPARK_E_UNSUPPORTED;
  if (!flags) return DSPARK_E_POINTER;
  const AbiRange range("dspark_debug_flags");
  unsigned* w = nullptr;
  if (debug_word(&w) != hipSuccess || hipDeviceSynchronize() != hipSuccess) return DSPARK_E_LAUNCH;
  unsigned v = 0;
  if (hipMemcpy(&v, w, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return DSPARK_E_LAUNCH;
  if (clear) {
    const unsigned zero = 0;
    if (hipMemcpy(w, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return DSPARK_E_LAUNCH;
  }
  *flags = v;
  return DSPARK_OK;
}

extern "C" dspark_status dspark_debug_check_inputs(const dspark_problem* P, const void* Z, const void* target,
                                                   const int32_t* anchor, const float* T_table, hipStream_t stream) {
  if (!kDebugChecks) return DSPARK_E_UNSUPPORTED;
  const dspark_status st = check_problem(P);
  if (st != DSPARK_OK) return st;
  for (const void* q : {Z, target})
    if (q && !aligned(q, 16)) return DSPARK_E_POINTER;
  for (const void* q : {(const void*)anchor, (const void*)T_table})
    if (q && !aligned(q, 4)) return DSPARK_E_POINTER;
  const AbiRange range("dspark_debug_check_inputs");
  (void)hipGetLastError();
  const dspark_problem& p = *P;
  const bool zb = p.logits_dtype == DSPARK_BF16;
  if ((Z && debug_scan_nonfinite(Z, (size_t)p.B * p.K * p.V, zb, DSPARK_DEBUG_LOGITS, stream) != hipSuccess) ||
      (target &&
       debug_scan_nonfinite(target, (size_t)p.B * (p.K + 1) * p.V, zb, DSPARK_DEBUG_LOGITS, stream) != hipSuccess) ||
      (anchor && debug_scan_range_i32(anchor, (size_t)p.B, 0, p.V - 1, DSPARK_DEBUG_IDS, stream) != hipSuccess) ||
      !debug_schedule_inputs(p, nullptr, T_table, stream))
    return DSPARK_E_LAUNCH;
  return DSPARK_OK;
}

extern "C" dspark_status dspark_debug_force_barrier_timeout(int32_t on) {
  if (!kDebugChecks) return DSPARK_E_UNSUPPORTED;
  g_debug_force_timeout = on != 0;
  return DSPARK_OK;
}
