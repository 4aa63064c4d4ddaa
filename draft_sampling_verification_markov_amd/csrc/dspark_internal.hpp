// Internal interfaces between the C-ABI layer (dspark_abi.hip) and the kernel
// translation units: workspace layout, kernel argument blocks, launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "../../include/dspark.h"
#include "../../include/dspark_instr.h"
#include "dspark_device.hpp"

namespace dspark {

// Workgroups of the vocabulary-split stream kernel (one per CU on MI355X).
constexpr int kStreamGridMax = 256;
// Target-row segment of the verify log-partition pass.
#ifndef DSPARK_VLSE_SEG
#define DSPARK_VLSE_SEG 8192
#endif
constexpr int kVlseSeg = DSPARK_VLSE_SEG;
// Workgroups of the verify log-partition pass.
#ifndef DSPARK_VLSE_GRID
#define DSPARK_VLSE_GRID 1024
#endif
constexpr int kVlseGrid = DSPARK_VLSE_GRID;

inline int n_chunks(int V) { return (V + kChunk - 1) / kChunk; }
// The smallest grid that gives no workgroup more chunks than an even split over
// kStreamGridMax would (1,187 chunks: 238 workgroups of 4-5, not 256 of 4-5):
// the step lasts as long as its busiest workgroup, and idle CUs take no share of
// the per-step fill.
inline int stream_grid(int V) {
  const int nc = n_chunks(V);
  const int per = (nc + kStreamGridMax - 1) / kStreamGridMax;
  return (nc + per - 1) / per;
}
inline int vlse_segments(int V) { return (V + kVlseSeg - 1) / kVlseSeg; }

// Byte offsets of the workspace regions (256-byte aligned each).
struct Layout {
  int G;        // stream-kernel workgroups
  int nseg;     // verify segments per target row
  size_t part;  // float4 [B][G]: per-(row, workgroup) partials of the stream kernel
  size_t zpart; // float2 [B][G]: resample pass, per-(row, workgroup) sums of p^ and q^ (residual normalisers)
  size_t vlse;  // float2 [B*K][nseg]: per-segment (max, sum) of target rows, base 2
  size_t lsep;  // float [B][K]: log-partition of p_k in nats
  size_t job;   // int32 [B]: position of the first rejection (0 = all accepted)
  size_t rows;  // int32 [B*K]: compact list of rows to verify, b * 64 + (k - 1)
  size_t nrows; // int32 [1]
  size_t rpart; // int32 [S][B*K]: partial ranks of the candidates over S segments
  size_t sorts; // float [B*K]: survivals in schedule order (candidate sets too large for LDS)
  size_t sorti; // int32 [B*K]: candidate indices in schedule order (same)
  size_t lagn;  // int32 [B + 1]: the lagged schedule of the asynchronous scheduler (n_b, then N)
  size_t efrag; // uint4 [ceil(B/32)][r/16][64]: E rows of the previous draft tokens, B-fragment order
  size_t prec;  // uint64 [B][persist_grid][4]: the persistent draft's tagged partial records (B <= 256)
  size_t ptok;  // uint64 [kSyncGroups][kTokRepSlots]: the persistent draft's tagged tokens, one replica per group
  size_t psync; // uint32 [kPersistSyncWords]: the persistent draft's time-out flag and launch generation
  size_t total;
};

Layout make_layout(const dspark_problem& P);

// Arguments of the stream kernel (draft step k, or the verify resample pass).
struct StreamArgs {
  const void* Z;         // [B][K][V] base logits
  const void* Zt;        // [B][K+1][V] target logits (verify)
  const void* E;         // [V][r]
  const void* Wt;        // [V][r]
  const int32_t* anchor; // [B]
  const int32_t* tok;    // [B][K] draft tokens
  const float* lse_q;    // [B][K] nats (verify)
  const float* lse_p;    // [B][K] nats (verify)
  const int32_t* job;    // [B] (verify)
  const int32_t* n_sched;// [B] (verify)
  float4* part;          // [B][G]
  float2* zpart;         // [B][G] (verify): sums of p^ and q^ over the workgroup's entries of a residual row
  const uint4* efrag;    // B fragments of the previous tokens (draft kernel with bf16 logits and factors)
  int first_from_anchor; // draft kernel with bf16 logits and factors: B fragments gathered from E[anchor]
  int B, K, V, k;        // k: 1-based draft position (draft mode)
  int nchunks;
  float scale2;          // log2(e) / T_s
  Key key;
};

// Arguments of the persistent draft kernel (all K positions in one cooperative
// launch, each workgroup's slice of Wt held on chip for the whole cycle).
struct PersistArgs {
  const void* Z;         // [B][K][V] bf16
  const void* E;         // [V][r] bf16
  const void* Wt;        // [V][r] bf16
  const int32_t* anchor; // [B]
  int32_t* tok;          // [B][K] outputs
  float* logq;
  float* lse;
  unsigned long long* rec;    // [B][G][4] tagged partial records of the latest positions
  unsigned long long* tokrep; // [kSyncGroups][kTokRepSlots] tagged tokens of the latest positions
  unsigned* sync;        // [kPersistSyncWords] time-out flag (zeroed) and launch generation (advanced) at launch
  uint32_t z_bytes;      // bytes of Z (below 2^32)
  uint32_t spin_limit;   // polls of a wait before it gives up (kPersistSpinLimit)
  uint32_t unreachable;  // 0; nonzero makes every wait's expected tag one that is never written (all time out)
  int B, K, V, nchunks;
  float scale2, inv_T;
  Key key;
};

struct SelectArgs {
  const void* Z;
  const void* E;
  const void* Wt;
  const int32_t* anchor;
  int32_t* tok;          // [B][K] written at position k
  float* logq;
  float* lse;
  const float4* part;
  uint4* efrag;          // if set, the chosen token's E row is stored there in B-fragment order
  const float* state;    // RNN head: [B][K][r] states; bf16(state[b][k-1]) replaces E[x_{k-1}] (bf16 factors)
  int B, K, V, r, k, G;
  float inv_T;
  Key key;
};

struct ConfArgs {
  const void* h;
  const void* E;
  const float* w_c;
  float b_c;
  const float* tau;
  const int32_t* anchor;
  const int32_t* tok;
  float* conf;
  float* surv;
  int B, K, V, d, r;
};

struct VerifyArgs {
  const void* Zt;
  const void* Z;
  const void* E;
  const void* Wt;
  const int32_t* anchor;
  const int32_t* tok;
  const float* logq;
  const float* lse_q;
  const int32_t* n_sched;
  int32_t* out_tok;
  int32_t* n_acc;
  int32_t* next_anchor;
  float* logp;
  float* resid_mass;
  // workspace
  float2* vlse;
  float* lse_p;
  int32_t* job;
  int32_t* rows;
  int32_t* nrows;
  const float4* part;
  const float2* zpart;   // [B][G]: the resample pass's sums of p^ and q^ (residual rows)
  uint4* efrag;          // if set, k_accept stores the resample pass's B fragments there
  const float* state;    // RNN head: [B][K][r] states, the projection operands (bf16-rounded) of the positions
  int B, K, V, r, G, nseg;
  float inv_T, scale2;
  Key key;
};

// E row of token x stored for row b in the B-fragment order of the streaming
// kernels: entries 8p..8p+7 go to 16-byte slot ((b/32)*(r/16) + p/2)*64 + b%32 + 32*(p%2),
// so lane l of the wave holding rows 32*(b/32).. reads K-step t as one
// contiguous 1 KB block.  x < 0 stores zeros (a row without a draft term).
__device__ __forceinline__ void efrag_store_piece(uint4* efrag, const uint16_t* E, int x, int b, int r, int p) {
  const uint4 v = x >= 0 ? *reinterpret_cast<const uint4*>(E + (size_t)x * r + 8 * p) : make_uint4(0, 0, 0, 0);
  efrag[((size_t)(b >> 5) * (r >> 4) + (p >> 1)) * 64 + (b & 31) + 32 * (p & 1)] = v;
}
// The same piece taken from a float row rounded to bfloat16 (null row: zeros).
__device__ __forceinline__ void efrag_store_piece_f32(uint4* efrag, const float* row, int b, int r, int p) {
  const uint4 v = row ? bf16x8_from_f32(row + 8 * p) : make_uint4(0, 0, 0, 0);
  efrag[((size_t)(b >> 5) * (r >> 4) + (p >> 1)) * 64 + (b & 31) + 32 * (p & 1)] = v;
}

// RNN head.  Gh: [B*K][3r] float, the hidden-state part of the input gates.
size_t rnn_extra_bytes(const dspark_problem& P);
bool rnn_supported(const dspark_problem& P);
hipError_t launch_rnn_gemm(const dspark_problem& P, const void* h, const void* W_ih, const float* b_ih, float* Gh,
                           hipStream_t s);
hipError_t launch_rnn_step(const dspark_problem& P, const float* Gh, const void* W_ih, const void* W_hh,
                           const float* b_hh, const void* E, const int32_t* anchor, const int32_t* tok, float* state,
                           uint4* efrag, int k, hipStream_t s);

// Launchers; each returns hipSuccess or the launch error.
hipError_t launch_stream_draft(const dspark_problem& P, const StreamArgs& a, int G, hipStream_t s);
// true when the draft step runs the buffer-DMA kernel, which takes its B
// fragments from the efrag region (filled by the select kernel of the previous
// position; position 1 gathers the anchors' E rows itself)
bool draft_uses_efrag(const dspark_problem& P);
hipError_t launch_stream_verify(const dspark_problem& P, const StreamArgs& a, int G, hipStream_t s);
// true when the verify resample pass runs the buffer-DMA kernel, which takes
// its B fragments from the efrag region (filled by k_accept)
bool verify_uses_efrag(const dspark_problem& P);
hipError_t launch_select(const dspark_problem& P, const SelectArgs& a, hipStream_t s);
// The persistent draft kernel: true when it serves P (bf16 logits and factors,
// r = 256, B <= 256 and at most 5 chunks of the vocabulary per workgroup) and
// the device can hold its whole grid at once.
// One roctx range per ABI call (rocprofv3 --marker-trace shows them around the
// call's kernels); pushed on entry, popped on every return.
struct AbiRange {
  explicit AbiRange(const char* name) { roctxRangePushA(name); }
  ~AbiRange() { roctxRangePop(); }
  AbiRange(const AbiRange&) = delete;
  AbiRange& operator=(const AbiRange&) = delete;
};

// Debug checks (k_debug.hip): scans that raise bits of the current device's flag
// word (whose address debug_word returns) instead of trapping.
hipError_t debug_word(unsigned** out);
hipError_t debug_scan_nonfinite(const void* x, size_t n, bool bf16, unsigned bit, hipStream_t s);
hipError_t debug_scan_range_i32(const int32_t* x, size_t n, int32_t lo, int32_t hi, unsigned bit, hipStream_t s);
hipError_t debug_scan_range_f32(const float* x, size_t n, float lo, float hi, unsigned bit, hipStream_t s);
hipError_t debug_check_schedule(const int32_t* n_sched, const int32_t* n_total, int B, int K, unsigned bit,
                                hipStream_t s);
hipError_t debug_check_verify(const int32_t* n_sched, const int32_t* out_tok, const int32_t* n_acc,
                              const int32_t* next_anchor, const float* resid_mass, int B, int K, int V, unsigned bit,
                              hipStream_t s);

// workgroups of the persistent draft launch: one per vocabulary chunk up to kStreamGridMax
int persist_grid(int V);
// dspark_draft takes the persistent draft where it applies and the batch is at
// most this (the measured crossovers: with bf16 logits the per-position kernels,
// with two waves per SIMD, are faster above it; with fp32 logits they stream
// twice the bytes and the persistent draft is faster up to its limit of 256)
inline int persist_max_b(const dspark_problem& P) { return P.logits_dtype == DSPARK_F32 ? 256 : 192; }
// polls of a persistent-draft barrier wait before it sets the time-out flag
constexpr uint32_t kPersistSpinLimit = 1u << 20;
// The persistent draft's hand-offs between workgroups carry their own tags
// (launch generation x 128 + position), so that a wait polls the data it needs
// instead of a barrier counter: the time-out flag and the generation each on
// their own 4 KiB, and kSyncGroups replicas of the latest tokens (one per group
// of workgroups, 4 KiB apart) so that no word has more than G / kSyncGroups + 1
// pollers.
constexpr int kSyncGroups = 16;
constexpr int kSyncStride = 1024;                // words between the flag and the generation
constexpr int kSyncFlag = 0;                     // time-out flag at kSyncFlag * kSyncStride
constexpr int kSyncGen = 1;                      // launch generation at kSyncGen * kSyncStride
constexpr size_t kPersistSyncWords = 2 * (size_t)kSyncStride;
constexpr int kTokRepSlots = 512;                // 8-byte slots per token replica (rows 0..255 used)
constexpr int kPersistMaxB = 256;
bool draft_persistent_supported(const dspark_problem& P);
hipError_t launch_draft_persistent(const dspark_problem& P, const PersistArgs& a, hipStream_t s);
hipError_t launch_conf(const dspark_problem& P, const ConfArgs& a, hipStream_t s);
// Segments of the candidate range that the partial-rank kernel splits the comparisons into.
#ifndef DSPARK_SCHED_SEG_MAX
#define DSPARK_SCHED_SEG_MAX 16
#endif
constexpr int kSchedSegMax = DSPARK_SCHED_SEG_MAX;
int sched_segments(int n);
hipError_t launch_schedule(const dspark_problem& P, const float* surv, const float* T, int32_t* n_sched,
                           int32_t* n_total, int32_t* part, float* sorted_s, int32_t* sorted_i, hipStream_t s);
// STS fitting: bin partial of one (candidate, sample split) pair.
struct StsPart {
  double sum;    // sum of predictions in the bin
  uint32_t cnt;  // observed samples in the bin
  uint32_t lab;  // of which accepted
};
constexpr int kStsBinsMax = 16;
struct StsLayout {
  int S;         // sample splits per candidate
  size_t zl;     // double [K][M]: logits of the raw confidences
  size_t fit;    // double [M]: running products with the fitted temperatures
  size_t raw;    // double [M]: same at temperature 1
  size_t part;   // StsPart [G+1][S][n_bins]
  size_t total;
};
int sts_splits(int M);
StsLayout make_sts_layout(int M, int K, int G, int n_bins);
hipError_t launch_sts_fit(int M, int K, const float* c, const int32_t* acc, const int32_t* nver, const double* grid,
                          int G, int n_bins, double* tau, int32_t* tau_idx, double* ece_fit, double* ece_raw,
                          void* ws, hipStream_t s);

// Baselines: mode 0 fixed length gamma, mode 1 survival threshold theta.
hipError_t launch_schedule_static(const dspark_problem& P, const float* surv, int mode, int gamma, float theta,
                                  int32_t* n_sched, int32_t* n_total, hipStream_t s);
// Asynchronous form: budget from surv_lag's first-drop schedule (into lag_n,
// lag_total), then the leading candidates of surv in schedule order.
hipError_t launch_schedule_async(const dspark_problem& P, const float* surv_lag, const float* surv, const float* T,
                                 int32_t* n_sched, int32_t* n_total, int32_t* part, float* sorted_s,
                                 int32_t* sorted_i, int32_t* lag_n, int32_t* lag_total, hipStream_t s);
hipError_t launch_verify_pre(const dspark_problem& P, const VerifyArgs& a, hipStream_t s);
hipError_t launch_verify_finish(const dspark_problem& P, const VerifyArgs& a, hipStream_t s);

}  // namespace dspark
