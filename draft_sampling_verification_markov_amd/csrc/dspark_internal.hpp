// Internal interfaces between the C-ABI layer (dspark_abi.hip) and the kernel
// translation units: workspace layout, kernel argument blocks, launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dspark.h"
#include "dspark_device.hpp"

namespace dspark {

// Workgroups of the vocabulary-split stream kernel (one per CU on MI355X).
constexpr int kStreamGridMax = 256;
// Target-row segment of the verify log-partition pass.
constexpr int kVlseSeg = 8192;
// Workgroups of the verify log-partition pass.
constexpr int kVlseGrid = 1024;

inline int n_chunks(int V) { return (V + kChunk - 1) / kChunk; }
inline int stream_grid(int V) { const int nc = n_chunks(V); return nc < kStreamGridMax ? nc : kStreamGridMax; }
inline int vlse_segments(int V) { return (V + kVlseSeg - 1) / kVlseSeg; }

// Byte offsets of the workspace regions (256-byte aligned each).
struct Layout {
  int G;        // stream-kernel workgroups
  int nseg;     // verify segments per target row
  size_t part;  // float4 [B][G]: per-(row, workgroup) partials of the stream kernel
  size_t vlse;  // float2 [B*K][nseg]: per-segment (max, sum) of target rows, base 2
  size_t lsep;  // float [B][K]: log-partition of p_k in nats
  size_t job;   // int32 [B]: position of the first rejection (0 = all accepted)
  size_t rows;  // int32 [B*K]: compact list of rows to verify, b * 64 + (k - 1)
  size_t nrows; // int32 [1]
  size_t sorted;// int32 [B*K]: candidates in schedule order
  size_t efrag; // uint4 [ceil(B/32)][r/16][64]: E rows of the previous draft tokens, B-fragment order
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
  const uint4* efrag;    // B fragments of the previous tokens (draft kernel with bf16 logits and factors)
  int B, K, V, k;        // k: 1-based draft position (draft mode)
  int nchunks;
  float scale2;          // log2(e) / T_s
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
  int B, K, V, r, G, nseg;
  float inv_T, scale2;
  Key key;
};

// Launchers; each returns hipSuccess or the launch error.
hipError_t launch_stream_draft(const dspark_problem& P, const StreamArgs& a, int G, hipStream_t s);
// true when the draft step runs the buffer-DMA kernel, which takes its B
// fragments from the efrag region (filled by launch_efrag_gather for the
// anchors and by the select kernel for later positions)
bool draft_uses_efrag(const dspark_problem& P);
hipError_t launch_efrag_gather(const dspark_problem& P, const void* E, const int32_t* tok, uint4* efrag,
                               hipStream_t s);
hipError_t launch_stream_verify(const dspark_problem& P, const StreamArgs& a, int G, hipStream_t s);
hipError_t launch_select(const dspark_problem& P, const SelectArgs& a, hipStream_t s);
hipError_t launch_conf(const dspark_problem& P, const ConfArgs& a, hipStream_t s);
hipError_t launch_schedule(const dspark_problem& P, const float* surv, const float* T, int32_t* n_sched,
                           int32_t* n_total, int32_t* sorted, hipStream_t s);
hipError_t launch_verify_pre(const dspark_problem& P, const VerifyArgs& a, hipStream_t s);
hipError_t launch_verify_finish(const dspark_problem& P, const VerifyArgs& a, hipStream_t s);

}  // namespace dspark
