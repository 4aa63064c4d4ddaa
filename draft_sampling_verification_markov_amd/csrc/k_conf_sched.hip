// Confidence head with Sequential Temperature Scaling, prefix survival, and the
// first-drop prefix scheduler.
//
// DSpark page, Method > Confidence-scheduled verification:
//   * confidence of position k: a linear projection of [backbone hidden h_k;
//     Markov embedding E[x_{k-1}] of the preceding draft token] through a
//     sigmoid, with one STS temperature per position dividing the logit;
//     survival is the running product along the block;
//   * the scheduler takes candidates in one global survival order (the block
//     prefix order is respected because survival never increases along a
//     block) and stops as soon as expected tokens per second, read from the
//     step-time table, would drop, which keeps verification non-anticipating.
#include "dspark_internal.hpp"

namespace dspark {
namespace {

// ---------------------------------------------------------------- confidence
// dot(x[0:n], w[0:n]) over one wave; lane-strided 16-byte pieces, four pieces
// in flight per lane.  w may live in LDS or global memory.
template <typename T>
__device__ __forceinline__ float dot_vec(const T* x, const float* w, int n, int lane);

template <>
__device__ __forceinline__ float dot_vec<uint16_t>(const uint16_t* x, const float* w, int n, int lane) {
  float acc = 0.f;
#pragma unroll 4
  for (int i = lane * 8; i < n; i += 64 * 8) {
    const uint4 hv = *reinterpret_cast<const uint4*>(x + i);
    const float4 w0 = *reinterpret_cast<const float4*>(w + i);
    const float4 w1 = *reinterpret_cast<const float4*>(w + i + 4);
    acc = fmaf(bf16_lo(hv.x), w0.x, acc);
    acc = fmaf(bf16_hi(hv.x), w0.y, acc);
    acc = fmaf(bf16_lo(hv.y), w0.z, acc);
    acc = fmaf(bf16_hi(hv.y), w0.w, acc);
    acc = fmaf(bf16_lo(hv.z), w1.x, acc);
    acc = fmaf(bf16_hi(hv.z), w1.y, acc);
    acc = fmaf(bf16_lo(hv.w), w1.z, acc);
    acc = fmaf(bf16_hi(hv.w), w1.w, acc);
  }
  return acc;
}

template <>
__device__ __forceinline__ float dot_vec<float>(const float* x, const float* w, int n, int lane) {
  float acc = 0.f;
#pragma unroll 4
  for (int i = lane * 4; i < n; i += 64 * 4) {
    const float4 hv = *reinterpret_cast<const float4*>(x + i);
    const float4 wv = *reinterpret_cast<const float4*>(w + i);
    acc = fmaf(hv.x, wv.x, acc);
    acc = fmaf(hv.y, wv.y, acc);
    acc = fmaf(hv.z, wv.z, acc);
    acc = fmaf(hv.w, wv.w, acc);
  }
  return acc;
}

constexpr int kConfThreads = 1024;
constexpr int kConfWaves = kConfThreads / 64;
constexpr int kConfWMax = 16384;  // floats of w_c staged in LDS (64 KB)

// One workgroup per request, one wave per position; with STAGE the
// confidence weights [w_h; w_e] are copied to LDS once per workgroup.
template <typename HT, typename WT, bool STAGE>
__global__ __launch_bounds__(kConfThreads) void k_conf(ConfArgs a) {
  extern __shared__ float s_w[];
  __shared__ float s_c[64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, d = a.d, r = a.r;
  const HT* h = static_cast<const HT*>(a.h);
  const WT* E = static_cast<const WT*>(a.E);
  const float* w = a.w_c;
  if (STAGE) {
    for (int i = tid * 4; i < d + r; i += kConfThreads * 4)
      *reinterpret_cast<float4*>(s_w + i) = *reinterpret_cast<const float4*>(a.w_c + i);
    __syncthreads();
    w = s_w;
  }
  for (int k = wave; k < K; k += kConfWaves) {
    const int prev = clamp_id(k == 0 ? a.anchor[b] : a.tok[(size_t)b * K + k - 1], a.V);
    float z = dot_vec<HT>(h + ((size_t)b * K + k) * d, w, d, lane);
    z += dot_vec<WT>(E + (size_t)prev * r, w + d, r, lane);
    z = wave_sum(z);
    if (lane == 0) {
      const float t = (z + a.b_c) / a.tau[k];
      s_c[k] = 1.0f / (1.0f + expf(-t));
    }
  }
  __syncthreads();
  if (tid == 0) {
    double S = 1.0;  // running product in double, rounded once per position
    for (int k = 0; k < K; ++k) {
      const float c = s_c[k];
      S *= (double)c;
      a.conf[(size_t)b * K + k] = c;
      a.surv[(size_t)b * K + k] = (float)S;
    }
  }
}

// ---------------------------------------------------------------- scheduler
// The scheduler takes candidates in the order (survival desc, request asc,
// position asc); with candidate index i = b*K + (k-1) that is (survival desc,
// i asc), i.e. ascending 64-bit keys: the complemented order-preserving bits
// of the survival above i.
__device__ __forceinline__ uint32_t float_order_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ unsigned long long sched_key(float s, int i) {
  return ((unsigned long long)(~float_order_bits(s)) << 32) | (unsigned)i;
}

// Partial ranks: candidate i (one per thread) counts the keys below its own
// in segment blockIdx.y of the candidates; part[seg][i] (no atomics, so
// nothing needs clearing).
constexpr int kRankTile = 2048;
__global__ __launch_bounds__(256) void k_sched_rank(const float* surv, int n, int S, int32_t* part) {
  __shared__ unsigned long long tile[kRankTile];
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int seg = blockIdx.y;
  const int j0 = (int)(((long long)seg * n) / S), j1 = (int)(((long long)(seg + 1) * n) / S);
  const unsigned long long ki = i < n ? sched_key(surv[i], i) : ~0ull;
  int cnt = 0;
  for (int t0 = j0; t0 < j1; t0 += kRankTile) {
    const int len = min(kRankTile, j1 - t0);
    __syncthreads();
    for (int j = threadIdx.x; j < len; j += 256) tile[j] = sched_key(surv[t0 + j], t0 + j);
    __syncthreads();
#pragma unroll 8
    for (int j = 0; j < len; ++j) cnt += tile[j] < ki ? 1 : 0;
  }
  if (i < n) part[(size_t)seg * n + i] = cnt;
}

// Greedy pass over candidates in schedule order (sorted_s / sorted_i, any
// address space): fp64 prefix sums over per-thread segments, the first
// refusal of (A + s) * T[N] >= A * T[N + 1], the total and per-request counts.
// The step-time entries of the first batch of a thread's segment, loaded at the
// start of the kernel (their round trip overlaps the ordering).
constexpr int kGreedyBatch = 8;
struct GreedyT {
  float tv[kGreedyBatch + 1];
  template <int THREADS>
  __device__ __forceinline__ void load(const float* T, int B, int K) {
    const int n = B * K;
    const int lo = (int)(((long long)threadIdx.x * n) / THREADS);
#pragma unroll
    for (int j = 0; j <= kGreedyBatch; ++j) tv[j] = T[B + min(lo + j, n)];  // T has B + n + 1 entries
  }
};

// LDS_COUNT: per-request counts in LDS (s_cnt, B entries, zeroed by the caller
// before an earlier barrier) stored to n_sched at the end, instead of global
// atomics on n_sched.
template <int THREADS, bool LDS_COUNT, typename SS, typename SI>
__device__ __forceinline__ void sched_greedy(const SS* sorted_s, const SI* sorted_i, const float* T, const GreedyT& t0,
                                             int B, int K, int32_t* n_sched, int32_t* n_total, double* s_wsum,
                                             int* s_wmin, int* s_stop, int* s_cnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = B * K;
  const int lo = (int)(((long long)tid * n) / THREADS);
  const int hi = (int)(((long long)(tid + 1) * n) / THREADS);
  // segments are read in register batches of kBatch (clamped, unconditional
  // loads), so a batch costs one memory round trip instead of one per element
  constexpr int kBatch = kGreedyBatch;
  double local = 0.0;
  for (int m0 = lo; m0 < hi; m0 += kBatch) {
    float sv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) sv[j] = (float)sorted_s[min(m0 + j, n - 1)];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (m0 + j < hi) local += (double)sv[j];
  }
  const double incl = wave_scan_incl(local);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  double wbase = 0.0;
  for (int w = 0; w < wave; ++w) wbase += s_wsum[w];
  double A = (double)B + wbase + (incl - local);
  int first = n;
  bool open = true;
  for (int m0 = lo; m0 < hi && open; m0 += kBatch) {
    float sv[kBatch], tv[kBatch + 1];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) sv[j] = (float)sorted_s[min(m0 + j, n - 1)];
    if (m0 == lo) {
#pragma unroll
      for (int j = 0; j <= kBatch; ++j) tv[j] = t0.tv[j];
    } else {
#pragma unroll
      for (int j = 0; j <= kBatch; ++j) tv[j] = T[B + min(m0 + j, n)];  // T has B + n + 1 entries
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (open && m0 + j < hi) {
        const double s_ = (double)sv[j];
        if (!((A + s_) * (double)tv[j] >= A * (double)tv[j + 1])) {
          first = m0 + j;
          open = false;
        } else {
          A += s_;
        }
      }
    }
  }
  first = wave_min_i(first);
  if (lane == 0) s_wmin[wave] = first;
  __syncthreads();
  if (tid == 0) {
    int f = s_wmin[0];
    for (int w = 1; w < THREADS / 64; ++w) f = min(f, s_wmin[w]);
    *s_stop = f;
    *n_total = B + f;
  }
  // The counts were zeroed by this workgroup before an earlier barrier, whose
  // workgroup release waits for those stores; the device-scope atomics below
  // execute at L2 and see them.  No device-wide fence (an L2 write-back) needed.
  __syncthreads();
  const int stop = *s_stop;
  for (int m = tid; m < stop; m += THREADS) {
    int idx = (int)sorted_i[m];
    idx = idx < 0 ? 0 : (idx >= n ? n - 1 : idx);
    if (LDS_COUNT) atomicAdd(&s_cnt[idx / K], 1);
    else atomicAdd(&n_sched[idx / K], 1);
  }
  if (LDS_COUNT) {
    __syncthreads();
    for (int b = tid; b < B; b += THREADS) n_sched[b] = s_cnt[b];
  }
}

constexpr int kGreedyThreads = 1024;

// Ranks -> schedule order in global memory, many workgroups (each candidate
// sums its segment counts); then the greedy pass in one workgroup.
constexpr int kScatterThreads = 64;
__global__ __launch_bounds__(kScatterThreads) void k_sched_scatter(const float* surv, const int32_t* part, int S,
                                                                   int n, float* sorted_s, int32_t* sorted_i) {
  const int i = blockIdx.x * kScatterThreads + threadIdx.x;
  if (i >= n) return;
  // every segment load in flight at once: unconditional loads (segments past S
  // re-read segment 0) and masked sums, not branches
  int v[kSchedSegMax];
#pragma unroll
  for (int q = 0; q < kSchedSegMax; ++q) v[q] = part[(size_t)(q < S ? q : 0) * n + i];
  int r = 0;
#pragma unroll
  for (int q = 0; q < kSchedSegMax; ++q) r += q < S ? v[q] : 0;
  r = r < 0 ? 0 : (r >= n ? n - 1 : r);
  sorted_s[r] = surv[i];
  sorted_i[r] = i;
}

__global__ __launch_bounds__(kGreedyThreads) void k_sched_greedy_global(const float* sorted_s,
                                                                      const int32_t* sorted_i, const float* T,
                                                                      int B, int K, int32_t* n_sched,
                                                                      int32_t* n_total) {
  __shared__ double s_wsum[kGreedyThreads / 64];
  __shared__ int s_wmin[kGreedyThreads / 64];
  __shared__ int s_stop;
  GreedyT t0;
  t0.load<kGreedyThreads>(T, B, K);
  for (int b = threadIdx.x; b < B; b += kGreedyThreads) n_sched[b] = 0;
  __syncthreads();
  sched_greedy<kGreedyThreads, false>(sorted_s, sorted_i, T, t0, B, K, n_sched, n_total, s_wsum, s_wmin, &s_stop,
                                      nullptr);
}

// Candidate sets up to kSchedLdsMax: each candidate's rank is summed from the
// partial ranks and the candidate is placed in schedule order in LDS by the
// workgroup that runs the greedy pass (no ordering round trip through memory).
constexpr int kSchedLdsMax = 8192;
__global__ __launch_bounds__(kGreedyThreads) void k_sched_greedy_lds(const float* surv, const int32_t* part, int S,
                                                                   const float* T, int B, int K, int32_t* n_sched,
                                                                   int32_t* n_total) {
  __shared__ float s_sorted_s[kSchedLdsMax];
  __shared__ int32_t s_sorted_i[kSchedLdsMax];
  __shared__ int s_cnt[kSchedLdsMax];
  __shared__ double s_wsum[kGreedyThreads / 64];
  __shared__ int s_wmin[kGreedyThreads / 64];
  __shared__ int s_stop;
  const int n = B * K;
  GreedyT t0;
  t0.load<kGreedyThreads>(T, B, K);
  for (int b = threadIdx.x; b < B; b += kGreedyThreads) s_cnt[b] = 0;
  // kBatchC candidates per thread at a time, all their loads in flight before the
  // first sum: kSchedSegMax segments each, unconditional (clamped) and masked after
  constexpr int kBatchC = 4;
  for (int u0 = 0; u0 * kGreedyThreads < n; u0 += kBatchC) {
    int v[kBatchC][kSchedSegMax];
    float sv[kBatchC];
#pragma unroll
    for (int u = 0; u < kBatchC; ++u) {
      const int i = min((int)threadIdx.x + (u0 + u) * kGreedyThreads, n - 1);
      sv[u] = surv[i];
#pragma unroll
      for (int q = 0; q < kSchedSegMax; ++q) v[u][q] = part[(size_t)(q < S ? q : 0) * n + i];
    }
#pragma unroll
    for (int u = 0; u < kBatchC; ++u) {
      const int i = (int)threadIdx.x + (u0 + u) * kGreedyThreads;
      if (i < n) {
        int r = 0;
#pragma unroll
        for (int q = 0; q < kSchedSegMax; ++q) r += q < S ? v[u][q] : 0;
        r = r < 0 ? 0 : (r >= n ? n - 1 : r);
        s_sorted_s[r] = sv[u];
        s_sorted_i[r] = i;
      }
    }
  }
  __syncthreads();
  sched_greedy<kGreedyThreads, true>(s_sorted_s, s_sorted_i, T, t0, B, K, n_sched, n_total, s_wsum, s_wmin, &s_stop,
                                     s_cnt);
}

// Asynchronous budget: the first M = lag_total - B candidates of the current
// schedule order are taken; one workgroup.
__global__ __launch_bounds__(kGreedyThreads) void k_sched_topk(const int32_t* sorted_i, const int32_t* lag_total,
                                                               int B, int K, int32_t* n_sched, int32_t* n_total) {
  const int n = B * K, tid = threadIdx.x;
  for (int b = tid; b < B; b += kGreedyThreads) n_sched[b] = 0;
  int M = *lag_total - B;
  M = M < 0 ? 0 : (M > n ? n : M);
  __syncthreads();  // the zeroed counts (workgroup release) before the counting atomics at L2
  for (int m = tid; m < M; m += kGreedyThreads) {
    int idx = sorted_i[m];
    idx = idx < 0 ? 0 : (idx >= n ? n - 1 : idx);
    atomicAdd(&n_sched[idx / K], 1);
  }
  if (tid == 0) *n_total = B + M;
}

// Fixed-length (mode 0) and survival-threshold (mode 1) baselines; one workgroup.
__global__ __launch_bounds__(kGreedyThreads) void k_sched_static(const float* surv, int B, int K, int mode,
                                                                 int gamma, float theta, int32_t* n_sched,
                                                                 int32_t* n_total) {
  __shared__ int s_sum[kGreedyThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int total = 0;
  for (int b = tid; b < B; b += kGreedyThreads) {
    int nb = gamma;
    if (mode == 1) {
      nb = 0;
      while (nb < K && surv[(size_t)b * K + nb] >= theta) ++nb;
    }
    n_sched[b] = nb;
    total += nb;
  }
  total = wave_sum_i(total);
  if (lane == 0) s_sum[wave] = total;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int w = 0; w < kGreedyThreads / 64; ++w) t += s_sum[w];
    *n_total = B + t;
  }
}

}  // namespace

hipError_t launch_conf(const dspark_problem& P, const ConfArgs& a, hipStream_t s) {
  const bool hb = P.hidden_dtype == DSPARK_BF16, wb = P.weight_dtype == DSPARK_BF16;
  const bool stage = P.d + P.r <= kConfWMax;  // d and r are multiples of 4, so the float4 copy is exact
  const size_t lds = stage ? (size_t)(P.d + P.r) * sizeof(float) : 0;
#define DSPARK_CONF(HT, WT)                                                                      \
  if (stage) hipLaunchKernelGGL((k_conf<HT, WT, true>), P.B, kConfThreads, lds, s, a);            \
  else hipLaunchKernelGGL((k_conf<HT, WT, false>), P.B, kConfThreads, 0, s, a);
  if (hb && wb) { DSPARK_CONF(uint16_t, uint16_t) }
  else if (hb) { DSPARK_CONF(uint16_t, float) }
  else if (wb) { DSPARK_CONF(float, uint16_t) }
  else { DSPARK_CONF(float, float) }
#undef DSPARK_CONF
  return hipGetLastError();
}

int sched_segments(int n) {
  const int s = (n + 255) / 256;
  return s < kSchedSegMax ? s : kSchedSegMax;
}

hipError_t launch_schedule(const dspark_problem& P, const float* surv, const float* T, int32_t* n_sched,
                           int32_t* n_total, int32_t* part, float* sorted_s, int32_t* sorted_i, hipStream_t s) {
  const int n = P.B * P.K;
  const int S = sched_segments(n);
  hipLaunchKernelGGL(k_sched_rank, dim3((n + 255) / 256, S), 256, 0, s, surv, n, S, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (n <= kSchedLdsMax) {
    hipLaunchKernelGGL(k_sched_greedy_lds, 1, kGreedyThreads, 0, s, surv, part, S, T, P.B, P.K, n_sched, n_total);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_sched_scatter, (n + kScatterThreads - 1) / kScatterThreads, kScatterThreads, 0, s, surv, part, S, n, sorted_s, sorted_i);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sched_greedy_global, 1, kGreedyThreads, 0, s, sorted_s, sorted_i, T, P.B, P.K, n_sched,
                     n_total);
  return hipGetLastError();
}

hipError_t launch_schedule_async(const dspark_problem& P, const float* surv_lag, const float* surv, const float* T,
                                 int32_t* n_sched, int32_t* n_total, int32_t* part, float* sorted_s,
                                 int32_t* sorted_i, int32_t* lag_n, int32_t* lag_total, hipStream_t s) {
  hipError_t e = launch_schedule(P, surv_lag, T, lag_n, lag_total, part, sorted_s, sorted_i, s);
  if (e != hipSuccess) return e;
  const int n = P.B * P.K;
  const int S = sched_segments(n);
  hipLaunchKernelGGL(k_sched_rank, dim3((n + 255) / 256, S), 256, 0, s, surv, n, S, part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sched_scatter, (n + kScatterThreads - 1) / kScatterThreads, kScatterThreads, 0, s, surv, part,
                     S, n, sorted_s, sorted_i);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sched_topk, 1, kGreedyThreads, 0, s, sorted_i, lag_total, P.B, P.K, n_sched, n_total);
  return hipGetLastError();
}

hipError_t launch_schedule_static(const dspark_problem& P, const float* surv, int mode, int gamma, float theta,
                                  int32_t* n_sched, int32_t* n_total, hipStream_t s) {
  hipLaunchKernelGGL(k_sched_static, 1, kGreedyThreads, 0, s, surv, P.B, P.K, mode, gamma, theta, n_sched, n_total);
  return hipGetLastError();
}

}  // namespace dspark
