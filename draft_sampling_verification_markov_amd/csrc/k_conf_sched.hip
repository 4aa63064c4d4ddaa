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
template <typename HT, typename WT>
__device__ __forceinline__ float dot_h(const HT* h, const float* w, int d, int lane);

template <>
__device__ __forceinline__ float dot_h<uint16_t, uint16_t>(const uint16_t* h, const float* w, int d, int lane) {
  float acc = 0.f;
  for (int i = lane * 8; i < d; i += 64 * 8) {
    const uint4 hv = *reinterpret_cast<const uint4*>(h + i);
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
__device__ __forceinline__ float dot_h<float, float>(const float* h, const float* w, int d, int lane) {
  float acc = 0.f;
  for (int i = lane * 4; i < d; i += 64 * 4) {
    const float4 hv = *reinterpret_cast<const float4*>(h + i);
    const float4 wv = *reinterpret_cast<const float4*>(w + i);
    acc = fmaf(hv.x, wv.x, acc);
    acc = fmaf(hv.y, wv.y, acc);
    acc = fmaf(hv.z, wv.z, acc);
    acc = fmaf(hv.w, wv.w, acc);
  }
  return acc;
}

// Same loops with the tag types used for dispatch (h and E may differ in dtype).
template <typename T>
__device__ __forceinline__ float dot_vec(const T* x, const float* w, int n, int lane) {
  return dot_h<T, T>(x, w, n, lane);
}

template <typename HT, typename WT>
__global__ __launch_bounds__(256) void k_conf(ConfArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, d = a.d, r = a.r;
  __shared__ float s_c[64];
  const HT* h = static_cast<const HT*>(a.h);
  const WT* E = static_cast<const WT*>(a.E);
  for (int k = wave; k < K; k += 4) {
    const int prev = clamp_id(k == 0 ? a.anchor[b] : a.tok[(size_t)b * K + k - 1], a.V);
    float z = dot_vec<HT>(h + ((size_t)b * K + k) * d, a.w_c, d, lane);
    z += dot_vec<WT>(E + (size_t)prev * r, a.w_c + d, r, lane);
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
// Rank of every candidate in the order (survival desc, request asc, position
// asc).  With candidate index i = b*K + (k-1), candidate j precedes i iff
// s_j > s_i, or s_j == s_i and j < i.  Each workgroup ranks 64 candidates
// against all n, streaming the survivals through LDS in 1024-entry tiles; its
// four waves split every tile and their counts are summed at the end.
constexpr int kRankCands = 64;
constexpr int kRankTile = 1024;

__global__ __launch_bounds__(256) void k_sched_rank(const float* surv, int n, int32_t* sorted) {
  __shared__ float tile[kRankTile];
  __shared__ int cnt[4][kRankCands];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = blockIdx.x * kRankCands + lane;
  const float si = i < n ? surv[i] : 0.f;
  int count = 0;
  for (int t0 = 0; t0 < n; t0 += kRankTile) {
    __syncthreads();
    for (int j = tid; j < kRankTile; j += 256) tile[j] = t0 + j < n ? surv[t0 + j] : -INFINITY;
    __syncthreads();
    const int lo = wave * (kRankTile / 4);
    const int hi = min(lo + kRankTile / 4, n - t0);
    for (int jj = lo; jj < hi; ++jj) {
      const float sj = tile[jj];
      const int j = t0 + jj;
      count += (sj > si) || (sj == si && j < i);
    }
  }
  cnt[wave][lane] = count;
  __syncthreads();
  if (wave == 0 && i < n) {
    const int rank = cnt[0][lane] + cnt[1][lane] + cnt[2][lane] + cnt[3][lane];
    if (rank >= 0 && rank < n) sorted[rank] = i;
  }
}

constexpr int kScanThreads = 1024;

// One workgroup: prefix sums of the sorted survivals (double), the greedy
// test for every candidate, the first refusal, and the per-request counts.
__global__ __launch_bounds__(kScanThreads) void k_sched_scan(const float* surv, const float* T, int B, int K,
                                                             const int32_t* sorted, int32_t* n_sched,
                                                             int32_t* n_total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = B * K;
  __shared__ double s_wsum[kScanThreads / 64];
  __shared__ int s_wmin[kScanThreads / 64];
  __shared__ int s_stop;
  const int lo = (int)(((long long)tid * n) / kScanThreads);
  const int hi = (int)(((long long)(tid + 1) * n) / kScanThreads);

  for (int b = tid; b < B; b += kScanThreads) n_sched[b] = 0;
  __threadfence();  // the zeros are visible before any counting atomic below

  double local = 0.0;
  for (int m = lo; m < hi; ++m) {
    int idx = sorted[m];
    idx = idx < 0 ? 0 : (idx >= n ? n - 1 : idx);
    local += (double)surv[idx];
  }
  // exclusive scan of the per-thread sums
  double incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  double wbase = 0.0;
  for (int w = 0; w < wave; ++w) wbase += s_wsum[w];
  double A = (double)B + wbase + (incl - local);

  int first = n;
  int N = B + lo;
  for (int m = lo; m < hi; ++m) {
    int idx = sorted[m];
    idx = idx < 0 ? 0 : (idx >= n ? n - 1 : idx);
    const double s = (double)surv[idx];
    const double lhs = (A + s) * (double)T[N];
    const double rhs = A * (double)T[N + 1];
    if (!(lhs >= rhs)) {
      first = m;
      break;
    }
    A += s;
    ++N;
  }
  // first refusal over the workgroup
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o));
  if (lane == 0) s_wmin[wave] = first;
  __syncthreads();
  if (tid == 0) {
    int f = s_wmin[0];
    for (int w = 1; w < kScanThreads / 64; ++w) f = min(f, s_wmin[w]);
    s_stop = f;
    *n_total = B + f;
  }
  __syncthreads();
  const int stop = s_stop;
  __threadfence_block();
  for (int m = tid; m < stop; m += kScanThreads) {
    int idx = sorted[m];
    idx = idx < 0 ? 0 : (idx >= n ? n - 1 : idx);
    atomicAdd(&n_sched[idx / K], 1);
  }
}

}  // namespace

hipError_t launch_conf(const dspark_problem& P, const ConfArgs& a, hipStream_t s) {
  const bool hb = P.hidden_dtype == DSPARK_BF16, wb = P.weight_dtype == DSPARK_BF16;
  if (hb && wb) hipLaunchKernelGGL((k_conf<uint16_t, uint16_t>), P.B, 256, 0, s, a);
  else if (hb) hipLaunchKernelGGL((k_conf<uint16_t, float>), P.B, 256, 0, s, a);
  else if (wb) hipLaunchKernelGGL((k_conf<float, uint16_t>), P.B, 256, 0, s, a);
  else hipLaunchKernelGGL((k_conf<float, float>), P.B, 256, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_schedule(const dspark_problem& P, const float* surv, const float* T, int32_t* n_sched,
                           int32_t* n_total, int32_t* sorted, hipStream_t s) {
  const int n = P.B * P.K;
  hipLaunchKernelGGL(k_sched_rank, (n + kRankCands - 1) / kRankCands, 256, 0, s, surv, n, sorted);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sched_scan, 1, kScanThreads, 0, s, surv, T, P.B, P.K, sorted, n_sched, n_total);
  return hipGetLastError();
}

}  // namespace dspark
