// Fitting the Sequential Temperature Scaling temperatures (DSpark page, Method >
// Confidence-scheduled verification, the STS paragraph).
//
// Position by position, left to right: every candidate temperature of the grid
// (one workgroup row each, plus one row for temperature 1 on the raw running
// product) scores the Expected Calibration Error of the survival
//   S_k = S_{k-1} * sigmoid(logit(c_k) / tau)
// against "the first k positions were all accepted", over the samples that
// verified position k; the pick takes the smallest ECE (ties to the smallest
// grid index), fixes tau_k and advances every sample's running product past
// position k (fitted and raw) for the positions after it.
//
// Arithmetic is float64 (the fit is a handful of evaluations per sample and
// candidate; fp64 keeps the argmin a property of the data, not of the order of
// the sums).  Bin sums are accumulated per lane in LDS and reduced in a fixed
// order, so a fit is bit-reproducible.
#include "dspark_internal.hpp"

namespace dspark {
namespace {

constexpr int kStsThreads = 256;
constexpr int kStsBatch = 8;

// 1 / (1 + e^-t), formed from e^-|t| so that neither sign overflows.
__device__ __forceinline__ double sigmoid64(double t) {
  const double e = exp(-fabs(t));
  return t >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
}

__device__ __forceinline__ bool usable(double tau) { return isfinite(tau) && tau > 0.0; }

// zl[k][m] = ln c - ln(1 - c) of the raw confidence c[m][k]; the running
// products start at 1.
__global__ __launch_bounds__(kStsThreads) void k_sts_logit(const float* __restrict__ c, double* __restrict__ zl,
                                                           double* __restrict__ fit, double* __restrict__ raw,
                                                           int M, int K) {
  const size_t n = (size_t)M * K;
  for (size_t i = (size_t)blockIdx.x * kStsThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kStsThreads) {
    const int k = (int)(i / M), m = (int)(i - (size_t)k * M);
    const double x = (double)c[(size_t)m * K + k];
    zl[i] = log(x) - log1p(-x);
    if (k == 0) { fit[m] = 1.0; raw[m] = 1.0; }
  }
}

struct StsEceArgs {
  const double* zl;        // [K][M]
  const int32_t* acc;      // [M]
  const int32_t* nver;     // [M]
  const double* grid;      // [G]
  const double* fit;       // [M] product over positions < j with the fitted temperatures
  const double* raw;       // [M] same at temperature 1
  StsPart* part;           // [(G+1)][S][n_bins]
  int M, G, S, n_bins, j;
};

// One (candidate, sample split) pair per workgroup; row G is temperature 1 on
// the raw running product.
__global__ __launch_bounds__(kStsThreads) void k_sts_ece(StsEceArgs a) {
  // per-lane bin slots: prediction sum, and observed count (low 16 bits) plus
  // accepted count (high 16 bits); a lane sees at most ceil(M / S / 256) <= 65535
  // samples (M <= 2^24, S >= 1)
  __shared__ double s_sum[kStsBinsMax][kStsThreads];
  __shared__ uint32_t s_cl[kStsBinsMax][kStsThreads];
  __shared__ double r_sum[kStsBinsMax][16];
  __shared__ uint32_t r_cnt[kStsBinsMax][16], r_lab[kStsBinsMax][16];
  const int tid = threadIdx.x, g = blockIdx.x, s = blockIdx.y, nb = a.n_bins, j = a.j;
  const bool raw_row = g == a.G;
  const double tau = raw_row ? 1.0 : a.grid[g];
  if (!raw_row && !usable(tau)) return;  // never chosen; the pick skips it
  for (int b = 0; b < nb; ++b) { s_sum[b][tid] = 0.0; s_cl[b][tid] = 0u; }
  const int per = (a.M + a.S - 1) / a.S;
  const int m0 = s * per, m1 = min(a.M, m0 + per);
  const double* zj = a.zl + (size_t)j * a.M;
  const double* prod = raw_row ? a.raw : a.fit;
  // kStsBatch samples per thread at a time, every load issued before the first use
  for (int base = m0 + tid; base < m1; base += kStsThreads * kStsBatch) {
    double zv[kStsBatch], pv[kStsBatch];
    int nv[kStsBatch], av[kStsBatch];
#pragma unroll
    for (int u = 0; u < kStsBatch; ++u) {
      const int m = base + u * kStsThreads;
      const bool in = m < m1;
      nv[u] = in ? a.nver[m] : 0;
      av[u] = in ? a.acc[m] : 0;
      zv[u] = in ? zj[m] : 0.0;
      pv[u] = in ? prod[m] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < kStsBatch; ++u) {
      if (j + 1 > nv[u]) continue;  // also every slot past the split
      const double p = pv[u] * sigmoid64(raw_row ? zv[u] : zv[u] / tau);
      const int b = max(0, min((int)floor(p * (double)nb), nb - 1));
      s_sum[b][tid] += p;
      s_cl[b][tid] += av[u] >= j + 1 ? 0x10001u : 1u;
    }
  }
  __syncthreads();
  {  // bin b = tid / 16 sums lanes 16q .. 16q + 15 in order
    const int b = tid >> 4, q = tid & 15;
    if (b < nb) {
      double sum = 0.0;
      uint32_t cnt = 0u, lab = 0u;
      for (int l = 16 * q; l < 16 * q + 16; ++l) {
        const uint32_t cl = s_cl[b][l];
        sum += s_sum[b][l]; cnt += cl & 0xffffu; lab += cl >> 16;
      }
      r_sum[b][q] = sum; r_cnt[b][q] = cnt; r_lab[b][q] = lab;
    }
  }
  __syncthreads();
  if (tid < nb) {
    double sum = 0.0;
    uint32_t cnt = 0u, lab = 0u;
    for (int q = 0; q < 16; ++q) { sum += r_sum[tid][q]; cnt += r_cnt[tid][q]; lab += r_lab[tid][q]; }
    StsPart o;
    o.sum = sum; o.cnt = cnt; o.lab = lab;
    a.part[((size_t)g * a.S + s) * nb + tid] = o;
  }
}

constexpr int kPickThreads = 1024;
constexpr int kPickRows = kPickThreads / kStsBinsMax;  // candidates per pass

// Every workgroup takes the same argmin (smallest ECE, then smallest index),
// workgroup 0 stores it, and each advances the running products of its slice of
// samples past position j.  Per pass, thread (row, bin) sums the bin over the
// sample splits in order; the row's ECE then sums its bins in order.
__global__ __launch_bounds__(kPickThreads) void k_sts_pick(const StsPart* part, const double* grid, const double* zl,
                                                           double* fit, double* raw, int M, int G, int S, int nb,
                                                           int j, double* tau, int32_t* tau_idx, double* ece_fit,
                                                           double* ece_raw) {
  __shared__ double s_d[kPickRows][kStsBinsMax];
  __shared__ uint32_t s_n[kPickRows][kStsBinsMax];
  __shared__ double s_e[kPickRows];
  __shared__ int s_g[kPickRows];
  __shared__ double s_tau, s_raw_e;
  __shared__ uint32_t s_raw_n;
  const int tid = threadIdx.x, row = tid / kStsBinsMax, b = tid % kStsBinsMax;
  double best = 0.0;  // thread row < kPickRows keeps its running best over the passes
  int best_g = -1;
  double raw_e = 0.0;
  uint32_t raw_n = 0u;
  // operands of the product update (independent of the choice), loaded first
  constexpr int kUpd = 4;
  const double* zj = zl + (size_t)j * M;
  double zu[kUpd], fu[kUpd], ru[kUpd];
  const int mstride = gridDim.x * kPickThreads;
  const int mfirst = blockIdx.x * kPickThreads + tid;
#pragma unroll
  for (int u = 0; u < kUpd; ++u) {
    const int m = mfirst + u * mstride;
    const bool in = m < M;
    zu[u] = in ? zj[m] : 0.0;
    fu[u] = in ? fit[m] : 0.0;
    ru[u] = in ? raw[m] : 0.0;
  }
  for (int g0 = 0; g0 <= G; g0 += kPickRows) {
    const int g = g0 + row;
    double d = 0.0;
    uint32_t n = 0u;
    if (g <= G && b < nb) {
      double sum = 0.0;
      uint32_t lab = 0u;
      for (int s = 0; s < S; ++s) {
        const StsPart p = part[((size_t)g * S + s) * nb + b];
        sum += p.sum; lab += p.lab; n += p.cnt;
      }
      d = fabs(sum - (double)lab);
    }
    s_d[row][b] = d;
    s_n[row][b] = n;
    __syncthreads();
    if (tid < kPickRows) {
      const int gg = g0 + tid;
      double total = 0.0;
      uint32_t cnt = 0u;
      for (int q = 0; q < nb; ++q) { total += s_d[tid][q]; cnt += s_n[tid][q]; }
      const double e = cnt ? total / (double)cnt : 0.0;
      if (gg == G) { raw_e = e; raw_n = cnt; }
      else if (gg < G && usable(grid[gg]) && (best_g < 0 || e < best)) { best = e; best_g = gg; }
    }
    __syncthreads();
  }
  // the thread that met the raw row (row G % 64 of the last pass) publishes it;
  // then (ECE, index) is reduced over the rows, ties to the smaller index
  if (tid == G % kPickRows) { s_raw_e = raw_e; s_raw_n = raw_n; }
  if (tid < kPickRows) { s_e[tid] = best; s_g[tid] = best_g; }
  __syncthreads();
  for (int w = kPickRows / 2; w > 0; w >>= 1) {
    if (tid < w) {
      const double e2 = s_e[tid + w];
      const int g2 = s_g[tid + w];
      const int g1 = s_g[tid];
      if (g2 >= 0 && (g1 < 0 || e2 < s_e[tid] || (e2 == s_e[tid] && g2 < g1))) { s_e[tid] = e2; s_g[tid] = g2; }
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double er = s_raw_e;
    const uint32_t n = s_raw_n;
    const double nan = __longlong_as_double(0x7ff8000000000000ll);
    const bool chosen = n && s_g[0] >= 0;
    const double t = chosen ? grid[s_g[0]] : 1.0;
    s_tau = t;
    if (blockIdx.x == 0) {
      ece_raw[j] = n ? er : nan;
      tau[j] = t;
      tau_idx[j] = chosen ? s_g[0] : -1;
      ece_fit[j] = chosen ? s_e[0] : nan;
    }
  }
  __syncthreads();
  const double t = s_tau;
#pragma unroll
  for (int u = 0; u < kUpd; ++u) {
    const int m = mfirst + u * mstride;
    if (m < M) {
      fit[m] = fu[u] * sigmoid64(zu[u] / t);
      raw[m] = ru[u] * sigmoid64(zu[u]);
    }
  }
  for (int m = mfirst + kUpd * mstride; m < M; m += mstride) {
    const double z = zj[m];
    fit[m] = fit[m] * sigmoid64(z / t);
    raw[m] = raw[m] * sigmoid64(z);
  }
}

}  // namespace

int sts_splits(int M) {
  const int s = (M + 4095) / 4096;
  return s < 1 ? 1 : (s > 64 ? 64 : s);
}

StsLayout make_sts_layout(int M, int K, int G, int n_bins) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  StsLayout L;
  L.S = sts_splits(M);
  size_t o = 0;
  L.zl = o;   o = up(o + sizeof(double) * (size_t)M * K);
  L.fit = o;  o = up(o + sizeof(double) * (size_t)M);
  L.raw = o;  o = up(o + sizeof(double) * (size_t)M);
  L.part = o; o = up(o + sizeof(StsPart) * (size_t)(G + 1) * L.S * n_bins);
  L.total = o;
  return L;
}

hipError_t launch_sts_fit(int M, int K, const float* c, const int32_t* acc, const int32_t* nver, const double* grid,
                          int G, int n_bins, double* tau, int32_t* tau_idx, double* ece_fit, double* ece_raw,
                          void* ws, hipStream_t st) {
  const StsLayout L = make_sts_layout(M, K, G, n_bins);
  char* w = static_cast<char*>(ws);
  double* zl = reinterpret_cast<double*>(w + L.zl);
  double* fit = reinterpret_cast<double*>(w + L.fit);
  double* raw = reinterpret_cast<double*>(w + L.raw);
  StsPart* part = reinterpret_cast<StsPart*>(w + L.part);
  const size_t n = (size_t)M * K;
  if (n) {
    const size_t want = (n + kStsThreads - 1) / kStsThreads;
    hipLaunchKernelGGL(k_sts_logit, (int)(want < 4096 ? want : 4096), kStsThreads, 0, st, c, zl, fit, raw, M, K);
  }
  const int pick_blocks = M > 0 ? (M + 4095) / 4096 < 64 ? (M + 4095) / 4096 : 64 : 1;
  for (int j = 0; j < K; ++j) {
    StsEceArgs a;
    a.zl = zl; a.acc = acc; a.nver = nver; a.grid = grid; a.fit = fit; a.raw = raw;
    a.part = part; a.M = M; a.G = G; a.S = L.S; a.n_bins = n_bins; a.j = j;
    hipLaunchKernelGGL(k_sts_ece, dim3(G + 1, L.S), kStsThreads, 0, st, a);
    hipLaunchKernelGGL(k_sts_pick, pick_blocks, kPickThreads, 0, st, part, grid, zl, fit, raw, M, G, L.S, n_bins, j,
                       tau, tau_idx, ece_fit, ece_raw);
  }
  return hipGetLastError();
}

}  // namespace dspark
