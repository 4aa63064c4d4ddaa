// Debug checks: scans of a call's inputs and outputs that raise bits of a
// per-device flag word, never a trap.  The library built with
// DSPARK_DEBUG_CHECKS runs them around its kernels (the input contract of
// dspark.h: finite logits and factors, token ids in [0, V), a positive finite
// step-time table; the output ranges it documents); dspark_debug_flags reads and
// clears the word.  The kernels themselves are in every build.
#include <mutex>

#include "dspark_internal.hpp"

namespace dspark {
namespace {

// the flag word: raised with device-scope atomic ORs (vector memory), read and
// cleared by the host through its address
static __device__ __align__(256) unsigned int debug_flags_word[64];

constexpr int kDbgThreads = 256;
constexpr int kDbgMaxGrid = 1024;
constexpr int kDbgMaxDevices = 64;

// non-finite: all exponent bits set (infinity or NaN)
__device__ __forceinline__ bool nonfinite_bf16(uint32_t half) { return (half & 0x7F80u) == 0x7F80u; }
__device__ __forceinline__ bool nonfinite_f32(uint32_t w) { return (w & 0x7F800000u) == 0x7F800000u; }

// n elements of 2 (bf16) or 4 (fp32) bytes at x, 16-byte aligned; any non-finite one raises bit
__global__ __launch_bounds__(kDbgThreads) void k_dbg_nonfinite(const void* x, size_t n, int bf16, unsigned bit,
                                                                unsigned* word) {
  const size_t per16 = bf16 ? 8 : 4;
  const size_t n16 = n / per16;
  const uint4* v = static_cast<const uint4*>(x);
  bool bad = false;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x) {
    const uint4 q = v[i];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bad |= bf16 ? (nonfinite_bf16(w[j] & 0xFFFFu) || nonfinite_bf16(w[j] >> 16)) : nonfinite_f32(w[j]);
  }
  // the tail past the last 16-byte piece
  const size_t tail = n16 * per16 + (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tail < n) {
    if (bf16)
      bad |= nonfinite_bf16(static_cast<const uint16_t*>(x)[tail]);
    else
      bad |= nonfinite_f32(static_cast<const uint32_t*>(x)[tail]);
  }
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && (threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(word, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// n int32 values at x; any outside [lo, hi] raises bit
__global__ __launch_bounds__(kDbgThreads) void k_dbg_range_i32(const int32_t* x, size_t n, int32_t lo, int32_t hi,
                                                                unsigned bit, unsigned* word) {
  bool bad = false;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    bad |= x[i] < lo || x[i] > hi;
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && (threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(word, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// n fp32 values at x; any outside [lo, hi] or NaN raises bit (the comparisons
// are false for NaN)
__global__ __launch_bounds__(kDbgThreads) void k_dbg_range_f32(const float* x, size_t n, float lo, float hi,
                                                                unsigned bit, unsigned* word) {
  bool bad = false;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    bad |= !(x[i] >= lo && x[i] <= hi);
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && (threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(word, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// one workgroup: n_sched[b] in [0, K] and n_total = B + their sum
__global__ __launch_bounds__(kDbgThreads) void k_dbg_schedule(const int32_t* n_sched, const int32_t* n_total, int B,
                                                               int K, unsigned bit, unsigned* word) {
  __shared__ int s_sum[kDbgThreads / 64];
  int sum = 0;
  bool bad = false;
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int n = n_sched[b];
    bad |= n < 0 || n > K;
    sum += n;
  }
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if ((threadIdx.x & 63) == 0) s_sum[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int w = 0; w < kDbgThreads / 64; ++w) tot += s_sum[w];
    bad |= tot + B != n_total[0];
  }
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && (threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(word, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// per request: n_acc in [0, n_sched], the n_acc + 1 emitted tokens and the next
// anchor in [0, V), the residual mass in [0, 1] or NaN (no rejection)
__global__ __launch_bounds__(kDbgThreads) void k_dbg_verify(const int32_t* n_sched, const int32_t* out_tok,
                                                             const int32_t* n_acc, const int32_t* next_anchor,
                                                             const float* resid_mass, int B, int K, int V,
                                                             unsigned bit, unsigned* word) {
  bool bad = false;
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < B; b += gridDim.x * blockDim.x) {
    const int n = n_acc[b], ns = n_sched[b];
    bad |= n < 0 || n > ns || ns < 0 || ns > K;
    const int ne = (n >= 0 && n <= K ? n : 0) + 1;
    for (int j = 0; j < ne; ++j) {
      const int t = out_tok[(size_t)b * (K + 1) + j];
      bad |= t < 0 || t >= V;
    }
    bad |= next_anchor[b] < 0 || next_anchor[b] >= V;
    const float m = resid_mass[b];
    bad |= !(m != m || (m >= 0.f && m <= 1.f + 1e-5f));
  }
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && (threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(word, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int grid_for(size_t n) {
  const size_t g = (n + kDbgThreads - 1) / kDbgThreads;
  return (int)(g < 1 ? 1 : (g > (size_t)kDbgMaxGrid ? (size_t)kDbgMaxGrid : g));
}

}  // namespace

hipError_t debug_word(unsigned** out) {
  static std::mutex mu;
  static unsigned* ptr[kDbgMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDbgMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(debug_flags_word));
    if (e != hipSuccess) return e;
    ptr[dev] = static_cast<unsigned*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

hipError_t debug_scan_nonfinite(const void* x, size_t n, bool bf16, unsigned bit, hipStream_t s) {
  if (n == 0) return hipSuccess;
  unsigned* w = nullptr;
  hipError_t e = debug_word(&w);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dbg_nonfinite, grid_for((n + 7) / 8), kDbgThreads, 0, s, x, n, bf16 ? 1 : 0, bit, w);
  return hipGetLastError();
}

hipError_t debug_scan_range_i32(const int32_t* x, size_t n, int32_t lo, int32_t hi, unsigned bit, hipStream_t s) {
  if (n == 0) return hipSuccess;
  unsigned* w = nullptr;
  hipError_t e = debug_word(&w);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dbg_range_i32, grid_for(n), kDbgThreads, 0, s, x, n, lo, hi, bit, w);
  return hipGetLastError();
}

hipError_t debug_scan_range_f32(const float* x, size_t n, float lo, float hi, unsigned bit, hipStream_t s) {
  if (n == 0) return hipSuccess;
  unsigned* w = nullptr;
  hipError_t e = debug_word(&w);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dbg_range_f32, grid_for(n), kDbgThreads, 0, s, x, n, lo, hi, bit, w);
  return hipGetLastError();
}

hipError_t debug_check_schedule(const int32_t* n_sched, const int32_t* n_total, int B, int K, unsigned bit,
                                hipStream_t s) {
  unsigned* w = nullptr;
  hipError_t e = debug_word(&w);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dbg_schedule, 1, kDbgThreads, 0, s, n_sched, n_total, B, K, bit, w);
  return hipGetLastError();
}

hipError_t debug_check_verify(const int32_t* n_sched, const int32_t* out_tok, const int32_t* n_acc,
                              const int32_t* next_anchor, const float* resid_mass, int B, int K, int V, unsigned bit,
                              hipStream_t s) {
  unsigned* w = nullptr;
  hipError_t e = debug_word(&w);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dbg_verify, grid_for((size_t)B), kDbgThreads, 0, s, n_sched, out_tok, n_acc, next_anchor,
                     resid_mass, B, K, V, bit, w);
  return hipGetLastError();
}

}  // namespace dspark
