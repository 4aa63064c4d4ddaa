// The device's random draws on given inputs, so that a test can check them
// against their published definition (Philox4x32-10, Salmon et al., SC'11) and
// the uniform and Gumbel transforms the cycle uses, independently of any
// sampling decision.  The kernels call the same device functions as the draft
// and verification kernels.
#include "dspark_internal.hpp"

namespace dspark {
namespace {

__global__ __launch_bounds__(256) void k_probe_philox(Key key, const uint4* ctr, int n, uint4* out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint4 c = ctr[i];
  const Words4 w = philox4x32_10(c.x, c.y, c.z, c.w, key.lo, key.hi);
  out[i] = make_uint4(w.w[0], w.w[1], w.w[2], w.w[3]);
}

__global__ __launch_bounds__(256) void k_probe_transforms(const uint32_t* w, int m, float* u, float* g) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= m) return;
  const uint32_t x = w[i];
  u[i] = uniform01(x);
  g[i] = gumbel_from_word(x);
}

}  // namespace
}  // namespace dspark

using namespace dspark;

extern "C" dspark_status dspark_probe_draws(uint64_t seed, const uint32_t* ctr, int32_t n, uint32_t* out_words,
                                            const uint32_t* w, int32_t m, float* uniform, float* gumbel,
                                            hipStream_t stream) {
  const AbiRange range("dspark_probe_draws");
  if (n < 0 || m < 0) return DSPARK_E_INVALID;
  if (n > 0 && (!ctr || !out_words || (uintptr_t)ctr % 16 || (uintptr_t)out_words % 16)) return DSPARK_E_POINTER;
  if (m > 0 && (!w || !uniform || !gumbel || (uintptr_t)w % 4 || (uintptr_t)uniform % 4 || (uintptr_t)gumbel % 4))
    return DSPARK_E_POINTER;
  (void)hipGetLastError();
  const Key key{(uint32_t)seed, (uint32_t)(seed >> 32)};
  if (n > 0)
    hipLaunchKernelGGL(k_probe_philox, (n + 255) / 256, 256, 0, stream, key, reinterpret_cast<const uint4*>(ctr), n,
                       reinterpret_cast<uint4*>(out_words));
  if (hipGetLastError() != hipSuccess) return DSPARK_E_LAUNCH;
  if (m > 0) hipLaunchKernelGGL(k_probe_transforms, (m + 255) / 256, 256, 0, stream, w, m, uniform, gumbel);
  if (hipGetLastError() != hipSuccess) return DSPARK_E_LAUNCH;
  return DSPARK_OK;
}
