// Device helpers shared by the dspark kernels: Philox4x32-10, the uniform and
// Gumbel transforms, bf16 unpacking, and wave/block reductions.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

// Vocabulary chunk of the two-level Gumbel-max draw.
constexpr int kChunk = 128;

// Purposes of the random draws of one cycle (counter word 3).
enum : uint32_t {
  kDraftChunk = 1,
  kDraftElem = 2,
  kAccept = 3,
  kResidChunk = 4,
  kResidElem = 5,
  kBonusChunk = 6,
  kBonusElem = 7,
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Words4 {
  uint32_t w[4];
};

// Philox4x32 with ten rounds (Salmon, Moraes, Dror, Shaw, SC'11): counter words
// 0 and 2 are multiplied by the two round multipliers into 64-bit products whose
// halves are mixed with words 1, 3 and the key; the key advances by the two
// Weyl increments between rounds.
__device__ __forceinline__ Words4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  Words4 r;
  r.w[0] = c0;
  r.w[1] = c1;
  r.w[2] = c2;
  r.w[3] = c3;
  return r;
}

struct Key {
  uint32_t lo, hi;
};

__device__ __forceinline__ Key make_key(uint64_t seed) { return Key{(uint32_t)seed, (uint32_t)(seed >> 32)}; }

// The four words of counter (idx >> 2, b, k, purpose); draw idx is word idx & 3.
__device__ __forceinline__ Words4 draw_quad(Key key, uint32_t idx, uint32_t b, uint32_t k, uint32_t purpose) {
  return philox4x32_10(idx >> 2, b, k, purpose, key.lo, key.hi);
}

__device__ __forceinline__ uint32_t draw_word(Key key, uint32_t idx, uint32_t b, uint32_t k, uint32_t purpose) {
  const Words4 q = draw_quad(key, idx, b, k, purpose);
  const uint32_t s = idx & 3u;
  return s == 0 ? q.w[0] : s == 1 ? q.w[1] : s == 2 ? q.w[2] : q.w[3];
}

// Odd multiple of 2^-24 in (0, 1); the 24-bit integer converts exactly.
__device__ __forceinline__ float uniform01(uint32_t w) { return (float)((w >> 8) | 1u) * 0x1p-24f; }

// -ln(-ln u); for u >= 1/2, -ln u is taken as -log1p(-(1 - u)) with 1 - u exact,
// which keeps the largest Gumbel values accurate.  Accurate libm calls, no
// fast-math approximations.
__device__ __forceinline__ float gumbel_from_word(uint32_t w) {
  const float u = uniform01(w);
  const float e = (u >= 0.5f) ? -log1pf(-(1.0f - u)) : -logf(u);
  return -logf(e);
}

// 2^x - 1 for 0 <= x <= 1/4 without the cancellation of exp2(x) - 1: the power
// series of e^y - 1 at y = x ln 2 through y^6 (coefficients (ln 2)^k / k!; the
// remainder is below 6e-9 of the result on this range), in Horner form.
__device__ __forceinline__ float exp2m1_small(float x) {
  float p = 1.5403530393381608e-04f;
  p = fmaf(x, p, 1.3333558146428443e-03f);
  p = fmaf(x, p, 9.618129107628477e-03f);
  p = fmaf(x, p, 5.550410866482158e-02f);
  p = fmaf(x, p, 2.402265069591007e-01f);
  p = fmaf(x, p, 6.931471805599453e-01f);
  return x * p;
}

// One vocabulary entry of a rejected position's residual max(0, p - q), in the
// row's reference units: p^ = 2^(t s2 - lp2) with t the target logit, q^ =
// 2^((z + bias) s2 - lq2) with z the base draft logit and bias the Markov term,
// s2 = log2(e) / T_s and lp2, lq2 the log2-partitions the row is referred to.
// The draft logit z + bias is never rounded as one number: q^'s exponent is
// fma(bias, s2, fma(z, s2, -lq2)), and d = log2(p^ / q^) is
// ((t - z) - bias) s2 - (lp2 - lq2) with t - z exact, so neither carries a
// rounding at the logits' magnitude (a bias accumulated onto the logit would
// round at every step of the contraction).  The weight is q^ (2^d - 1) for
// 0 < d <= 1/4 (no cancellation where p and q are close), p^ - q^ for d > 1/4
// (where 2^d - 1 > 0.189 bounds the cancellation to a few ulps) and 0 otherwise.  dlp = lp2 - lq2; a row without a draft term (a bonus row)
// passes lq2 = +inf and dlp = -inf, and gets r = p^; an entry past the end of
// the row passes t = z = -inf and gets zeros.  Every kernel that forms residual
// weights uses this function, so the chunk masses of the resample pass and the
// entry weights of the final draw come from one formula.
// qa is q^ where d > 0 (the entries the residual keeps), else 0: the residual
// mass normalised by the row's own sums of p^ and q^ is then
// (sum r + sum qa) / sum p^ - sum qa / sum q^.
struct ResidEntry {
  float p, q, r, qa;
};
__device__ __forceinline__ ResidEntry resid_entry(float t, float z, float bias, float s2, float lp2, float lq2,
                                                  float dlp) {
  ResidEntry e;
  e.p = __builtin_amdgcn_exp2f(fmaf(t, s2, -lp2));
  e.q = __builtin_amdgcn_exp2f(fmaf(bias, s2, fmaf(z, s2, -lq2)));
  const float d = fmaf((t - z) - bias, s2, -dlp);
  const float small = e.q * exp2m1_small(d);
  e.r = d > 0.25f ? e.p - e.q : (d > 0.f ? small : 0.f);
  e.qa = d > 0.f ? e.q : 0.f;
  return e;
}
// Running sums of the residual terms of one row in two interleaved partials
// per quantity (entry i goes to partial i & 1), so that a sum of n terms has
// n / 2 + 1 roundings in its longest chain instead of n.
struct ResidSums {
  float r[2], p[2], q[2], qa[2];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int j = 0; j < 2; ++j) r[j] = p[j] = q[j] = qa[j] = 0.f;
  }
  __device__ __forceinline__ void add(int i, const ResidEntry& e) {
    r[i & 1] += e.r;
    p[i & 1] += e.p;
    q[i & 1] += e.q;
    qa[i & 1] += e.qa;
  }
  __device__ __forceinline__ static float fold(const float (&x)[2]) { return x[0] + x[1]; }
};
// The residual mass of a row from the fp64 sums of r, qa, p^ and q^ over the
// whole vocabulary (the resample pass's partials merged): p = p^ / Zp and
// q = q^ / Zq exactly, whatever the error of the log-partitions the entries
// were referred to.
__device__ __forceinline__ double resid_mass_normalised(double R, double QA, double Zp, double Zq) {
  return R / Zp + QA * ((Zq - Zp) / (Zp * Zq));
}

// bf16 halves of a packed 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
// acc + (lo(a) lo(b) + hi(a) hi(b)) for two packed bf16 pairs: one v_dot2c_f32_bf16
// (measured on this part: correctly rounded more often than two chained fmas)
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  bf16x2_t x, y;
  __builtin_memcpy(&x, &a, 4);
  __builtin_memcpy(&y, &b, 4);
  return __builtin_amdgcn_fdot2_f32_bf16(x, y, acc, false);
}
// the dot product of two 16-byte pieces of bf16 rows (8 products, in order of the pairs)
__device__ __forceinline__ float dot_bf16x8(uint4 e, uint4 w) {
  float acc = dot2_bf16(e.x, w.x, 0.f);
  acc = dot2_bf16(e.y, w.y, acc);
  acc = dot2_bf16(e.z, w.z, acc);
  return dot2_bf16(e.w, w.w, acc);
}

// Agent-scope (device-wide) relaxed loads and stores: past the L2, which one
// XCD does not keep coherent with another's.
__device__ __forceinline__ unsigned ld_agent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 8-byte words past the L2 (an XCD's L2 is not kept coherent with another's):
// a 32-bit value in the low half and its tag in the high half, so that one
// single-copy-atomic load returns the value together with the proof of which
// position (and launch) wrote it
__device__ __forceinline__ void st_tagged(unsigned long long* p, uint32_t v, uint32_t tag) {
  __hip_atomic_store(p, ((unsigned long long)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_tagged(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Poll N consecutive tagged words of this lane until every tag is `expect`;
// bounded: past `limit` polls (at once if the flag is already set) the
// time-out flag is set and the words are returned as they are.  Lanes poll
// independently; the wave leaves when every lane is done.
template <int N>
__device__ __forceinline__ void poll_tagged(const unsigned long long* p, uint32_t expect, unsigned* flag,
                                            uint32_t limit, uint32_t (&v)[N]) {
  unsigned spins = ld_agent(flag) ? limit : 0u;
  for (;;) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const unsigned long long w = ld_tagged(p + i);
      v[i] = (uint32_t)w;
      ok = ok && (uint32_t)(w >> 32) == expect;
    }
    if (ok) break;
    if (++spins > limit) {
      st_agent(flag, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}
// Workgroup barrier ordering LDS only: this wave's LDS operations complete
// first; vector-memory operations (LDS DMA included) are the caller's to wait
// for.  __syncthreads() carries a release fence that drains every load of the
// wave, prefetches meant to stay in flight included.  The memory clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds_only() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// waits until every vector-memory operation of this wave has completed
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order), lgkm and export counters untouched
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// 128-bit buffer descriptor over [base, base + bytes) (raw; reads past the end return 0)
// four dwords, the result type of a 16-byte buffer load
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4_t;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// float -> bfloat16 bits, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
// eight consecutive floats rounded to bfloat16, as one 16-byte piece
__device__ __forceinline__ uint4 bf16x8_from_f32(const float* p) {
  const float4 x0 = reinterpret_cast<const float4*>(p)[0], x1 = reinterpret_cast<const float4*>(p)[1];
  return make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w), pack_bf16x2(x1.x, x1.y),
                    pack_bf16x2(x1.z, x1.w));
}

// Token id used as an index, clamped into [0, V) so that a corrupt id cannot
// address outside the factor tables.
__device__ __forceinline__ int clamp_id(int v, int V) { return v < 0 ? 0 : (v >= V ? V - 1 : v); }

// Argmax with the smallest-index tie-break.
__device__ __forceinline__ bool better(float s, int i, float best, int best_i) {
  return s > best || (s == best && i < best_i);
}

// The two half-wave values of x seen from any lane: {x[l & 31], x[(l & 31) + 32]}.
// One VALU lane swap (gfx950), no trip through the LDS crossbar; both halves
// receive the operands in the same order, so a combination is bitwise equal.
__device__ __forceinline__ float2 halves32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves32_max(float x) { const float2 h = halves32(x); return fmaxf(h.x, h.y); }
// The same sum of the two half-wave values in float64 (both 32-bit halves swapped alike).
__device__ __forceinline__ double halves32_sum_d(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const auto lo = __builtin_amdgcn_permlane32_swap((unsigned)u, (unsigned)u, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((unsigned)(u >> 32), (unsigned)(u >> 32), false, false);
  const double a = __longlong_as_double((long long)(((unsigned long long)hi[0] << 32) | lo[0]));
  const double b = __longlong_as_double((long long)(((unsigned long long)hi[1] << 32) | lo[1]));
  return a + b;
}
__device__ __forceinline__ float halves32_sum(float x) { const float2 h = halves32(x); return h.x + h.y; }

// Whole-wave reductions on the VALU cross-lane paths instead of the LDS
// crossbar (ds_bpermute, which __shfl_xor becomes, costs a round trip through
// the LDS unit per step): DPP quad permutes pair lanes i and i ^ 1, then i and
// i ^ 2; once every lane of a quad holds the quad's value, row_half_mirror
// (i <-> 7 - i) joins the two quads of an octet and row_mirror (i <-> 15 - i)
// the two octets of a row; v_permlane16_swap and v_permlane32_swap join rows.
// Each step combines a lane's value with its partner's by a commutative
// operation (or takes the two swapped values in a fixed order), so every lane
// ends with the same bitwise result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
// {x of the lane with bit 4 clear, x of the lane with bit 4 set}, from either
__device__ __forceinline__ float2 rows16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int2 rows16_i(int x) {
  const auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  return make_int2((int)r[0], (int)r[1]);
}
__device__ __forceinline__ int2 halves32_i(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return make_int2((int)r[0], (int)r[1]);
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  float2 h = rows16(v);
  v = fmaxf(h.x, h.y);
  h = halves32(v);
  return fmaxf(h.x, h.y);
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  float2 h = rows16(v);
  v = h.x + h.y;
  h = halves32(v);
  return h.x + h.y;
}

// float64 sum over the wave (ds_bpermute exchanges; for once-per-row merges)
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<kDppXor1>(v));
  v = min(v, dpp_i<kDppXor2>(v));
  v = min(v, dpp_i<kDppHalfMirror>(v));
  v = min(v, dpp_i<kDppMirror>(v));
  int2 h = rows16_i(v);
  v = min(h.x, h.y);
  h = halves32_i(v);
  return min(h.x, h.y);
}

__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<kDppXor1>(v);
  v += dpp_i<kDppXor2>(v);
  v += dpp_i<kDppHalfMirror>(v);
  v += dpp_i<kDppMirror>(v);
  int2 h = rows16_i(v);
  v = h.x + h.y;
  h = halves32_i(v);
  return h.x + h.y;
}

// Inclusive prefix sum over the wave in fp64 on the same VALU paths: DPP
// row_shr 1, 2, 4, 8 (bound_ctrl: a lane with no source in its row of 16 adds
// zero) scan each row, row_bcast:15 adds row 0's (row 2's) total to row 1
// (row 3), row_bcast:31 adds the first half's total to the second.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_d(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, ROWMASK, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, ROWMASK, 0xF, true);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
__device__ __forceinline__ double wave_scan_incl(double v) {
  v += dpp_d<0x111, 0xF>(v);
  v += dpp_d<0x112, 0xF>(v);
  v += dpp_d<0x114, 0xF>(v);
  v += dpp_d<0x118, 0xF>(v);
  v += dpp_d<0x142, 0xA>(v);
  v += dpp_d<0x143, 0xC>(v);
  return v;
}

__device__ __forceinline__ void argmax_step(float& s, int& i, float so, int io) {
  if (better(so, io, s, i)) {
    s = so;
    i = io;
  }
}
__device__ __forceinline__ void wave_argmax(float& s, int& i) {
  argmax_step(s, i, dpp_f<kDppXor1>(s), dpp_i<kDppXor1>(i));
  argmax_step(s, i, dpp_f<kDppXor2>(s), dpp_i<kDppXor2>(i));
  argmax_step(s, i, dpp_f<kDppHalfMirror>(s), dpp_i<kDppHalfMirror>(i));
  argmax_step(s, i, dpp_f<kDppMirror>(s), dpp_i<kDppMirror>(i));
  float2 hs = rows16(s);
  int2 hi = rows16_i(i);
  s = hs.x;
  i = hi.x;
  argmax_step(s, i, hs.y, hi.y);
  hs = halves32(s);
  hi = halves32_i(i);
  s = hs.x;
  i = hi.x;
  argmax_step(s, i, hs.y, hi.y);
}

// Combine two (max, sum of 2^(x - max)) pairs in base 2.
__device__ __forceinline__ void lse2_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * exp2f(m - mn) + s2 * exp2f(m2 - mn);
  m = mn;
}

// lse2_merge over the whole wave, on the same cross-lane paths as wave_sum
// (the merge is symmetric in its two operands up to the order of one addition,
// which is commutative, so every lane ends with the same result)
__device__ __forceinline__ void wave_lse2_merge(float& m, float& s) {
  lse2_merge(m, s, dpp_f<kDppXor1>(m), dpp_f<kDppXor1>(s));
  lse2_merge(m, s, dpp_f<kDppXor2>(m), dpp_f<kDppXor2>(s));
  lse2_merge(m, s, dpp_f<kDppHalfMirror>(m), dpp_f<kDppHalfMirror>(s));
  lse2_merge(m, s, dpp_f<kDppMirror>(m), dpp_f<kDppMirror>(s));
  float2 hm = rows16(m), hs = rows16(s);
  m = hm.x;
  s = hs.x;
  lse2_merge(m, s, hm.y, hs.y);
  hm = halves32(m);
  hs = halves32(s);
  m = hm.x;
  s = hs.x;
  lse2_merge(m, s, hm.y, hs.y);
}


// Logit at vocabulary id v of a row (bf16 bits or fp32).
template <typename ZT>
__device__ __forceinline__ float logit_at(const ZT* row, int v);
template <>
__device__ __forceinline__ float logit_at<uint16_t>(const uint16_t* row, int v) { return bf16_to_f32(row[v]); }
template <>
__device__ __forceinline__ float logit_at<float>(const float* row, int v) { return row[v]; }

// Dot product of E[prev] with Wt[v] over a contiguous half of the rank.
template <typename WT>
__device__ __forceinline__ float half_dot(const WT* E, const WT* Wt, int prev, int v, int r, int h);

template <>
__device__ __forceinline__ float half_dot<uint16_t>(const uint16_t* E, const uint16_t* Wt, int prev, int v, int r,
                                                    int h) {
  const int n = r >> 1;
  const uint4* e = reinterpret_cast<const uint4*>(E + (size_t)prev * r + h * n);
  const uint4* w = reinterpret_cast<const uint4*>(Wt + (size_t)v * r + h * n);
  float acc = 0.f;
  for (int j = 0; j < n / 8; ++j) {
    const uint4 ev = e[j], wv = w[j];
    acc = fmaf(bf16_lo(ev.x), bf16_lo(wv.x), acc);
    acc = fmaf(bf16_hi(ev.x), bf16_hi(wv.x), acc);
    acc = fmaf(bf16_lo(ev.y), bf16_lo(wv.y), acc);
    acc = fmaf(bf16_hi(ev.y), bf16_hi(wv.y), acc);
    acc = fmaf(bf16_lo(ev.z), bf16_lo(wv.z), acc);
    acc = fmaf(bf16_hi(ev.z), bf16_hi(wv.z), acc);
    acc = fmaf(bf16_lo(ev.w), bf16_lo(wv.w), acc);
    acc = fmaf(bf16_hi(ev.w), bf16_hi(wv.w), acc);
  }
  return acc;
}

// The same product with the operand taken from a float row rounded to bfloat16
// (the RNN head's state) instead of a row of E.
__device__ __forceinline__ float half_dot_state(const float* srow, const uint16_t* Wt, int v, int r, int h) {
  const int n = r >> 1;
  const float* e = srow + h * n;
  const uint4* w = reinterpret_cast<const uint4*>(Wt + (size_t)v * r + h * n);
  float acc = 0.f;
  for (int j = 0; j < n / 8; ++j) {
    const uint4 ev = bf16x8_from_f32(e + 8 * j), wv = w[j];
    acc = fmaf(bf16_lo(ev.x), bf16_lo(wv.x), acc);
    acc = fmaf(bf16_hi(ev.x), bf16_hi(wv.x), acc);
    acc = fmaf(bf16_lo(ev.y), bf16_lo(wv.y), acc);
    acc = fmaf(bf16_hi(ev.y), bf16_hi(wv.y), acc);
    acc = fmaf(bf16_lo(ev.z), bf16_lo(wv.z), acc);
    acc = fmaf(bf16_hi(ev.z), bf16_hi(wv.z), acc);
    acc = fmaf(bf16_lo(ev.w), bf16_lo(wv.w), acc);
    acc = fmaf(bf16_hi(ev.w), bf16_hi(wv.w), acc);
  }
  return acc;
}

template <>
__device__ __forceinline__ float half_dot<float>(const float* E, const float* Wt, int prev, int v, int r, int h) {
  const int n = r >> 1;
  const float4* e = reinterpret_cast<const float4*>(E + (size_t)prev * r + h * n);
  const float4* w = reinterpret_cast<const float4*>(Wt + (size_t)v * r + h * n);
  float acc = 0.f;
  for (int j = 0; j < n / 4; ++j) {
    const float4 ev = e[j], wv = w[j];
    acc = fmaf(ev.x, wv.x, acc);
    acc = fmaf(ev.y, wv.y, acc);
    acc = fmaf(ev.z, wv.z, acc);
    acc = fmaf(ev.w, wv.w, acc);
  }
  return acc;
}

// The same half dot product with the rank R fixed at compile time: a half row
// of E or Wt held in registers (so the loads of a whole half row are in flight
// at once), and the fmas in the same order as half_dot.
template <typename WT, int R>
struct HalfRow;
template <int R>
struct HalfRow<uint16_t, R> {
  static constexpr int kN = R / 16;  // uint4 pieces of R/2 bf16 entries
  uint4 q[kN];
  __device__ __forceinline__ void load(const uint16_t* row, int h) {
    const uint4* p = reinterpret_cast<const uint4*>(row + h * (R / 2));
#pragma unroll
    for (int j = 0; j < kN; ++j) q[j] = p[j];
  }
  // a float row (a recurrent state), rounded to bfloat16 as the projection operand
  __device__ __forceinline__ void load_f32(const float* row, int h) {
#pragma unroll
    for (int j = 0; j < kN; ++j) q[j] = bf16x8_from_f32(row + h * (R / 2) + 8 * j);
  }
};
template <int R>
struct HalfRow<float, R> {
  static constexpr int kN = R / 8;  // float4 pieces of R/2 fp32 entries
  float4 q[kN];
  __device__ __forceinline__ void load(const float* row, int h) {
    const float4* p = reinterpret_cast<const float4*>(row + h * (R / 2));
#pragma unroll
    for (int j = 0; j < kN; ++j) q[j] = p[j];
  }
  __device__ __forceinline__ void load_f32(const float* row, int h) { load(row, h); }
};

template <int R>
__device__ __forceinline__ float half_dot_regs(const HalfRow<uint16_t, R>& e, const HalfRow<uint16_t, R>& w) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < HalfRow<uint16_t, R>::kN; ++j) {
    const uint4 ev = e.q[j], wv = w.q[j];
    acc = fmaf(bf16_lo(ev.x), bf16_lo(wv.x), acc);
    acc = fmaf(bf16_hi(ev.x), bf16_hi(wv.x), acc);
    acc = fmaf(bf16_lo(ev.y), bf16_lo(wv.y), acc);
    acc = fmaf(bf16_hi(ev.y), bf16_hi(wv.y), acc);
    acc = fmaf(bf16_lo(ev.z), bf16_lo(wv.z), acc);
    acc = fmaf(bf16_hi(ev.z), bf16_hi(wv.z), acc);
    acc = fmaf(bf16_lo(ev.w), bf16_lo(wv.w), acc);
    acc = fmaf(bf16_hi(ev.w), bf16_hi(wv.w), acc);
  }
  return acc;
}
template <int R>
__device__ __forceinline__ float half_dot_regs(const HalfRow<float, R>& e, const HalfRow<float, R>& w) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < HalfRow<float, R>::kN; ++j) {
    const float4 ev = e.q[j], wv = w.q[j];
    acc = fmaf(ev.x, wv.x, acc);
    acc = fmaf(ev.y, wv.y, acc);
    acc = fmaf(ev.z, wv.z, acc);
    acc = fmaf(ev.w, wv.w, acc);
  }
  return acc;
}

}  // namespace dspark
