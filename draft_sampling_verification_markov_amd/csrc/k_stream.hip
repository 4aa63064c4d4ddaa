// Vocabulary-split stream kernel and the per-row select kernel of the Markov
// draft step.
//
// Draft step k (DSpark page, Method > Semi-autoregressive generation: base
// logits plus a rank-r transition bias that depends on the previous token only,
// sampled position after position):
//
//   k_stream<DRAFT>  every workgroup owns a contiguous range of 128-entry
//                    vocabulary chunks and processes all B rows for them.  Per
//                    chunk it stages Wt[chunk] (128 x r) in LDS, forms the bias
//                    tile bias[v][b] = Wt[v] . E[prev_b] with MFMA (M = vocab,
//                    N = requests, K = rank), adds the logits, scales by
//                    log2(e)/T_s, and reduces each row's chunk to (max, sum of
//                    2^(x - max)) in registers: in the 32x32 accumulator layout
//                    a lane holds one request and 16 vocabulary entries per tile,
//                    so the reduction is in-lane plus one exchange with lane^32.
//                    The chunk score log(mass) + Gumbel(chunk) is kept as a
//                    running best; the row's running (max, sum) as an online
//                    log-partition.  One float4 partial per (row, workgroup).
//   k_select         one workgroup per row: merges the partials into the row's
//                    log-partition and winning chunk, recomputes the 128 logits
//                    of that chunk, draws the entry by Gumbel-max and writes the
//                    token, log q(token) and the log-partition.
//
// The same stream kernel in VERIFY mode runs the resample pass of verification
// (DSpark page, Overview/Background): per request either the residual
// max(0, p - q) at the first rejected position (q recomputed with the same
// MFMA tiles) or the target row of the bonus position.
#include "dspark_internal.hpp"

namespace dspark {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerPass = kWaves * 32;

enum { MODE_DRAFT = 0, MODE_VERIFY = 1 };

// ---------------------------------------------------------------- Markov factor fragments
// A-operand = Wt rows of the chunk (from LDS), B-operand = E[prev] of the lane's
// request (registers, loaded once per pass).  32x32 MFMA accumulator layout:
// lane l holds column (request) l % 32 and rows 8*(i/4) + 4*(l/32) + i%4, i < 16.
template <typename WT, int R>
struct Frag;

template <int R>
struct Frag<uint16_t, R> {  // bf16 factors: v_mfma_f32_32x32x16_bf16
  static constexpr int kSteps = R / 16;
  static constexpr int kStride = R + 8;  // LDS row stride in elements (16-byte pad)
  static constexpr int kLdsElems = kChunk * kStride;
  bf16x8_t b[kSteps];

  __device__ __forceinline__ void load(const uint16_t* E, int tok, bool valid, int lane) {
    const uint16_t* src = E + (size_t)tok * R + 8 * (lane >> 5);
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      if (valid) {
        b[t] = *reinterpret_cast<const bf16x8_t*>(src + 16 * t);
      } else {
        b[t] = bf16x8_t{};
      }
    }
  }
  __device__ __forceinline__ static void stage(uint16_t* lds, const uint16_t* Wt, int c, int V, int tid) {
    constexpr int kPerRow = R / 8;
    constexpr int kPieces = kChunk * kPerRow;
#pragma unroll 4
    for (int p = tid; p < kPieces; p += kThreads) {
      const int row = p / kPerRow, col = (p % kPerRow) * 8;
      const int v = c * kChunk + row;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (v < V) val = *reinterpret_cast<const uint4*>(Wt + (size_t)v * R + col);
      *reinterpret_cast<uint4*>(lds + row * kStride + col) = val;
    }
  }
  __device__ __forceinline__ void mma(const uint16_t* lds, int mt, f32x16_t& acc, int lane) const {
    const uint16_t* a = lds + (mt * 32 + (lane & 31)) * kStride + 8 * (lane >> 5);
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(a + 16 * t);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b[t], acc, 0, 0, 0);
    }
  }
};

template <int R>
struct Frag<float, R> {  // fp32 factors: v_mfma_f32_32x32x2f32
  static constexpr int kSteps = R / 2;
  static constexpr int kStride = R + 1;
  static constexpr int kLdsElems = kChunk * kStride;
  float b[kSteps];

  __device__ __forceinline__ void load(const float* E, int tok, bool valid, int lane) {
    const float* src = E + (size_t)tok * R + (lane >> 5);
#pragma unroll
    for (int t = 0; t < kSteps; ++t) b[t] = valid ? src[2 * t] : 0.0f;
  }
  __device__ __forceinline__ static void stage(float* lds, const float* Wt, int c, int V, int tid) {
    constexpr int kPerRow = R / 4;
    constexpr int kPieces = kChunk * kPerRow;
    for (int p = tid; p < kPieces; p += kThreads) {
      const int row = p / kPerRow, col = (p % kPerRow) * 4;
      const int v = c * kChunk + row;
      float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
      if (v < V) val = *reinterpret_cast<const float4*>(Wt + (size_t)v * R + col);
      float* d = lds + row * kStride + col;
      d[0] = val.x;
      d[1] = val.y;
      d[2] = val.z;
      d[3] = val.w;
    }
  }
  __device__ __forceinline__ void mma(const float* lds, int mt, f32x16_t& acc, int lane) const {
    const float* a = lds + (mt * 32 + (lane & 31)) * kStride + (lane >> 5);
#pragma unroll
    for (int t = 0; t < kSteps; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2 * t], b[t], acc, 0, 0, 0);
  }
};

// ---------------------------------------------------------------- logits access
template <typename ZT>
struct Logits;

template <>
struct Logits<uint16_t> {  // bf16
  struct Raw {
    uint2 u[16];
  };
  // the lane's 64 entries of a chunk: 16 groups of 4 consecutive ids (V % 8 == 0,
  // so a group lies entirely inside or entirely past the end of the row)
  __device__ __forceinline__ static void load(Raw& r, const uint16_t* row, int v0, int V, int lane) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int v = v0 + (q >> 2) * 32 + (q & 3) * 8 + 4 * (lane >> 5);
      r.u[q] = v < V ? *reinterpret_cast<const uint2*>(row + v) : make_uint2(0u, 0u);
    }
  }
  __device__ __forceinline__ static float get(const Raw& r, int q, int i) {
    const uint32_t w = (i < 2) ? r.u[q].x : r.u[q].y;
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  __device__ __forceinline__ static float one(const uint16_t* row, int v) { return bf16_to_f32(row[v]); }
};

template <>
struct Logits<float> {
  struct Raw {
    float4 f[16];
  };
  __device__ __forceinline__ static void load(Raw& r, const float* row, int v0, int V, int lane) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int v = v0 + (q >> 2) * 32 + (q & 3) * 8 + 4 * (lane >> 5);
      r.f[q] = v < V ? *reinterpret_cast<const float4*>(row + v) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ static float get(const Raw& r, int q, int i) {
    return i == 0 ? r.f[q].x : i == 1 ? r.f[q].y : i == 2 ? r.f[q].z : r.f[q].w;
  }
  __device__ __forceinline__ static float one(const float* row, int v) { return row[v]; }
};

__device__ __forceinline__ uint32_t quad_word(const Words4& q, int s) {
  return s == 0 ? q.w[0] : s == 1 ? q.w[1] : s == 2 ? q.w[2] : q.w[3];
}

// ---------------------------------------------------------------- stream kernel
template <typename ZT, typename WT, int R, int MODE>
__global__ __launch_bounds__(kThreads, 1) void k_stream(StreamArgs a) {
  using F = Frag<WT, R>;
  using L = Logits<ZT>;
  __shared__ __attribute__((aligned(16))) WT lds[F::kLdsElems];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x, g = blockIdx.x;
  const int c_begin = (int)(((long long)g * a.nchunks) / G);
  const int c_end = (int)(((long long)(g + 1) * a.nchunks) / G);
  const ZT* Z = static_cast<const ZT*>(a.Z);
  const ZT* Zt = static_cast<const ZT*>(a.Zt);
  const int V = a.V, K = a.K;

  for (int base = 0; base < a.B; base += kRowsPerPass) {
    const int b = base + wave * 32 + (lane & 31);
    const bool rv = b < a.B;
    const bool wave_on = base + wave * 32 < a.B;

    // per-row set-up
    int prev = 0, kpos = a.k;
    uint32_t purpose = kDraftChunk;
    const ZT* zrow = Z;
    const ZT* trow = Zt;
    bool resid = false;
    float lsq2 = 0.f, lsp2 = 0.f;
    if (rv) {
      if (MODE == MODE_DRAFT) {
        prev = clamp_id(a.k == 1 ? a.anchor[b] : a.tok[(size_t)b * K + a.k - 2], V);
        zrow = Z + ((size_t)b * K + (a.k - 1)) * V;
      } else {
        const int ks = a.job[b];
        if (ks > 0) {
          resid = true;
          kpos = ks;
          purpose = kResidChunk;
          prev = clamp_id(ks == 1 ? a.anchor[b] : a.tok[(size_t)b * K + ks - 2], V);
          zrow = Z + ((size_t)b * K + (ks - 1)) * V;
          trow = Zt + ((size_t)b * (K + 1) + (ks - 1)) * V;
          lsq2 = a.lse_q[(size_t)b * K + ks - 1] * kLog2e;
          lsp2 = a.lse_p[(size_t)b * K + ks - 1] * kLog2e;
        } else {
          int nb = a.n_sched[b];
          nb = nb < 0 ? 0 : (nb > K ? K : nb);
          kpos = nb + 1;
          purpose = kBonusChunk;
          trow = Zt + ((size_t)b * (K + 1) + nb) * V;
        }
      }
    }
    const bool need_bias = rv && (MODE == MODE_DRAFT || resid);
    F frag;
    frag.load(static_cast<const WT*>(a.E), prev, need_bias, lane);

    float run_m = -INFINITY, run_s = 0.f, best = -INFINITY, mass = 0.f;
    int best_c = 0x7fffffff;
    int quad_id = -1;
    Words4 quad = {};

    for (int c = c_begin; c < c_end; ++c) {
      __syncthreads();
      F::stage(lds, static_cast<const WT*>(a.Wt), c, V, tid);
      __syncthreads();
      if (!wave_on) continue;

      const int v0 = c * kChunk;
      // logits of this chunk, issued before the MFMAs so that their latency overlaps
      typename L::Raw zr = {}, tr = {};
      if (rv) {
        if (MODE == MODE_DRAFT || resid) L::load(zr, zrow, v0, V, lane);
        if (MODE == MODE_VERIFY) L::load(tr, trow, v0, V, lane);
      }

      f32x16_t acc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        acc[mt] = f32x16_t{};
        frag.mma(lds, mt, acc[mt], lane);
      }
      if (!rv) continue;

      if (c >> 2 != quad_id) {
        quad = draw_quad(a.key, (uint32_t)c, (uint32_t)b, (uint32_t)kpos, purpose);
        quad_id = c >> 2;
      }
      const float gum = gumbel_from_word(quad_word(quad, c & 3));

      if (MODE == MODE_VERIFY && resid) {
        // residual max(0, p - q) of the rejected position
        float rs = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int q = mt * 4 + (i >> 2);
            const int v = v0 + mt * 32 + (i >> 2) * 8 + 4 * (lane >> 5) + (i & 3);
            if (v < V) {
              const float p = exp2f(L::get(tr, q, i & 3) * a.scale2 - lsp2);
              const float qq = exp2f((L::get(zr, q, i & 3) + acc[mt][i]) * a.scale2 - lsq2);
              rs += fmaxf(p - qq, 0.f);
            }
          }
        }
        rs += __shfl_xor(rs, 32);
        mass += rs;
        const float score = rs > 0.f ? logf(rs) + gum : -INFINITY;
        if (score > best) {
          best = score;
          best_c = c;
        }
      } else {
        // log-mass of the chunk under softmax(x / T_s): draft logits + bias, or bonus target row
        float m = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int q = mt * 4 + (i >> 2);
            const int v = v0 + mt * 32 + (i >> 2) * 8 + 4 * (lane >> 5) + (i & 3);
            float x;
            if (MODE == MODE_DRAFT) {
              x = (L::get(zr, q, i & 3) + acc[mt][i]) * a.scale2;
            } else {
              x = L::get(tr, q, i & 3) * a.scale2;
            }
            x = v < V ? x : -INFINITY;
            acc[mt][i] = x;
            m = fmaxf(m, x);
          }
        }
        m = fmaxf(m, __shfl_xor(m, 32));
        float s = 0.f;
        if (m != -INFINITY) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s += exp2f(acc[mt][i] - m);
          }
        }
        s += __shfl_xor(s, 32);
        if (MODE == MODE_DRAFT) lse2_merge(run_m, run_s, m, s);
        const float score = (m + log2f(s)) * kLn2 + gum;
        if (s > 0.f && score > best) {
          best = score;
          best_c = c;
        }
      }
    }

    if (rv && lane < 32) {
      float4 out;
      if (MODE == MODE_DRAFT) {
        out = make_float4(run_m, run_s, best, __int_as_float(best_c));
      } else {
        out = make_float4(mass, 0.f, best, __int_as_float(best_c));
      }
      a.part[(size_t)b * G + g] = out;
    }
  }
}

// ---------------------------------------------------------------- select kernel
template <typename ZT, typename WT>
__global__ __launch_bounds__(256) void k_select(SelectArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, V = a.V;
  __shared__ float s_m[4], s_s[4], s_best[4], s_ell[kChunk];
  __shared__ int s_c[4];
  __shared__ float s_lse;
  __shared__ int s_cstar;

  // 1. merge the per-workgroup partials of row b
  float m = -INFINITY, s = 0.f, best = -INFINITY;
  int bc = 0x7fffffff;
  for (int i = tid; i < a.G; i += 256) {
    const float4 p = a.part[(size_t)b * a.G + i];
    lse2_merge(m, s, p.x, p.y);
    const int pc = __float_as_int(p.w);
    if (better(p.z, pc, best, bc)) {
      best = p.z;
      bc = pc;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    lse2_merge(m, s, m2, s2);
  }
  wave_argmax(best, bc);
  if (lane == 0) {
    s_m[wave] = m;
    s_s[wave] = s;
    s_best[wave] = best;
    s_c[wave] = bc;
  }
  __syncthreads();
  if (tid == 0) {
    float M = s_m[0], S = s_s[0], B0 = s_best[0];
    int C0 = s_c[0];
    for (int w = 1; w < 4; ++w) {
      lse2_merge(M, S, s_m[w], s_s[w]);
      if (better(s_best[w], s_c[w], B0, C0)) {
        B0 = s_best[w];
        C0 = s_c[w];
      }
    }
    s_lse = (M + log2f(S)) * kLn2;
    // a row without any finite chunk score (non-finite logits) falls back to chunk 0
    s_cstar = (C0 >= 0 && C0 * kChunk < V) ? C0 : 0;
  }
  __syncthreads();
  const int cstar = s_cstar;
  const float lse = s_lse;

  // 2. recompute the winning chunk's logits and draw the entry
  const int prev = clamp_id(a.k == 1 ? a.anchor[b] : a.tok[(size_t)b * K + a.k - 2], V);
  const int j = tid >> 1, h = tid & 1;
  const int v = cstar * kChunk + j;
  const bool inside = v < V;
  float dot = inside ? half_dot<WT>(static_cast<const WT*>(a.E), static_cast<const WT*>(a.Wt), prev, v, a.r, h)
                     : 0.f;
  dot += __shfl_xor(dot, 1);
  float score = -INFINITY;
  int idx = 0x7fffffff;
  if (h == 0 && inside) {
    const ZT* zrow = static_cast<const ZT*>(a.Z) + ((size_t)b * K + (a.k - 1)) * V;
    const float ell = (logit_at<ZT>(zrow, v) + dot) * a.inv_T;
    s_ell[j] = ell;
    score = ell + gumbel_from_word(draw_word(a.key, (uint32_t)v, (uint32_t)b, (uint32_t)a.k, kDraftElem));
    idx = v;
  }
  wave_argmax(score, idx);
  __syncthreads();
  if (lane == 0) {
    s_best[wave] = score;
    s_c[wave] = idx;
  }
  __syncthreads();
  if (tid == 0) {
    float B0 = s_best[0];
    int X = s_c[0];
    for (int w = 1; w < 4; ++w) {
      if (better(s_best[w], s_c[w], B0, X)) {
        B0 = s_best[w];
        X = s_c[w];
      }
    }
    const size_t o = (size_t)b * K + (a.k - 1);
    if (X < cstar * kChunk || X >= cstar * kChunk + kChunk || X >= V) X = cstar * kChunk;  // no finite score
    a.tok[o] = X;
    a.logq[o] = s_ell[X - cstar * kChunk] - lse;
    a.lse[o] = lse;
  }
}

}  // namespace

// ---------------------------------------------------------------- dispatch
#define DSPARK_R_CASES_BF16(ZT, MODE)                                                            \
  switch (P.r) {                                                                                 \
    case 16: hipLaunchKernelGGL((k_stream<ZT, uint16_t, 16, MODE>), G, kThreads, 0, s, a); break;   \
    case 32: hipLaunchKernelGGL((k_stream<ZT, uint16_t, 32, MODE>), G, kThreads, 0, s, a); break;   \
    case 64: hipLaunchKernelGGL((k_stream<ZT, uint16_t, 64, MODE>), G, kThreads, 0, s, a); break;   \
    case 128: hipLaunchKernelGGL((k_stream<ZT, uint16_t, 128, MODE>), G, kThreads, 0, s, a); break; \
    case 256: hipLaunchKernelGGL((k_stream<ZT, uint16_t, 256, MODE>), G, kThreads, 0, s, a); break; \
    default: return hipErrorInvalidValue;                                                        \
  }
#define DSPARK_R_CASES_F32(ZT, MODE)                                                         \
  switch (P.r) {                                                                             \
    case 16: hipLaunchKernelGGL((k_stream<ZT, float, 16, MODE>), G, kThreads, 0, s, a); break; \
    case 32: hipLaunchKernelGGL((k_stream<ZT, float, 32, MODE>), G, kThreads, 0, s, a); break; \
    case 64: hipLaunchKernelGGL((k_stream<ZT, float, 64, MODE>), G, kThreads, 0, s, a); break; \
    default: return hipErrorInvalidValue;                                                    \
  }

template <int MODE>
static hipError_t launch_stream(const dspark_problem& P, const StreamArgs& a, int G, hipStream_t s) {
  const bool zb = P.logits_dtype == DSPARK_BF16, wb = P.weight_dtype == DSPARK_BF16;
  if (zb && wb) {
    DSPARK_R_CASES_BF16(uint16_t, MODE)
  } else if (zb && !wb) {
    DSPARK_R_CASES_F32(uint16_t, MODE)
  } else if (!zb && wb) {
    DSPARK_R_CASES_BF16(float, MODE)
  } else {
    DSPARK_R_CASES_F32(float, MODE)
  }
  return hipGetLastError();
}

hipError_t launch_stream_draft(const dspark_problem& P, const StreamArgs& a, int G, hipStream_t s) {
  return launch_stream<MODE_DRAFT>(P, a, G, s);
}

hipError_t launch_stream_verify(const dspark_problem& P, const StreamArgs& a, int G, hipStream_t s) {
  return launch_stream<MODE_VERIFY>(P, a, G, s);
}

hipError_t launch_select(const dspark_problem& P, const SelectArgs& a, hipStream_t s) {
  const bool zb = P.logits_dtype == DSPARK_BF16, wb = P.weight_dtype == DSPARK_BF16;
  if (zb && wb) hipLaunchKernelGGL((k_select<uint16_t, uint16_t>), P.B, 256, 0, s, a);
  else if (zb) hipLaunchKernelGGL((k_select<uint16_t, float>), P.B, 256, 0, s, a);
  else if (wb) hipLaunchKernelGGL((k_select<float, uint16_t>), P.B, 256, 0, s, a);
  else hipLaunchKernelGGL((k_select<float, float>), P.B, 256, 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
