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
  // the four groups of M-tile mt only, into groups 0..3 of r
  __device__ __forceinline__ static void load_mt(Raw& r, const uint16_t* row, int v0, int V, int lane, int mt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = v0 + mt * 32 + j * 8 + 4 * (lane >> 5);
      r.u[j] = v < V ? *reinterpret_cast<const uint2*>(row + v) : make_uint2(0u, 0u);
    }
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
  __device__ __forceinline__ static void load_mt(Raw& r, const float* row, int v0, int V, int lane, int mt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = v0 + mt * 32 + j * 8 + 4 * (lane >> 5);
      r.f[j] = v < V ? *reinterpret_cast<const float4*>(row + v) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ static float one(const float* row, int v) { return row[v]; }
};

__device__ __forceinline__ uint32_t quad_word(const Words4& q, int s) {
  return s == 0 ? q.w[0] : s == 1 ? q.w[1] : s == 2 ? q.w[2] : q.w[3];
}

// ---------------------------------------------------------------- stream kernel (generic: fp32 factors)
// Single LDS buffer, logits loaded per chunk.  Serves the fp32-factor path.
template <typename ZT, typename WT, int R, int MODE>
__global__ __launch_bounds__(kThreads, 1) void k_stream_generic(StreamArgs a) {
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
    float lsq2 = 0.f, lsp2 = 0.f, dlp = 0.f;
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
          dlp = lsp2 - lsq2;
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

    float run_m = -INFINITY, run_s = 0.f, best = -INFINITY;
    double Rs = 0.0, QAs = 0.0, Zps = 0.0, Zqs = 0.0;  // residual rows: this lane's sums of r, qa, p^, q^
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
        ResidSums sums;
        sums.clear();
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int q = mt * 4 + (i >> 2);
            const int v = v0 + mt * 32 + (i >> 2) * 8 + 4 * (lane >> 5) + (i & 3);
            // entries past V: the target and draft logit -inf, so every weight is 0
            const bool in = v < V;
            sums.add(i, resid_entry(in ? L::get(tr, q, i & 3) : -INFINITY, in ? L::get(zr, q, i & 3) : -INFINITY,
                                    acc[mt][i], a.scale2, lsp2, lsq2, dlp));
          }
        }
        float rs = ResidSums::fold(sums.r);
        Rs += (double)rs;
        QAs += (double)ResidSums::fold(sums.qa);
        Zps += (double)ResidSums::fold(sums.p);
        Zqs += (double)ResidSums::fold(sums.q);
        rs = halves32_sum(rs);
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

    if (MODE == MODE_DRAFT) {
      if (rv && lane < 32) a.part[(size_t)b * G + g] = make_float4(run_m, run_s, best, __int_as_float(best_c));
    } else {
      const double R_g = halves32_sum_d(Rs), QA_g = halves32_sum_d(QAs);
      const double Zp_g = halves32_sum_d(Zps), Zq_g = halves32_sum_d(Zqs);
      if (rv && lane < 32) {
        a.part[(size_t)b * G + g] = make_float4((float)R_g, (float)QA_g, best, __int_as_float(best_c));
        a.zpart[(size_t)b * G + g] = make_float2((float)Zp_g, (float)Zq_g);
      }
    }
  }
}

// ---------------------------------------------------------------- verify, small batches
// The resample pass of the generic path (fp32 logits or fp32 factors) for
// B <= 64.  The all-rows mapping gives each wave 32 rows and every M-tile of a
// chunk, so at B <= 32 one wave of eight does all the MFMAs and the whole
// residual epilogue; here wave w takes rows 32 (w / 4) .. + 31 and M-tile w % 4
// of each chunk, and the four M-tile waves of a row group exchange their
// per-chunk results through LDS (the residual mass, or a bonus row's (max,
// sum)), from which the first keeps the chunk score and the best chunk.  Same
// per-entry arithmetic as k_stream_generic; the fp64 sums meet across the four
// waves at the end.
template <typename ZT, typename WT, int R>
__global__ __launch_bounds__(kThreads, 1) void k_verify_smallb(StreamArgs a) {
  using F = Frag<WT, R>;
  using L = Logits<ZT>;
  __shared__ __attribute__((aligned(16))) WT lds[F::kLdsElems];
  __shared__ float s_x[2][4][2][32];   // [row group][M-tile][residual mass or max, sum][row]
  __shared__ double s_d[2][4][4][32];  // [row group][M-tile][R, QA, Zp, Zq][row]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = wave >> 2, mt = wave & 3;
  const int G = gridDim.x, g = blockIdx.x;
  const int c_begin = (int)(((long long)g * a.nchunks) / G);
  const int c_end = (int)(((long long)(g + 1) * a.nchunks) / G);
  const ZT* Z = static_cast<const ZT*>(a.Z);
  const ZT* Zt = static_cast<const ZT*>(a.Zt);
  const int V = a.V, K = a.K;
  const int b = rg * 32 + (lane & 31);
  const bool rv = b < a.B;
  const bool wave_on = rg * 32 < a.B;

  // per-row set-up (the generic kernel's verify mode)
  int prev = 0, kpos = 1;
  uint32_t purpose = kBonusChunk;
  const ZT* zrow = Z;
  const ZT* trow = Zt;
  bool resid = false;
  float lsq2 = 0.f, lsp2 = 0.f, dlp = 0.f;
  if (rv) {
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
      dlp = lsp2 - lsq2;
    } else {
      int nb = a.n_sched[b];
      nb = nb < 0 ? 0 : (nb > K ? K : nb);
      kpos = nb + 1;
      trow = Zt + ((size_t)b * (K + 1) + nb) * V;
    }
  }
  F frag;
  frag.load(static_cast<const WT*>(a.E), prev, rv && resid, lane);

  float best = -INFINITY;
  int best_c = 0x7fffffff;
  int quad_id = -1;
  Words4 quad = {};
  double Rs = 0.0, QAs = 0.0, Zps = 0.0, Zqs = 0.0;

  for (int c = c_begin; c < c_end; ++c) {
    __syncthreads();
    F::stage(lds, static_cast<const WT*>(a.Wt), c, V, tid);
    __syncthreads();
    const int v0 = c * kChunk;
    typename L::Raw zr = {}, tr = {};
    if (wave_on && rv) {
      if (resid) L::load_mt(zr, zrow, v0, V, lane, mt);
      L::load_mt(tr, trow, v0, V, lane, mt);
    }
    f32x16_t acc = {};
    if (wave_on) frag.mma(lds, mt, acc, lane);
    float x0 = 0.f, x1 = 0.f;
    if (wave_on && rv) {
      if (resid) {
        ResidSums sums;
        sums.clear();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = i >> 2;  // the M-tile's groups sit in groups 0..3
          const int v = v0 + mt * 32 + (i >> 2) * 8 + 4 * (lane >> 5) + (i & 3);
          const bool in = v < V;  // entries past V: target and draft logit -inf, every weight 0
          sums.add(i, resid_entry(in ? L::get(tr, q, i & 3) : -INFINITY, in ? L::get(zr, q, i & 3) : -INFINITY,
                                  acc[i], a.scale2, lsp2, lsq2, dlp));
        }
        const float rs = ResidSums::fold(sums.r);
        Rs += (double)rs;
        QAs += (double)ResidSums::fold(sums.qa);
        Zps += (double)ResidSums::fold(sums.p);
        Zqs += (double)ResidSums::fold(sums.q);
        x0 = halves32_sum(rs);
      } else {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = i >> 2;
          const int v = v0 + mt * 32 + (i >> 2) * 8 + 4 * (lane >> 5) + (i & 3);
          const float x = v < V ? L::get(tr, q, i & 3) * a.scale2 : -INFINITY;
          acc[i] = x;
          m = fmaxf(m, x);
        }
        m = fmaxf(m, __shfl_xor(m, 32));
        float sm = 0.f;
        if (m != -INFINITY) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sm += exp2f(acc[i] - m);
        }
        sm += __shfl_xor(sm, 32);
        x0 = m;
        x1 = sm;
      }
    }
    if (lane < 32) {
      s_x[rg][mt][0][lane] = x0;
      s_x[rg][mt][1][lane] = x1;
    }
    __syncthreads();
    if (wave_on && rv && mt == 0) {
      if (c >> 2 != quad_id) {
        quad = draw_quad(a.key, (uint32_t)c, (uint32_t)b, (uint32_t)kpos, purpose);
        quad_id = c >> 2;
      }
      const float gum = gumbel_from_word(quad_word(quad, c & 3));
      const int r = lane & 31;
      float score = -INFINITY;
      if (resid) {
        const float rs = (s_x[rg][0][0][r] + s_x[rg][1][0][r]) + (s_x[rg][2][0][r] + s_x[rg][3][0][r]);
        score = rs > 0.f ? logf(rs) + gum : -INFINITY;
      } else {
        float m = s_x[rg][0][0][r], sm = s_x[rg][0][1][r];
#pragma unroll
        for (int j = 1; j < 4; ++j) lse2_merge(m, sm, s_x[rg][j][0][r], s_x[rg][j][1][r]);
        score = sm > 0.f ? (m + log2f(sm)) * kLn2 + gum : -INFINITY;
      }
      if (score > best) {
        best = score;
        best_c = c;
      }
    }
  }
  // the row's fp64 sums over the four M-tile waves
  const double R_w = halves32_sum_d(Rs), QA_w = halves32_sum_d(QAs);
  const double Zp_w = halves32_sum_d(Zps), Zq_w = halves32_sum_d(Zqs);
  if (lane < 32) {
    s_d[rg][mt][0][lane] = R_w;
    s_d[rg][mt][1][lane] = QA_w;
    s_d[rg][mt][2][lane] = Zp_w;
    s_d[rg][mt][3][lane] = Zq_w;
  }
  __syncthreads();
  if (mt == 0 && rv && lane < 32) {
    double t[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) t[q] = (s_d[rg][0][q][lane] + s_d[rg][1][q][lane]) + (s_d[rg][2][q][lane] + s_d[rg][3][q][lane]);
    a.part[(size_t)b * G + g] = make_float4((float)t[0], (float)t[1], best, __int_as_float(best_c));
    a.zpart[(size_t)b * G + g] = make_float2((float)t[2], (float)t[3]);
  }
}

// ---------------------------------------------------------------- stream kernel (bf16 factors)
// Two-stage LDS pipeline over vocabulary units (one unit = 128 bytes of every
// request's logits row in draft mode: 64 bf16 / 32 fp32 entries; 64 bytes in
// verify mode, where a third tile carries the target row of residual requests):
//  * every tile (logits 256 requests x unit, target likewise, Wt unit x r) is
//    brought in by LDS DMA with coalesced 1 KB wave instructions, unit u+1
//    streaming in while unit u is multiplied;
//  * 16-byte slots of every LDS row are XOR-swizzled by the row index, so the
//    A-fragment reads (32 Wt rows, same slot) and the logits reads (32
//    requests, same slot) fall on distinct banks;
//  * MFMA row rho of an M-tile is bound to vocabulary entry
//    16*((rho >> 2) & 1) + 4*(rho >> 3) + (rho & 3): in the 32x32 accumulator
//    layout lane l then holds 16 consecutive entries (16*(l/32) ... +15) of its
//    request, reads its logits with 16-byte LDS loads, and the accumulator
//    starts from them (D = logits + bias);
//  * draft epilogue per unit: max, one fma into base-2 units, raw v_exp_f32,
//    add; units merge into the chunk's (max, sum), finished chunks into the
//    row's running log-partition and best chunk score.
template <typename ZT, int R, int MODE>
struct Tiles {
  static constexpr int kZRow = MODE == MODE_DRAFT ? 128 : 64;  // bytes of one request's unit
  static constexpr int kZSlots = kZRow / 16;
  static constexpr int kUnit = kZRow / (int)sizeof(ZT);        // vocabulary entries per unit
  static constexpr int kMt = kUnit / 32;                       // M-tiles per unit
  static constexpr int kUnitsPerChunk = kChunk / kUnit;
  static constexpr int kZBytes = kRowsPerPass * kZRow;
  static constexpr int kTBytes = MODE == MODE_DRAFT ? 0 : kZBytes;
  static constexpr int kWSlots = R / 8;
  static constexpr int kWRow = R * 2;
  static constexpr int kWBytes = kUnit * kWRow;
  static constexpr int kStage = kZBytes + kTBytes + kWBytes;
  static constexpr int kSteps = R / 16;
  static constexpr int kZRowsPerBlk = 1024 / kZRow;

  __device__ __forceinline__ static int z_off(int row, int s) {
    return row * kZRow + ((s ^ (row & (kZSlots - 1))) << 4);
  }
  __device__ __forceinline__ static int w_off(int row, int s) {
    return kZBytes + kTBytes + row * kWRow + ((s ^ (row & (kWSlots - 1))) << 4);
  }
  // DMA of the unit starting at vocabulary entry v0.  zsrc/tsrc: the row
  // pointers of the requests whose logits (target) this lane brings in, one per
  // block it handles (block blk = wave + j * kWaves).
  __device__ __forceinline__ static void stage(unsigned char* buf, const ZT* const* zsrc, const ZT* const* tsrc,
                                               const uint16_t* Wt, int V, int v0, int wave, int lane) {
    constexpr int kPer = 16 / (int)sizeof(ZT);
#pragma unroll
    for (int j = 0; j < kZBytes / 1024 / kWaves; ++j) {
      const int blk = wave + j * kWaves;
      const int row = blk * kZRowsPerBlk + lane / kZSlots;
      const int s = (lane % kZSlots) ^ (row & (kZSlots - 1));
      int v = v0 + s * kPer;
      v = v < V ? v : V - kPer;
      __builtin_amdgcn_global_load_lds(zsrc[j] + v, (__attribute__((address_space(3))) void*)(buf + blk * 1024), 16,
                                       0, 0);
      if (MODE == MODE_VERIFY)
        __builtin_amdgcn_global_load_lds(tsrc[j] + v,
                                         (__attribute__((address_space(3))) void*)(buf + kZBytes + blk * 1024), 16, 0,
                                         0);
    }
#pragma unroll
    for (int blk = wave; blk < kWBytes / 1024; blk += kWaves) {
      const int row = blk * (1024 / kWRow) + lane / kWSlots;
      const int s = (lane % kWSlots) ^ (row & (kWSlots - 1));
      int v = v0 + row;
      v = v < V ? v : V - 1;
      __builtin_amdgcn_global_load_lds(Wt + (size_t)v * R + s * 8,
                                       (__attribute__((address_space(3))) void*)(buf + kZBytes + kTBytes + blk * 1024),
                                       16, 0, 0);
    }
  }
};

// Chunks [c_begin, c_end) of workgroup g of G: nchunks / G each, the first
// nchunks % G workgroups one more.  32-bit arithmetic (nchunks < 2^24): the
// 64-bit division it replaces cost hundreds of scalar instructions ahead of the
// first DMA of every launch.
__device__ __forceinline__ void chunk_range(int g, int G, int nchunks, int& c_begin, int& c_end) {
  const unsigned q = (unsigned)nchunks / (unsigned)G, rem = (unsigned)nchunks - q * (unsigned)G;
  const unsigned ug = (unsigned)g;
  c_begin = (int)(ug * q + (ug < rem ? ug : rem));
  c_end = c_begin + (int)q + (ug < rem ? 1 : 0);
}


// Tiles of the draft step (bf16 logits): per stage a logits tile (256 requests
// x 64 entries, 128-byte rows, 16-byte slots XOR-swizzled by the row) and a Wt
// tile (64 vocabulary rows x r) whose rows are padded to 2r + 16 bytes and
// stored at their MFMA row: Wt row of entry mt*32 + vmap(rho) sits at LDS row
// mt*32 + rho, so lane rho's A fragment of K-step t is at
// base(rho) + mt*32*stride + 32*t, and 16 consecutive lanes hit 16 different
// bank groups.  Both tiles arrive by buffer DMA with per-lane offsets that are
// constant over the kernel plus a uniform per-unit offset.
template <int R>
struct DraftTiles {
  using ZT = uint16_t;
  static constexpr int kUnit = 64;
  static constexpr int kMt = 2;
  static constexpr int kZRow = 128, kZSlots = 8;
  static constexpr int kZBytes = kRowsPerPass * kZRow;            // 32 KB
  static constexpr int kWRow = R * 2;                               // bytes of a Wt row
  static constexpr int kWStride = kWRow + 16;                       // padded LDS row
  static constexpr int kWSlots = R / 8;
  static constexpr int kWBytes = kUnit * kWStride;
  static constexpr int kWBlocks = (kWBytes + 1023) / 1024;
  // 1 KB sink after the tiles: target of the filler DMA slots (never read)
  static constexpr int kSink = kZBytes + kWBlocks * 1024;
  static constexpr int kStage = kSink + 1024;
  static constexpr int kSteps = R / 16;
  static constexpr int kUnitsPerChunk = 2;
  static constexpr int kZRowsPerBlk = 1024 / kZRow;

  __device__ __forceinline__ static int z_off(int row, int s) { return row * kZRow + ((s ^ (row & 7)) << 4); }
};

// MFMA row rho -> vocabulary entry within its M-tile (see the layout notes above)
__device__ __forceinline__ int mfma_row_entry(int rho) { return ((rho >> 2) & 1) * 16 + (rho >> 3) * 4 + (rho & 3); }

// Per-lane constant byte offsets of the draft DMA (logits: 4 blocks, Wt: up to 5).
// Every wave issues the same number of DMA instructions per stage, so that the
// vector-memory counter means the same on every wave and the compiler's own
// wait accounting stays exact: slots past the Wt tile read past the end of the
// buffer (the bounds check returns zeros without a memory access) into the sink.
template <int R>
struct DraftDma {
  using T = DraftTiles<R>;
  static constexpr int kZPer = T::kZBytes / 1024 / kWaves;        // 4
  static constexpr int kWPer = (T::kWBlocks + kWaves - 1) / kWaves;
  uint32_t zoff[kZPer];
  uint32_t woff[kWPer];

  __device__ __forceinline__ void init(int wave, int lane, int rows_valid, uint32_t zrow_bytes) {
#pragma unroll
    for (int j = 0; j < kZPer; ++j) {
      const int blk = wave + j * kWaves;
      int row = blk * T::kZRowsPerBlk + lane / T::kZSlots;
      const int s = (lane % T::kZSlots) ^ (row & (T::kZSlots - 1));
      row = row < rows_valid ? row : rows_valid - 1;
      zoff[j] = (uint32_t)row * zrow_bytes + (uint32_t)s * 16;
    }
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      const int blk = wave + j * kWaves;
      const int byte = blk * 1024 + lane * 16;
      const int lrow = byte / T::kWStride, slot = (byte % T::kWStride) / 16;
      const bool real = slot < T::kWSlots && lrow < T::kUnit;
      const int entry = (lrow / 32) * 32 + mfma_row_entry(lrow % 32);
      woff[j] = blk >= T::kWBlocks ? kOutOfRange : real ? (uint32_t)entry * T::kWRow + (uint32_t)slot * 16 : 0u;
    }
  }
  static constexpr uint32_t kOutOfRange = 0x80000000u;  // beyond any Wt buffer (V * r * 2 < 2^31)
  static constexpr int kOps = kZPer + kWPer;              // DMA instructions per wave and stage
  // wait until only the most recent stage() of this wave is still in flight
  __device__ __forceinline__ static void wait_all_but_last_stage() { wait_vmem_n<kOps>(); }
  // DMA of the unit starting at entry v0 into `buf`
  __device__ __forceinline__ void stage(unsigned char* buf, __amdgpu_buffer_rsrc_t zr, __amdgpu_buffer_rsrc_t wr, int v0,
                                        int wave) const {
    stage_z(buf, zr, v0, wave);
    stage_w(buf, wr, v0, wave);
  }
  // the logits tile of the unit
  __device__ __forceinline__ void stage_z(unsigned char* buf, __amdgpu_buffer_rsrc_t zr, int v0, int wave) const {
#pragma unroll
    for (int j = 0; j < kZPer; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          zr, (__attribute__((address_space(3))) void*)(buf + (wave + j * kWaves) * 1024), 16, (int)zoff[j],
          v0 * 2, 0, 0);
  }
  // the Wt tile of the unit
  __device__ __forceinline__ void stage_w(unsigned char* buf, __amdgpu_buffer_rsrc_t wr, int v0, int wave) const {
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      const int blk = wave + j * kWaves;
      const int dst = blk < T::kWBlocks ? T::kZBytes + blk * 1024 : T::kSink;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void*)(buf + dst), 16,
                                               (int)woff[j], v0 * T::kWRow, 0, 0);
    }
  }
};



// 16 consecutive logits of one request from a tile row (two or four 16-byte slots)
template <typename ZT, typename TL>
__device__ __forceinline__ void read16(const unsigned char* tile, int row, int s0, float* o);

template <typename ZT, typename TL>
__device__ __forceinline__ void read16(const unsigned char* tile, int row, int s0, float* o) {
  if (sizeof(ZT) == 2) {
    const uint4 a = *reinterpret_cast<const uint4*>(tile + TL::z_off(row, s0));
    const uint4 b = *reinterpret_cast<const uint4*>(tile + TL::z_off(row, s0 + 1));
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o[2 * i] = bf16_lo(w[i]);
      o[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = *reinterpret_cast<const float4*>(tile + TL::z_off(row, s0 + q));
      o[4 * q] = f.x;
      o[4 * q + 1] = f.y;
      o[4 * q + 2] = f.z;
      o[4 * q + 3] = f.w;
    }
  }
}

template <typename ZT, int R, int MODE>
__global__ __launch_bounds__(kThreads, 1) void k_stream(StreamArgs a) {
  using T = Tiles<ZT, R, MODE>;
  constexpr int kDmaPerWave = T::kZBytes / 1024 / kWaves;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * T::kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x, g = blockIdx.x;
  const int c_begin = (int)(((long long)g * a.nchunks) / G);
  const int c_end = (int)(((long long)(g + 1) * a.nchunks) / G);
  const int nunits = (c_end - c_begin) * T::kUnitsPerChunk;
  const ZT* Z = static_cast<const ZT*>(a.Z);
  const ZT* Zt = static_cast<const ZT*>(a.Zt);
  const uint16_t* Wt = static_cast<const uint16_t*>(a.Wt);
  const int V = a.V, K = a.K, B = a.B;
  const float scale2 = a.scale2;
  const int h = lane >> 5;
  const int wrow = mfma_row_entry(lane & 31);

  for (int base = 0; base < B; base += kRowsPerPass) {
    // rows this lane brings in by DMA: the logits row seeding the accumulator
    // (draft row k; residual base row k*; bonus target row n_b + 1) and, in
    // verify mode, the target row of a residual
    const ZT* zsrc[kDmaPerWave];
    const ZT* tsrc[kDmaPerWave];
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
      const int row = (wave + j * kWaves) * T::kZRowsPerBlk + lane / T::kZSlots;
      int bb = base + row;
      bb = bb < B ? bb : B - 1;
      if (MODE == MODE_DRAFT) {
        zsrc[j] = Z + ((size_t)bb * K + (a.k - 1)) * V;
        tsrc[j] = zsrc[j];
      } else {
        const int ks = a.job[bb];
        int nb = a.n_sched[bb];
        nb = nb < 0 ? 0 : (nb > K ? K : nb);
        if (ks > 0) {
          zsrc[j] = Z + ((size_t)bb * K + (ks - 1)) * V;
          tsrc[j] = Zt + ((size_t)bb * (K + 1) + (ks - 1)) * V;
        } else {
          zsrc[j] = Zt + ((size_t)bb * (K + 1) + nb) * V;
          tsrc[j] = zsrc[j];
        }
      }
    }

    const int prow = wave * 32 + (lane & 31);
    const int b = base + prow;
    const bool rv = b < B;
    const bool wave_on = base + wave * 32 < B;
    int prev = 0, kpos = a.k;
    uint32_t purpose = kDraftChunk;
    bool resid = false;
    float lsq2 = 0.f, lsp2 = 0.f, dlp = 0.f;
    if (rv) {
      if (MODE == MODE_DRAFT) {
        prev = clamp_id(a.k == 1 ? a.anchor[b] : a.tok[(size_t)b * K + a.k - 2], V);
      } else {
        const int ks = a.job[b];
        if (ks > 0) {
          resid = true;
          kpos = ks;
          purpose = kResidChunk;
          prev = clamp_id(ks == 1 ? a.anchor[b] : a.tok[(size_t)b * K + ks - 2], V);
          lsq2 = a.lse_q[(size_t)b * K + ks - 1] * kLog2e;
          lsp2 = a.lse_p[(size_t)b * K + ks - 1] * kLog2e;
          dlp = lsp2 - lsq2;
        } else {
          int nb = a.n_sched[b];
          nb = nb < 0 ? 0 : (nb > K ? K : nb);
          kpos = nb + 1;
          purpose = kBonusChunk;
        }
      }
    }
    bf16x8_t bfrag[T::kSteps];
    {
      const bool need = rv && (MODE == MODE_DRAFT || resid);
      const uint16_t* src = static_cast<const uint16_t*>(a.E) + (size_t)prev * R + 8 * h;
#pragma unroll
      for (int t = 0; t < T::kSteps; ++t)
        bfrag[t] = need ? *reinterpret_cast<const bf16x8_t*>(src + 16 * t) : bf16x8_t{};
    }

    float run_m = -INFINITY, run_s = 0.f, best = -INFINITY;
    double Rs = 0.0, QAs = 0.0, Zps = 0.0, Zqs = 0.0;  // residual rows: this lane's sums of r, qa, p^, q^
    int best_c = 0x7fffffff;
    float cm = -INFINITY, cs = 0.f;  // current chunk: (max, sum) base 2, or residual sum
    int quad_id = -1;
    Words4 quad = {};

    if (nunits > 0) T::stage(lds, zsrc, tsrc, Wt, V, c_begin * kChunk, wave, lane);
    for (int u = 0; u < nunits; ++u) {
      const int c = c_begin + u / T::kUnitsPerChunk;
      const int part = u % T::kUnitsPerChunk;
      const int v0 = c * kChunk + part * T::kUnit;
      unsigned char* cur = lds + (u & 1) * T::kStage;
      wait_vmem();      // this wave's DMA for unit u has landed
      __syncthreads();  // every wave's; the other stage buffer is free again
      if (u + 1 < nunits) {
        const int u1 = u + 1;
        const int v1 = (c_begin + u1 / T::kUnitsPerChunk) * kChunk + (u1 % T::kUnitsPerChunk) * T::kUnit;
        T::stage(lds + (u1 & 1) * T::kStage, zsrc, tsrc, Wt, V, v1, wave, lane);
      }
      if (!wave_on) continue;

      // draft mode: the accumulator starts from the logits (D = logits + bias);
      // verify mode: from zero, so that the Markov term of a residual row is
      // accumulated at its own small magnitude and the logits are added once,
      // in the epilogue (the residual is sensitive to that rounding)
      f32x16_t acc[T::kMt];
#pragma unroll
      for (int mt = 0; mt < T::kMt; ++mt) {
        float z[16];
        if (MODE == MODE_DRAFT) read16<ZT, T>(cur, prow, (mt * 32 + 16 * h) * (int)sizeof(ZT) / 16, z);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mt][i] = MODE == MODE_DRAFT ? z[i] : 0.f;
      }
#pragma unroll
      for (int t = 0; t < T::kSteps; ++t) {
#pragma unroll
        for (int mt = 0; mt < T::kMt; ++mt) {
          const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(cur + T::w_off(mt * 32 + wrow, 2 * t + h));
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bfrag[t], acc[mt], 0, 0, 0);
        }
      }
      if (!rv) continue;
      const bool ragged = v0 + T::kUnit > V;

      if (MODE == MODE_VERIFY && resid) {
        // residual max(0, p - q) of the rejected position; q from the same tiles as the draft
        ResidSums sums;
        sums.clear();
#pragma unroll
        for (int mt = 0; mt < T::kMt; ++mt) {
          float tz[16], zz[16];
          read16<ZT, T>(cur + T::kZBytes, prow, (mt * 32 + 16 * h) * (int)sizeof(ZT) / 16, tz);
          read16<ZT, T>(cur, prow, (mt * 32 + 16 * h) * (int)sizeof(ZT) / 16, zz);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            // entries past V: the target and draft logit -inf, so every weight is 0
            const bool in = !ragged || v0 + mt * 32 + 16 * h + i < V;
            sums.add(i, resid_entry(in ? tz[i] : -INFINITY, in ? zz[i] : -INFINITY, acc[mt][i], scale2, lsp2, lsq2,
                                    dlp));
          }
        }
        const float rs = ResidSums::fold(sums.r);
        cs += rs;
        Rs += (double)rs;
        QAs += (double)ResidSums::fold(sums.qa);
        Zps += (double)ResidSums::fold(sums.p);
        Zqs += (double)ResidSums::fold(sums.q);
      } else {
        if (MODE == MODE_VERIFY) {  // a bonus row: its target row (the logits tile); no draft term
#pragma unroll
          for (int mt = 0; mt < T::kMt; ++mt) {
            float zz[16];
            read16<ZT, T>(cur, prow, (mt * 32 + 16 * h) * (int)sizeof(ZT) / 16, zz);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][i] += zz[i];
          }
        }
        if (ragged) {
#pragma unroll
          for (int mt = 0; mt < T::kMt; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (v0 + mt * 32 + 16 * h + i >= V) acc[mt][i] = -INFINITY;
        }
        float m = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < T::kMt; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) m = fmaxf(m, acc[mt][i]);
        m = fmaxf(m, __shfl_xor(m, 32));
        float s = 0.f;
        if (m != -INFINITY) {
          const float off = -m * scale2;
#pragma unroll
          for (int mt = 0; mt < T::kMt; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) s += __builtin_amdgcn_exp2f(fmaf(acc[mt][i], scale2, off));
        }
        s += __shfl_xor(s, 32);
        lse2_merge(cm, cs, m * scale2, s);
      }
      if (part == T::kUnitsPerChunk - 1) {  // chunk finished
        if (c >> 2 != quad_id) {
          quad = draw_quad(a.key, (uint32_t)c, (uint32_t)b, (uint32_t)kpos, purpose);
          quad_id = c >> 2;
        }
        const float gum = gumbel_from_word(quad_word(quad, c & 3));
        float score;
        if (MODE == MODE_VERIFY && resid) {
          const float rc = halves32_sum(cs);
          score = rc > 0.f ? logf(rc) + gum : -INFINITY;
        } else {
          score = cs > 0.f ? (cm + log2f(cs)) * kLn2 + gum : -INFINITY;
          if (MODE == MODE_DRAFT) lse2_merge(run_m, run_s, cm, cs);
        }
        if (score > best) {
          best = score;
          best_c = c;
        }
        cm = -INFINITY;
        cs = 0.f;
      }
    }
    __syncthreads();  // the next pass restages buffer 0
    if (MODE == MODE_DRAFT) {
      if (rv && lane < 32) a.part[(size_t)b * G + g] = make_float4(run_m, run_s, best, __int_as_float(best_c));
    } else {
      const double R_g = halves32_sum_d(Rs), QA_g = halves32_sum_d(QAs);
      const double Zp_g = halves32_sum_d(Zps), Zq_g = halves32_sum_d(Zqs);
      if (rv && lane < 32) {
        a.part[(size_t)b * G + g] = make_float4((float)R_g, (float)QA_g, best, __int_as_float(best_c));
        a.zpart[(size_t)b * G + g] = make_float2((float)Zp_g, (float)Zq_g);
      }
    }
  }
}

// ---------------------------------------------------------------- draft-step kernel (bf16 logits and factors)
// One draft step over a two-stage LDS pipeline of half chunks (DraftTiles).
// Iteration u issues the DMA of unit u+1, the MFMA chain of unit u (into
// accumulator set u & 1, seeded with the unit's logits) and the epilogue of
// unit u-1 (the other set).  The two waves sharing a SIMD (w and w+4) take
// these two independent tasks in opposite order, so one feeds the matrix pipe
// while the other runs the VALU epilogue.  A fragments are read two K-steps
// ahead of their MFMA.
#ifndef DSPARK_DRAFT_PREFETCH
#define DSPARK_DRAFT_PREFETCH 2
#endif
template <int R>
struct DraftUnit {
  using T = DraftTiles<R>;
  static constexpr int kPrefetch = DSPARK_DRAFT_PREFETCH;  // K-steps of A fragments read ahead
  template <int D = kPrefetch>
  __device__ __forceinline__ static void mma(const unsigned char* wtile, const bf16x8_t* bfrag, f32x16_t* acc) {
    constexpr int S = T::kSteps, M = T::kMt;
    bf16x8_t af[D + 1][M];
#pragma unroll
    for (int t = 0; t < D && t < S; ++t)
#pragma unroll
      for (int mt = 0; mt < M; ++mt)
        af[t][mt] = *reinterpret_cast<const bf16x8_t*>(wtile + mt * 32 * T::kWStride + 32 * t);
#pragma unroll
    for (int t = 0; t < S; ++t) {
      if (t + D < S) {
#pragma unroll
        for (int mt = 0; mt < M; ++mt)
          af[(t + D) % (D + 1)][mt] = *reinterpret_cast<const bf16x8_t*>(wtile + mt * 32 * T::kWStride + 32 * (t + D));
      }
      // keep the prefetch D K-steps ahead: without this the scheduler sinks
      // each read next to its MFMA and every MFMA pair waits a full LDS latency
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < M; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t % (D + 1)][mt], bfrag[t], acc[mt], 0, 0, 0);
    }
  }
  // accumulator <- this lane's 16 + 16 consecutive logits (entries 16h + [0,16) of each M-tile)
  __device__ __forceinline__ static void seed(const unsigned char* buf, f32x16_t* acc, int prow, int h) {
#pragma unroll
    for (int mt = 0; mt < T::kMt; ++mt) {
      const int s0 = (mt * 32 + 16 * h) * 2 / 16;
      const uint4 x = *reinterpret_cast<const uint4*>(buf + T::z_off(prow, s0));
      const uint4 y = *reinterpret_cast<const uint4*>(buf + T::z_off(prow, s0 + 1));
      const uint32_t w[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[mt][2 * i] = bf16_lo(w[i]);
        acc[mt][2 * i + 1] = bf16_hi(w[i]);
      }
    }
  }
};

// (max, sum) merge in base 2 without branches (an empty side contributes 0)
__device__ __forceinline__ void lse2_merge_nb(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  const float a = m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f(m - mn);
  const float c = m2 == -INFINITY ? 0.f : s2 * __builtin_amdgcn_exp2f(m2 - mn);
  s = a + c;
  m = mn;
}

struct DraftRowState {
  float run_m, run_s, best, cm, cs;
  int best_c;
};

// epilogue of one half chunk, branch-free; LAST closes chunk c, whose chunk
// Gumbel gc was read from the table one iteration earlier (a table read next
// to its use would wait on every DMA issued before it)
template <typename T, bool LAST>
__device__ __forceinline__ void draft_half(const f32x16_t* acc, DraftRowState& st, int c, float scale2, float gc) {
  float m = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < T::kMt; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, acc[mt][i]);
  m = halves32_max(m);
  const float off = m == -INFINITY ? 0.f : -m * scale2;
  float s = 0.f;
#pragma unroll
  for (int mt = 0; mt < T::kMt; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += __builtin_amdgcn_exp2f(fmaf(acc[mt][i], scale2, off));
  s = halves32_sum(s);
  lse2_merge_nb(st.cm, st.cs, m * scale2, s);
  if (LAST) {
    const float score = st.cs > 0.f ? (st.cm + __log2f(st.cs)) * kLn2 + gc : -INFINITY;
    lse2_merge_nb(st.run_m, st.run_s, st.cm, st.cs);
    const bool take = score > st.best;
    st.best = take ? score : st.best;
    st.best_c = take ? c : st.best_c;
    st.cm = -INFINITY;
    st.cs = 0.f;
  }
}

// Ragged tail of the vocabulary: logits of entries >= V become -inf (Wt rows
// past V already read as zero through the buffer bound).  Final unit(s) only.
template <typename T>
__device__ __forceinline__ void mask_tail(unsigned char* buf, int v0, int V, int tid) {
  const int nvalid = V - v0;
  for (int e = tid; e < kRowsPerPass * T::kUnit; e += kThreads) {
    const int row = e / T::kUnit, col = e % T::kUnit;
    if (col >= nvalid) reinterpret_cast<uint16_t*>(buf + T::z_off(row, col / 8))[col % 8] = 0xFF80u;  // -inf
  }
}

// Chunk Gumbels of one row, one Philox quad per four consecutive chunks: the
// two half-waves holding the row each evaluate two of the four Gumbels and
// swap them.  The quad index is wave-uniform, so the refill branch is scalar.
struct ChunkGumbels {
  int quad = -1;
  float4 g;  // one vector value: picking a component must not become an indexed (scratch) load
  __device__ __forceinline__ float get(Key key, int b, int k, int c, int h, uint32_t purpose = kDraftChunk) {
    if ((c >> 2) != quad) {
      quad = c >> 2;
      const Words4 w = draw_quad(key, (uint32_t)(quad * 4), (uint32_t)b, (uint32_t)k, purpose);
      const float x0 = gumbel_from_word(h ? w.w[2] : w.w[0]);
      const float x1 = gumbel_from_word(h ? w.w[3] : w.w[1]);
      const float2 e0 = halves32(x0), e1 = halves32(x1);
      g = make_float4(e0.x, e1.x, e0.y, e1.y);
    }
    const float4 v = g;
    const int i = c & 3;
    const float lo = (i & 1) ? v.y : v.x, hi = (i & 1) ? v.w : v.z;
    return (i & 2) ? hi : lo;
  }
};

// FIRST (position 1 of the Markov head): the B fragments are the E rows of the
// anchors, gathered straight from E (two lanes per row, one 16-byte piece per
// K-step each) instead of from the fragment-ordered region a select kernel
// wrote.  buf0 / buf1: the two LDS stages, distinct __shared__ objects of the
// kernel (the compiler gives them separate alias scopes, so reads of one stage
// need not wait for the DMA still landing in the other).
template <int R, bool FIRST>
__device__ __forceinline__ void draft_step(const StreamArgs& a, unsigned char* buf0, unsigned char* buf1) {
  using T = DraftTiles<R>;
  using D = DraftUnit<R>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x, g = blockIdx.x;
  int c_begin, c_end;
  chunk_range(g, G, a.nchunks, c_begin, c_end);
  const int nc = c_end - c_begin;
  const uint16_t* Z = static_cast<const uint16_t*>(a.Z);
  const int V = a.V, K = a.K, B = a.B, k = a.k;
  const float scale2 = a.scale2;
  const int h = lane >> 5;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.Wt, (uint32_t)((size_t)V * T::kWRow));
  const uint32_t zrow_bytes = (uint32_t)((size_t)K * V * 2);
  // this lane's A-fragment base in a Wt tile: LDS row (lane & 31) of M-tile 0, slot h
  const int abase = T::kZBytes + (lane & 31) * T::kWStride + 16 * h;

  for (int base = 0; base < B; base += kRowsPerPass) {
    const int rows_valid = B - base < kRowsPerPass ? B - base : kRowsPerPass;
    const __amdgpu_buffer_rsrc_t zr =
        make_rsrc(Z + ((size_t)base * K + (k - 1)) * V, (uint32_t)((size_t)(rows_valid - 1) * zrow_bytes + (size_t)V * 2));
    DraftDma<R> dma;
    dma.init(wave, lane, rows_valid, zrow_bytes);
    const int prow = wave * 32 + (lane & 31);
    const int b = base + prow;
    const bool rv = b < B;
    const int vb = c_begin * kChunk;
    // Fill: the first unit's tiles, this wave's B fragments (the E rows of the
    // previous tokens, stored in fragment order so that each K-step is one
    // contiguous 1 KB block), then the second unit's tiles.  Compute starts
    // when all but the second unit have landed; the first chunk Gumbels are
    // drawn in the meantime.  (FIRST: the anchor is loaded ahead of the first
    // stage, so waiting for it leaves that stage in flight.)
    bf16x8_t bfrag[T::kSteps];
    if (FIRST) {
      const int anc = a.anchor[rv ? b : B - 1];
      __builtin_amdgcn_sched_barrier(0);
      dma.stage(buf0, zr, wr, vb, wave);
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8_t* src =
          reinterpret_cast<const bf16x8_t*>(static_cast<const uint16_t*>(a.E) + (size_t)clamp_id(anc, V) * R + 8 * h);
#pragma unroll
      for (int t = 0; t < T::kSteps; ++t) bfrag[t] = src[2 * t];
    } else {
      // the fragments (L2-resident, written by the selection) ahead of the first
      // stage's DMA, so that they do not queue behind 64 KB of HBM requests
      const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(a.efrag) + (size_t)((base >> 5) + wave) * T::kSteps * 64 + lane;
#pragma unroll
      for (int t = 0; t < T::kSteps; ++t) bfrag[t] = src[t * 64];  // rows past B: unwritten slots, own column only
      __builtin_amdgcn_sched_barrier(0);
      dma.stage(buf0, zr, wr, vb, wave);
    }
    __builtin_amdgcn_sched_barrier(0);
    dma.stage(buf1, zr, wr, vb + T::kUnit, wave);  // every workgroup has at least one chunk (two units)
    __builtin_amdgcn_sched_barrier(0);
    ChunkGumbels cg;
    float g_prev = cg.get(a.key, b, k, c_begin, h);  // chunk Gumbel of the chunk the next closing epilogue ends
    DraftRowState st;
    st.run_m = -INFINITY;
    st.run_s = 0.f;
    st.best = -INFINITY;
    st.cm = -INFINITY;
    st.cs = 0.f;
    st.best_c = 0x7fffffff;

    f32x16_t acc0[T::kMt], acc1[T::kMt];
    // chunk c_begin: first half (nothing pending yet), then second half
    DraftDma<R>::wait_all_but_last_stage();
    barrier_lds_only();
    if (vb + T::kUnit > V) {
      mask_tail<T>(buf0, vb, V, tid);
      __syncthreads();
    }
    D::seed(buf0, acc0, prow, h);
    D::mma(buf0 + abase, bfrag, acc0);
    wait_vmem();
    __syncthreads();
    if (nc > 1) dma.stage_z(buf0, zr, vb + kChunk, wave);
    if (vb + 2 * T::kUnit > V) {
      mask_tail<T>(buf1, vb + T::kUnit, V, tid);
      __syncthreads();
    }
    D::seed(buf1, acc1, prow, h);
    D::mma(buf1 + abase, bfrag, acc1);
    __builtin_amdgcn_sched_barrier(0);
    if (nc > 1) dma.stage_w(buf0, wr, vb + kChunk, wave);
    __builtin_amdgcn_sched_barrier(0);
    draft_half<T, false>(acc0, st, c_begin, scale2, 0.f);
    for (int j = 1; j < nc; ++j) {
      const int c = c_begin + j;
      const int v0 = c * kChunk;
      // unit 2j (first half of chunk c) from buf0, with the epilogue closing chunk c-1
      wait_vmem();
      __syncthreads();
      // the next unit's logits tile now, its Wt tile between this unit's two
      // phases: the waves do not all block in issue before computing
      dma.stage_z(buf1, zr, v0 + T::kUnit, wave);
      const float g_cur = cg.get(a.key, b, k, c, h);  // closes chunk c in the next iteration
      if (v0 + T::kUnit > V) {
        mask_tail<T>(buf0, v0, V, tid);
        __syncthreads();
      }
      if (wave & 4) {  // the partner wave on this SIMD runs the other order: MFMA and VALU overlap
        draft_half<T, true>(acc1, st, c - 1, scale2, g_prev);
        __builtin_amdgcn_sched_barrier(0);
        dma.stage_w(buf1, wr, v0 + T::kUnit, wave);
        __builtin_amdgcn_sched_barrier(0);
        D::seed(buf0, acc0, prow, h);
        D::mma(buf0 + abase, bfrag, acc0);
      } else {
        D::seed(buf0, acc0, prow, h);
        D::mma(buf0 + abase, bfrag, acc0);
        __builtin_amdgcn_sched_barrier(0);
        dma.stage_w(buf1, wr, v0 + T::kUnit, wave);
        __builtin_amdgcn_sched_barrier(0);
        draft_half<T, true>(acc1, st, c - 1, scale2, g_prev);
      }
      g_prev = g_cur;
      // unit 2j+1 (second half of chunk c) from buf1, with the epilogue of unit 2j
      wait_vmem();
      __syncthreads();
      const bool more = j + 1 < nc;
      if (more) dma.stage_z(buf0, zr, v0 + kChunk, wave);
      if (v0 + 2 * T::kUnit > V) {
        mask_tail<T>(buf1, v0 + T::kUnit, V, tid);
        __syncthreads();
      }
      if (wave & 4) {
        draft_half<T, false>(acc0, st, c, scale2, 0.f);
        __builtin_amdgcn_sched_barrier(0);
        if (more) dma.stage_w(buf0, wr, v0 + kChunk, wave);
        __builtin_amdgcn_sched_barrier(0);
        D::seed(buf1, acc1, prow, h);
        D::mma(buf1 + abase, bfrag, acc1);
      } else {
        D::seed(buf1, acc1, prow, h);
        D::mma(buf1 + abase, bfrag, acc1);
        __builtin_amdgcn_sched_barrier(0);
        if (more) dma.stage_w(buf0, wr, v0 + kChunk, wave);
        __builtin_amdgcn_sched_barrier(0);
        draft_half<T, false>(acc0, st, c, scale2, 0.f);
      }
    }
    draft_half<T, true>(acc1, st, c_end - 1, scale2, g_prev);
    __syncthreads();  // the next pass restages buf0
    if (rv && lane < 32) a.part[(size_t)b * G + g] = make_float4(st.run_m, st.run_s, st.best, __int_as_float(st.best_c));
  }
}

template <int R>
__global__ __launch_bounds__(kThreads, 1) void k_draft(StreamArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char buf0[DraftTiles<R>::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char buf1[DraftTiles<R>::kStage];
  draft_step<R, false>(a, buf0, buf1);
}

template <int R>
__global__ __launch_bounds__(kThreads, 1) void k_draft_first(StreamArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char buf0[DraftTiles<R>::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char buf1[DraftTiles<R>::kStage];
  draft_step<R, true>(a, buf0, buf1);
}


// ---------------------------------------------------------------- verify resample pass
// One pass over the vocabulary for every request's final draw of the cycle
// (bf16 logits and factors): the residual max(0, p - q) at the first
// rejection k* (p: target row k*, q: the draft distribution at k*, recomputed
// as logits + E[x_{k*-1}] Wt^T), or, when every scheduled position passed, the
// bonus target row n_b + 1.  Per chunk: the residual mass (or the bonus row's
// log-partition) and its chunk Gumbel score; per (row, workgroup) the mass and
// the best chunk, which the finishing kernel merges.
//
// The draft step's tile machinery with 64-entry units: per stage a target tile
// (256 requests x 128 bytes, the draft kernel's logits-tile layout) and a Wt
// tile, 65 KB, two stages.  The residual rows' draft logits only seed the MFMA
// accumulator, so they go straight to registers (two 16-byte buffer loads per
// lane and M-tile, one unit ahead; a bonus row's, or a row past the batch, read
// past the buffer: zeros, no traffic) instead of a third tile.  The B fragments
// come from the fragment-ordered region that the acceptance kernel fills
// (zeros for bonus rows, whose q is 0).
struct VerifyRowState {
  float best, cm, cs;
  int best_c;
  double R, QA, Zp, Zq;  // residual rows: sums of r, qa, p^ and q^ over this lane's entries
};

template <int R>
struct VerifyDma {
  using T = DraftTiles<R>;
  static constexpr int kZPer = T::kZBytes / 1024 / kWaves;
  static constexpr int kWPer = (T::kWBlocks + kWaves - 1) / kWaves;
  static constexpr uint32_t kOutOfRange = 0x80000000u;
  uint32_t toff[kZPer], woff[kWPer];
  __device__ __forceinline__ void init(int wave, int lane, const uint32_t* trow_lds) {
#pragma unroll
    for (int j = 0; j < kZPer; ++j) {
      const int blk = wave + j * kWaves;
      const int row = blk * T::kZRowsPerBlk + lane / T::kZSlots;
      const int sl = (lane % T::kZSlots) ^ (row & (T::kZSlots - 1));
      toff[j] = trow_lds[row] + (uint32_t)sl * 16;
    }
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      const int blk = wave + j * kWaves;
      const int byte = blk * 1024 + lane * 16;
      const int lrow = byte / T::kWStride, slot = (byte % T::kWStride) / 16;
      const bool real = slot < T::kWSlots && lrow < T::kUnit;
      const int entry = (lrow / 32) * 32 + mfma_row_entry(lrow % 32);
      woff[j] = blk >= T::kWBlocks ? kOutOfRange : real ? (uint32_t)entry * T::kWRow + (uint32_t)slot * 16 : 0u;
    }
  }
  static constexpr int kOps = kZPer + kWPer;
  // unit starting at entry v0, or (v0 < 0) a dummy stage whose reads fall past
  // the buffers (a Wt filler slot may wrap to the start of Wt: it lands in the sink)
  __device__ __forceinline__ void stage(unsigned char* buf, __amdgpu_buffer_rsrc_t tr, __amdgpu_buffer_rsrc_t wr,
                                        int v0, int wave) const {
    stage_t(buf, tr, v0, wave);
    stage_w(buf, wr, v0, wave);
  }
  // the target tile of the unit
  __device__ __forceinline__ void stage_t(unsigned char* buf, __amdgpu_buffer_rsrc_t tr, int v0, int wave) const {
    const int ts = v0 >= 0 ? v0 * 2 : (int)kOutOfRange;
#pragma unroll
    for (int j = 0; j < kZPer; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          tr, (__attribute__((address_space(3))) void*)(buf + (wave + j * kWaves) * 1024), 16, (int)toff[j], ts, 0, 0);
  }
  // the Wt tile of the unit
  __device__ __forceinline__ void stage_w(unsigned char* buf, __amdgpu_buffer_rsrc_t wr, int v0, int wave) const {
    const int ws = v0 >= 0 ? v0 * T::kWRow : (int)kOutOfRange;
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      const int blk = wave + j * kWaves;
      const int dst = blk < T::kWBlocks ? T::kZBytes + blk * 1024 : T::kSink;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void*)(buf + dst), 16,
                                               (int)woff[j], ws, 0, 0);
    }
  }
};


template <int R>
__global__ __launch_bounds__(kThreads, 1) void k_verify64(StreamArgs a) {
  using T = DraftTiles<R>;
  using D = DraftUnit<R>;
  __shared__ __attribute__((aligned(1024))) unsigned char buf0[T::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char buf1[T::kStage];
  __shared__ uint32_t s_trow[kRowsPerPass];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x, g = blockIdx.x;
  int c_begin, c_end;
  chunk_range(g, G, a.nchunks, c_begin, c_end);
  const int nunits = (c_end - c_begin) * T::kUnitsPerChunk;
  const int V = a.V, K = a.K, B = a.B;
  const float scale2 = a.scale2;
  const int h = lane >> 5;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.Wt, (uint32_t)((size_t)V * T::kWRow));
  const uint16_t* Z = static_cast<const uint16_t*>(a.Z);
  const uint16_t* Zt = static_cast<const uint16_t*>(a.Zt);
  const int abase = T::kZBytes + (lane & 31) * T::kWStride + 16 * h;

  for (int base = 0; base < B; base += kRowsPerPass) {
    const int rows_valid = B - base < kRowsPerPass ? B - base : kRowsPerPass;
    // byte offsets of each pass row's target row (rows past B read past the buffer)
    for (int row = tid; row < kRowsPerPass; row += kThreads) {
      uint32_t off = VerifyDma<R>::kOutOfRange;
      if (row < rows_valid) {
        const int bb = base + row;
        const int ks = a.job[bb];
        int nb = a.n_sched[bb];
        nb = nb < 0 ? 0 : (nb > K ? K : nb);
        off = (uint32_t)(((size_t)row * (K + 1) + (ks > 0 ? ks - 1 : nb)) * V * 2);
      }
      s_trow[row] = off;
    }
    barrier_lds_only();
    const __amdgpu_buffer_rsrc_t tr =
        make_rsrc(Zt + (size_t)base * (K + 1) * V, (uint32_t)((size_t)rows_valid * (K + 1) * V * 2));
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(Z + (size_t)base * K * V, (uint32_t)((size_t)rows_valid * K * V * 2));
    VerifyDma<R> dma;
    dma.init(wave, lane, s_trow);

    const int prow = wave * 32 + (lane & 31);
    const int b = base + prow;
    const bool rv = b < B;
    bool resid = false;
    int kpos = 1;
    uint32_t purpose = kBonusChunk;
    float lsq2 = INFINITY, lsp2 = 0.f;  // a bonus row: q = exp2(-inf) = 0
    float dlp = -INFINITY;              // lsp2 - lsq2 (a bonus row: every weight is p^)
    uint32_t zoff = VerifyDma<R>::kOutOfRange;  // this lane's draft-logit row (residual rows only)
    if (rv) {
      const int ks = a.job[b];
      if (ks > 0) {
        resid = true;
        kpos = ks;
        purpose = kResidChunk;
        lsq2 = a.lse_q[(size_t)b * K + ks - 1] * kLog2e;
        lsp2 = a.lse_p[(size_t)b * K + ks - 1] * kLog2e;
        dlp = lsp2 - lsq2;
        zoff = (uint32_t)(((size_t)prow * K + (ks - 1)) * V * 2);
      } else {
        int nb = a.n_sched[b];
        nb = nb < 0 ? 0 : (nb > K ? K : nb);
        kpos = nb + 1;
      }
    }
    const int v_first = c_begin * kChunk;
    auto unit_v0 = [&](int u) { return u < nunits ? v_first + u * T::kUnit : -1; };
    // this lane's 2 x 16 draft logits of unit u (entries mt * 32 + 16h + [0, 16))
    auto zload = [&](int u, u32x4_t (&zr4)[4]) {
      const int v0 = unit_v0(u);
      const uint32_t zo = v0 >= 0 ? zoff : VerifyDma<R>::kOutOfRange;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          zr4[2 * mt + q] = __builtin_amdgcn_raw_buffer_load_b128(
              zr, (int)(zo + (uint32_t)((v0 < 0 ? 0 : v0) + mt * 32 + 16 * h) * 2u + 16u * q), 0, 0);
    };
    bf16x8_t bfrag[T::kSteps];
    {
      const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(a.efrag) + (size_t)((base >> 5) + wave) * T::kSteps * 64 + lane;
#pragma unroll
      for (int t = 0; t < T::kSteps; ++t) bfrag[t] = src[t * 64];
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4_t zA[4];  // this lane's draft logits of the current unit (loaded after the previous unit's epilogue)
    dma.stage(buf0, tr, wr, unit_v0(0), wave);
    zload(0, zA);
    __builtin_amdgcn_sched_barrier(0);

    VerifyRowState st;
    st.R = st.QA = st.Zp = st.Zq = 0.0;
    st.best = -INFINITY;
    st.cm = -INFINITY;
    st.cs = 0.f;
    st.best_c = 0x7fffffff;
    ChunkGumbels cg;
    const bool any_bonus = __builtin_amdgcn_ballot_w64(!resid) != 0;  // this wave holds a bonus row

    // z: this unit's draft logits on entry, the next unit's requested into the same registers at the end
    auto step = [&](int u, unsigned char* cur, unsigned char* nxt, u32x4_t (&z)[4]) {
      // unit u's tiles have landed (the four draft-logit loads requested after
      // them may still be in flight: they are first read in the epilogue, after
      // the MFMAs, where the compiler waits for them)
      wait_vmem_n<4>();
      barrier_lds_only();   // everyone's tiles have; unit u - 1's stage is free
      // the next unit's requests in two bursts: its target tile now, its Wt
      // tile and draft logits after this unit's MFMA, so the waves do not all
      // block in issue before computing
      dma.stage_t(nxt, tr, unit_v0(u + 1), wave);
      if (u >= nunits) {
        zload(u + 1, z);
        dma.stage_w(nxt, wr, unit_v0(u + 1), wave);
        return;
      }
      const int v0 = v_first + u * T::kUnit;
      if (v0 + T::kUnit > V) {  // ragged tail (final unit only): targets past V become -inf
        mask_tail<T>(cur, v0, V, tid);
        barrier_lds_only();
      }
      // the Markov term from zero: accumulated at its own small magnitude, the
      // draft logits added once, in the epilogue (the residual is sensitive to
      // a rounding at the logits' magnitude at every step of the contraction)
      f32x16_t acc[T::kMt];
#pragma unroll
      for (int mt = 0; mt < T::kMt; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
      D::template mma<1>(cur + abase, bfrag, acc);  // A fragments one K-step ahead (registers are short here)
      __builtin_amdgcn_sched_barrier(0);
      dma.stage_w(nxt, wr, unit_v0(u + 1), wave);
      __builtin_amdgcn_sched_barrier(0);
      // this lane's 16 target logits of M-tile mt, read from the tile when needed
      // (the 32 of a unit are never all held in registers)
      auto tload = [&](int mt, float (&t)[16]) {
        const int s0 = (mt * 32 + 16 * h) * 2 / 16;
        const uint4 x = *reinterpret_cast<const uint4*>(cur + T::z_off(prow, s0));
        const uint4 y = *reinterpret_cast<const uint4*>(cur + T::z_off(prow, s0 + 1));
        const uint32_t w[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          t[2 * i] = bf16_lo(w[i]);
          t[2 * i + 1] = bf16_hi(w[i]);
        }
      };
      // One formula for both kinds of row, resid_entry with t the target, z the
      // draft logit and bias the Markov term.  A residual row: o and lq are the
      // log2 partitions, so r is the residual weight of the entry.  A bonus row:
      // lq = +inf (no draft term), dlp = -inf and o = the unit's maximum, so r
      // is the target weight relative to that maximum, merged into the chunk's
      // log-partition once per unit.  Entries past V hold -inf targets and draft
      // logits: every weight 0.
      // draft logit of entry i of M-tile mt (residual rows; zeros for a bonus row); in
      // the ragged last unit the 16-byte pieces past V (wholly past it, V % 8 == 0)
      // are set to -inf once, so that the entries need no test
      if (v0 + T::kUnit > V) {
#pragma unroll
        for (int pc = 0; pc < 4; ++pc)
          if (v0 + (pc >> 1) * 32 + 16 * h + 8 * (pc & 1) >= V)
            z[pc] = u32x4_t{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
      }
      auto zl = [&](int mt, int i) {
        const uint32_t w = z[2 * mt + (i >> 3)][(i >> 1) & 3];
        return (i & 1) ? bf16_hi(w) : bf16_lo(w);
      };
      float off = lsp2, mb = -INFINITY;
      if (any_bonus) {
        float m = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < T::kMt; ++mt) {
          float t[16];
          tload(mt, t);
#pragma unroll
          for (int i = 0; i < 16; ++i) m = fmaxf(m, t[i]);
        }
        m = halves32_max(m);
        mb = m * scale2;
        if (!resid) off = m == -INFINITY ? 0.f : mb;
      }
      ResidSums sums;
      sums.clear();
#pragma unroll
      for (int mt = 0; mt < T::kMt; ++mt) {
        float t[16];
        tload(mt, t);
#pragma unroll
        for (int i = 0; i < 16; ++i) sums.add(i, resid_entry(t[i], zl(mt, i), acc[mt][i], scale2, off, lsq2, dlp));
      }
      const float rs = ResidSums::fold(sums.r);
      if (any_bonus) {
        const float sb = halves32_sum(rs);
        if (!resid) lse2_merge(st.cm, st.cs, mb, sb);
      }
      if (resid) {
        st.cs += rs;
        st.R += (double)rs;
        st.QA += (double)ResidSums::fold(sums.qa);
        st.Zp += (double)ResidSums::fold(sums.p);
        st.Zq += (double)ResidSums::fold(sums.q);
      }
      if ((u & (T::kUnitsPerChunk - 1)) == T::kUnitsPerChunk - 1) {  // chunk closes
        const int c = c_begin + u / T::kUnitsPerChunk;
        const float gum = cg.get(a.key, b, kpos, c, h, purpose);
        float score;
        if (resid) {
          const float rc = halves32_sum(st.cs);
          score = rc > 0.f ? logf(rc) + gum : -INFINITY;
        } else {
          score = st.cs > 0.f ? (st.cm + log2f(st.cs)) * kLn2 + gum : -INFINITY;
        }
        if (score > st.best) {
          st.best = score;
          st.best_c = c;
        }
        st.cm = -INFINITY;
        st.cs = 0.f;
      }
      // the next unit's draft logits once this unit's are consumed (one
      // register set for both)
      zload(u + 1, z);
    };
    // the first step is peeled (the fragments are first used outside the loop)
    step(0, buf0, buf1, zA);
    for (int u = 1; u < nunits; u += 2) {
      step(u, buf1, buf0, zA);
      step(u + 1, buf0, buf1, zA);
    }
    wait_vmem();         // the dummy stages have landed
    barrier_lds_only();  // the next pass restages the ring and the row offsets
    const double R_g = halves32_sum_d(st.R), QA_g = halves32_sum_d(st.QA);
    const double Zp_g = halves32_sum_d(st.Zp), Zq_g = halves32_sum_d(st.Zq);
    if (rv && lane < 32) {
      a.part[(size_t)b * G + g] = make_float4((float)R_g, (float)QA_g, st.best, __int_as_float(st.best_c));
      a.zpart[(size_t)b * G + g] = make_float2((float)Zp_g, (float)Zq_g);
    }
  }
}

// ---------------------------------------------------------------- select kernel
// One workgroup per row.  The loads that do not depend on the winning chunk
// (the previous token, then its E half row) are issued before the partials
// are merged, so the chain is: partials -> winning chunk -> its Wt rows.
template <typename ZT, typename WT, int R>
__global__ __launch_bounds__(256) void k_select(SelectArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, V = a.V;
  __shared__ float s_m[4], s_s[4], s_best[4], s_ell[kChunk];
  __shared__ int s_c[4];

  const int j = tid >> 1, h = tid & 1;
  // the partials first (G <= 256: at most one per thread), so that the merge
  // waits for nothing else; then the previous token and its E half row
  const float4 p = tid < a.G ? a.part[(size_t)b * a.G + tid] : make_float4(-INFINITY, 0.f, -INFINITY, 0.f);
  HalfRow<WT, R> erow;
  if (a.state) {  // RNN head: the state of position k
    erow.load_f32(a.state + ((size_t)b * K + (a.k - 1)) * R, h);
  } else {
    const int prev = clamp_id(a.k == 1 ? a.anchor[b] : a.tok[(size_t)b * K + a.k - 2], V);
    erow.load(static_cast<const WT*>(a.E) + (size_t)prev * R, h);
  }

  // 1. the winning chunk of row b: argmax of the chunk scores over the partials
  // (the log-partition, needed only for log q, is merged later, off this path)
  float best = -INFINITY;
  int bc = 0x7fffffff;
  if (tid < a.G) {
    const int pc = __float_as_int(p.w);
    if (better(p.z, pc, best, bc)) {
      best = p.z;
      bc = pc;
    }
  }
  wave_argmax(best, bc);
  if (lane == 0) {
    s_best[wave] = best;
    s_c[wave] = bc;
  }
  __syncthreads();
  int cstar;
  {
    float B0 = s_best[0];
    int C0 = s_c[0];
    for (int w = 1; w < 4; ++w) {
      if (better(s_best[w], s_c[w], B0, C0)) {
        B0 = s_best[w];
        C0 = s_c[w];
      }
    }
    // a row without any finite chunk score (non-finite logits) falls back to chunk 0
    // (compared with the chunk count: C0 * kChunk could wrap)
    cstar = (C0 >= 0 && C0 < (V + kChunk - 1) / kChunk) ? C0 : 0;
  }

  // 2. recompute the winning chunk's logits and draw the entry
  const int v = cstar * kChunk + j;
  const bool inside = v < V;
  HalfRow<WT, R> wrow;
  wrow.load(static_cast<const WT*>(a.Wt) + (size_t)(inside ? v : 0) * R, h);
  const ZT* zrow = static_cast<const ZT*>(a.Z) + ((size_t)b * K + (a.k - 1)) * V;
  const float z = logit_at<ZT>(zrow, inside ? v : 0);
  // the entry's Gumbel and the row's log-partition do not need the Wt rows:
  // computed while they arrive
  const float gum = gumbel_from_word(draw_word(a.key, (uint32_t)v, (uint32_t)b, (uint32_t)a.k, kDraftElem));
  {
    float m = -INFINITY, s = 0.f;
    if (tid < a.G) lse2_merge(m, s, p.x, p.y);
    wave_lse2_merge(m, s);
    if (lane == 0) {
      s_m[wave] = m;
      s_s[wave] = s;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float dot = inside ? half_dot_regs<R>(erow, wrow) : 0.f;
  dot += dpp_f<kDppXor1>(dot);
  float score = -INFINITY;
  int idx = 0x7fffffff;
  if (h == 0 && inside) {
    const float ell = (z + dot) * a.inv_T;
    s_ell[j] = ell;
    score = ell + gum;
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
    float M = s_m[0], S = s_s[0];
    for (int w = 1; w < 4; ++w) lse2_merge(M, S, s_m[w], s_s[w]);
    const float lse = (M + log2f(S)) * kLn2;
    const size_t o = (size_t)b * K + (a.k - 1);
    if (X < cstar * kChunk || X >= cstar * kChunk + kChunk || X >= V) X = cstar * kChunk;  // no finite score
    a.tok[o] = X;
    a.logq[o] = s_ell[X - cstar * kChunk] - lse;
    a.lse[o] = lse;
    s_c[0] = X;
  }
  if (a.efrag) {  // the next draft step's B fragments (bf16 factors only)
    __syncthreads();
    const int X = s_c[0];
    if (tid < (R >> 3)) efrag_store_piece(a.efrag, static_cast<const uint16_t*>(a.E), X, b, R, tid);
  }
}

// Select kernel for bf16 factors.  The winning chunk's Wt rows form one
// contiguous block (128 rows x R); the 256 threads read it in 16-byte pieces,
// consecutive threads on consecutive pieces, so every wave instruction reads
// 1 KB of contiguous memory.  Thread t then holds column piece t % PR of rows
// i * (256 / PR) + t / PR (i < PR / 2; PR = R / 8 pieces per row) and the
// matching piece of the Markov operand (E[x_{k-1}], or the RNN state rounded
// to bf16), one 16-byte load per thread instead of a half row per thread.  The
// partial dot products go through LDS once: thread r < 128 sums the PR
// partials of row r in column order (a cross-lane shuffle tree costs more).
template <typename ZT, int R>
__global__ __launch_bounds__(256) void k_select_b16(SelectArgs a) {
  constexpr int PR = R / 8;                         // 16-byte pieces per Wt row (2..32)
  constexpr int NP = PR / 2;                        // pieces per thread (1..16)
  constexpr int RG = 256 / PR;                      // rows per piece step
  constexpr int STR = PR % 4 == 0 ? PR + 4 : PR;    // LDS row stride of the partials (floats)
  static_assert(NP * RG == kChunk, "one chunk of rows over the workgroup");
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, V = a.V;
  __shared__ float s_m[4], s_s[4], s_best[4], s_ell[kChunk];
  __shared__ __attribute__((aligned(16))) float s_part[kChunk * STR];
  __shared__ int s_c[4], s_x;
  const int c = tid % PR, grp = tid / PR;

  // the previous token and the partials (G <= 256: at most one per thread);
  // the piece of the Markov operand is requested with the Wt block below, so
  // that the merge waits for nothing else.  (Unconditional loads, values past
  // G masked: a branch around a load makes the compiler wait for every load in
  // flight before later ones.)
  const int prev_raw = a.k == 1 ? a.anchor[b] : a.tok[(size_t)b * K + a.k - 2];
  float4 p = a.part[(size_t)b * a.G + (tid < a.G ? tid : 0)];
  if (tid >= a.G) p = make_float4(-INFINITY, 0.f, -INFINITY, 0.f);

  // 1. the winning chunk of row b: argmax of the chunk scores over the partials
  float best = -INFINITY;
  int bc = 0x7fffffff;
  if (tid < a.G) {
    const int pc = __float_as_int(p.w);
    if (better(p.z, pc, best, bc)) {
      best = p.z;
      bc = pc;
    }
  }
  wave_argmax(best, bc);
  if (lane == 0) {
    s_best[wave] = best;
    s_c[wave] = bc;
  }
  __syncthreads();
  int cstar;
  {
    float B0 = s_best[0];
    int C0 = s_c[0];
    for (int w = 1; w < 4; ++w) {
      if (better(s_best[w], s_c[w], B0, C0)) {
        B0 = s_best[w];
        C0 = s_c[w];
      }
    }
    // a row without any finite chunk score (non-finite logits) falls back to chunk 0
    // (compared with the chunk count: C0 * kChunk could wrap)
    cstar = (C0 >= 0 && C0 < (V + kChunk - 1) / kChunk) ? C0 : 0;
  }

  // 2. the chunk's Wt block, coalesced, and this thread's operand piece; for
  // thread r < 128 the logit and Gumbel of entry r; the row's log-partition
  const int v0 = cstar * kChunk;
  const int nrow = V - v0 < kChunk ? V - v0 : kChunk;
  const uint16_t* blk = static_cast<const uint16_t*>(a.Wt) + (size_t)v0 * R;
  // (the block in two bursts around the entry Gumbel: all 64 KB at once kept
  // the waves blocked in issue, and the Gumbel's arithmetic waited behind it)
  uint4 w[NP];
  constexpr int NH = NP > 1 ? NP / 2 : NP;
#pragma unroll
  for (int i = 0; i < NH; ++i) {
    const int row = i * RG + grp;
    w[i] = *reinterpret_cast<const uint4*>(blk + (size_t)(row < nrow ? row : 0) * R + 8 * c);
  }
  // both operand loads unconditional (the state's from E's first bytes when
  // there is no state)
  uint4 ep = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.E) + (size_t)clamp_id(prev_raw, V) * R + 8 * c);
  const float4* sp = a.state ? reinterpret_cast<const float4*>(a.state + ((size_t)b * K + (a.k - 1)) * R + 8 * c)
                             : static_cast<const float4*>(a.E);
  const float4 sf0 = sp[0], sf1 = sp[1];
  const int r = tid & (kChunk - 1);
  const int v = v0 + r;
  const bool inside = tid < kChunk && r < nrow;
  const ZT* zrow = static_cast<const ZT*>(a.Z) + ((size_t)b * K + (a.k - 1)) * V;
  const float z = logit_at<ZT>(zrow, r < nrow ? v : v0);
  __builtin_amdgcn_sched_barrier(0);
  const float gum = gumbel_from_word(draw_word(a.key, (uint32_t)v, (uint32_t)b, (uint32_t)a.k, kDraftElem));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = NH; i < NP; ++i) {
    const int row = i * RG + grp;
    w[i] = *reinterpret_cast<const uint4*>(blk + (size_t)(row < nrow ? row : 0) * R + 8 * c);
  }
  {
    float m = -INFINITY, sm = 0.f;
    if (tid < a.G) lse2_merge(m, sm, p.x, p.y);
    wave_lse2_merge(m, sm);
    if (lane == 0) {
      s_m[wave] = m;
      s_s[wave] = sm;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (a.state)
    ep = make_uint4(pack_bf16x2(sf0.x, sf0.y), pack_bf16x2(sf0.z, sf0.w), pack_bf16x2(sf1.x, sf1.y),
                    pack_bf16x2(sf1.z, sf1.w));
#pragma unroll
  for (int i = 0; i < NP; ++i) s_part[(i * RG + grp) * STR + c] = dot_bf16x8(ep, w[i]);
  __syncthreads();
  float score = -INFINITY;
  int idx = 0x7fffffff;
  if (inside) {
    float dot = 0.f;
    if constexpr (STR != PR) {
      const float4* q = reinterpret_cast<const float4*>(s_part + r * STR);
#pragma unroll
      for (int j = 0; j < PR / 4; ++j) {
        const float4 x = q[j];
        dot += x.x;
        dot += x.y;
        dot += x.z;
        dot += x.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < PR; ++j) dot += s_part[r * STR + j];
    }
    const float ell = (z + dot) * a.inv_T;
    s_ell[r] = ell;
    score = ell + gum;
    idx = v;
  }
  wave_argmax(score, idx);
  // the E row of this wave's best entry, requested before the waves' results
  // meet: the winner's row (the next draft step's B operand) is then already in
  // the winning wave's registers when the token is known
  const uint16_t* E16 = static_cast<const uint16_t*>(a.E);
  const int cand = (idx >= v0 && idx < V) ? idx : v0;
  const uint4 erow_pre = *reinterpret_cast<const uint4*>(E16 + (size_t)cand * R + 8 * (lane < (R >> 3) ? lane : 0));
  if (lane == 0) {
    s_best[wave] = score;
    s_c[wave] = idx;
  }
  __syncthreads();
  if (tid == 0) {
    float B0 = s_best[0];
    int X = s_c[0];
    for (int ww = 1; ww < 4; ++ww) {
      if (better(s_best[ww], s_c[ww], B0, X)) {
        B0 = s_best[ww];
        X = s_c[ww];
      }
    }
    float M = s_m[0], S = s_s[0];
    for (int ww = 1; ww < 4; ++ww) lse2_merge(M, S, s_m[ww], s_s[ww]);
    const float lse = (M + log2f(S)) * kLn2;
    const size_t o = (size_t)b * K + (a.k - 1);
    if (X < v0 || X >= v0 + kChunk || X >= V) X = v0;  // no finite score
    a.tok[o] = X;
    a.logq[o] = s_ell[X - v0] - lse;
    a.lse[o] = lse;
    s_x = X;
  }
  if (a.efrag) {  // the next draft step's B fragments
    __syncthreads();
    const int X = s_x;
    // the wave whose candidate won stores the row it holds; if none did (no
    // finite score), wave 0 loads the row of the fallback token
    int owner = -1;
    for (int ww = 0; ww < 4; ++ww)
      if (owner < 0 && s_c[ww] == X) owner = ww;
    if (wave == (owner < 0 ? 0 : owner) && lane < (R >> 3)) {
      const uint4 v = owner < 0 ? *reinterpret_cast<const uint4*>(E16 + (size_t)X * R + 8 * lane) : erow_pre;
      a.efrag[((size_t)(b >> 5) * (R >> 4) + (lane >> 1)) * 64 + (b & 31) + 32 * (lane & 1)] = v;
    }
  }
}

}  // namespace

// ---------------------------------------------------------------- dispatch
#define DSPARK_R_CASES_BF16(ZT, MODE)                                                   \
  switch (P.r) {                                                                        \
    case 16: hipLaunchKernelGGL((k_stream<ZT, 16, MODE>), G, kThreads, 0, s, a); break;   \
    case 32: hipLaunchKernelGGL((k_stream<ZT, 32, MODE>), G, kThreads, 0, s, a); break;   \
    case 64: hipLaunchKernelGGL((k_stream<ZT, 64, MODE>), G, kThreads, 0, s, a); break;   \
    case 128: hipLaunchKernelGGL((k_stream<ZT, 128, MODE>), G, kThreads, 0, s, a); break; \
    case 256: hipLaunchKernelGGL((k_stream<ZT, 256, MODE>), G, kThreads, 0, s, a); break; \
    default: return hipErrorInvalidValue;                                               \
  }
#define DSPARK_R_CASES_VERIFY16                                                        \
  switch (P.r) {                                                                       \
    case 16: hipLaunchKernelGGL((k_verify64<16>), G, kThreads, 0, s, a); break;         \
    case 32: hipLaunchKernelGGL((k_verify64<32>), G, kThreads, 0, s, a); break;         \
    case 64: hipLaunchKernelGGL((k_verify64<64>), G, kThreads, 0, s, a); break;         \
    case 128: hipLaunchKernelGGL((k_verify64<128>), G, kThreads, 0, s, a); break;       \
    case 256: hipLaunchKernelGGL((k_verify64<256>), G, kThreads, 0, s, a); break;       \
    default: return hipErrorInvalidValue;                                              \
  }
#define DSPARK_DRAFT_K(R)                                                              \
  if (a.first_from_anchor) hipLaunchKernelGGL((k_draft_first<R>), G, kThreads, 0, s, a); \
  else hipLaunchKernelGGL((k_draft<R>), G, kThreads, 0, s, a);
#define DSPARK_R_CASES_DRAFT16                                                         \
  switch (P.r) {                                                                       \
    case 16: DSPARK_DRAFT_K(16) break;                                                 \
    case 32: DSPARK_DRAFT_K(32) break;                                                 \
    case 64: DSPARK_DRAFT_K(64) break;                                                 \
    case 128: DSPARK_DRAFT_K(128) break;                                               \
    case 256: DSPARK_DRAFT_K(256) break;                                               \
    default: return hipErrorInvalidValue;                                              \
  }
#define DSPARK_R_CASES_GENERIC(ZT, WT, MODE)                                                      \
  switch (P.r) {                                                                                 \
    case 16: hipLaunchKernelGGL((k_stream_generic<ZT, WT, 16, MODE>), G, kThreads, 0, s, a); break;   \
    case 32: hipLaunchKernelGGL((k_stream_generic<ZT, WT, 32, MODE>), G, kThreads, 0, s, a); break;   \
    case 64: hipLaunchKernelGGL((k_stream_generic<ZT, WT, 64, MODE>), G, kThreads, 0, s, a); break;   \
    case 128: hipLaunchKernelGGL((k_stream_generic<ZT, WT, 128, MODE>), G, kThreads, 0, s, a); break; \
    case 256: hipLaunchKernelGGL((k_stream_generic<ZT, WT, 256, MODE>), G, kThreads, 0, s, a); break; \
    default: return hipErrorInvalidValue;                                                        \
  }

#define DSPARK_R_CASES_SMALLB(ZT, WT)                                                            \
  switch (P.r) {                                                                                 \
    case 16: hipLaunchKernelGGL((k_verify_smallb<ZT, WT, 16>), G, kThreads, 0, s, a); break;     \
    case 32: hipLaunchKernelGGL((k_verify_smallb<ZT, WT, 32>), G, kThreads, 0, s, a); break;     \
    case 64: hipLaunchKernelGGL((k_verify_smallb<ZT, WT, 64>), G, kThreads, 0, s, a); break;     \
    case 128: hipLaunchKernelGGL((k_verify_smallb<ZT, WT, 128>), G, kThreads, 0, s, a); break;   \
    case 256: hipLaunchKernelGGL((k_verify_smallb<ZT, WT, 256>), G, kThreads, 0, s, a); break;   \
    default: return hipErrorInvalidValue;                                                        \
  }
#define DSPARK_R_CASES_SMALLB_F32W(ZT)                                                             \
  switch (P.r) {                                                                                   \
    case 16: hipLaunchKernelGGL((k_verify_smallb<ZT, float, 16>), G, kThreads, 0, s, a); break;    \
    case 32: hipLaunchKernelGGL((k_verify_smallb<ZT, float, 32>), G, kThreads, 0, s, a); break;    \
    case 64: hipLaunchKernelGGL((k_verify_smallb<ZT, float, 64>), G, kThreads, 0, s, a); break;    \
    default: return hipErrorInvalidValue;                                                          \
  }
#define DSPARK_R_CASES_F32W(ZT, MODE)                                                                \
  switch (P.r) {                                                                                     \
    case 16: hipLaunchKernelGGL((k_stream_generic<ZT, float, 16, MODE>), G, kThreads, 0, s, a); break; \
    case 32: hipLaunchKernelGGL((k_stream_generic<ZT, float, 32, MODE>), G, kThreads, 0, s, a); break; \
    case 64: hipLaunchKernelGGL((k_stream_generic<ZT, float, 64, MODE>), G, kThreads, 0, s, a); break; \
    default: return hipErrorInvalidValue;                                                            \
  }

// bf16 factors: the LDS-pipelined kernel (fp32 logits in verify mode would need
// 160 KB of LDS per two stages and use the generic kernel); fp32 factors: generic.
// The generic kernel's verify mode at B <= kSmallVerifyB: k_verify_smallb.
constexpr int kSmallVerifyB = 64;
template <int MODE>
static hipError_t launch_stream(const dspark_problem& P, const StreamArgs& a, int G, hipStream_t s) {
  const bool zb = P.logits_dtype == DSPARK_BF16, wb = P.weight_dtype == DSPARK_BF16;
  if (wb && MODE == MODE_DRAFT) {
    if (draft_uses_efrag(P)) {
      DSPARK_R_CASES_DRAFT16
    } else if (zb) {
      DSPARK_R_CASES_BF16(uint16_t, MODE_DRAFT)
    } else {
      DSPARK_R_CASES_BF16(float, MODE_DRAFT)
    }
  } else if (wb) {
    if (verify_uses_efrag(P)) {
      DSPARK_R_CASES_VERIFY16
    } else if (zb) {
      DSPARK_R_CASES_BF16(uint16_t, MODE_VERIFY)
    } else if (P.B <= kSmallVerifyB) {
      DSPARK_R_CASES_SMALLB(float, uint16_t)
    } else {
      DSPARK_R_CASES_GENERIC(float, uint16_t, MODE_VERIFY)
    }
  } else if (MODE == MODE_VERIFY && P.B <= kSmallVerifyB) {
    if (zb) {
      DSPARK_R_CASES_SMALLB_F32W(uint16_t)
    } else {
      DSPARK_R_CASES_SMALLB_F32W(float)
    }
  } else {
    if (zb) {
      DSPARK_R_CASES_F32W(uint16_t, MODE)
    } else {
      DSPARK_R_CASES_F32W(float, MODE)
    }
  }
  return hipGetLastError();
}

bool draft_uses_efrag(const dspark_problem& P) {
  // the buffer-descriptor draft kernel (bf16 logits and factors) addresses a
  // pass of 256 logits rows with 32-bit offsets, (255 * K + 1) * V * 2 bytes
  // below 2^32, and its filler DMA slots read at offset 2^31, past the end of Wt
  return P.logits_dtype == DSPARK_BF16 && P.weight_dtype == DSPARK_BF16 &&
         ((unsigned long long)(kRowsPerPass - 1) * P.K + 1) * (unsigned long long)P.V * 2ull < (1ull << 32) &&
         (unsigned long long)P.V * (unsigned long long)P.r * 2ull < (1ull << 31);
}

bool verify_uses_efrag(const dspark_problem& P) {
  // the buffer-descriptor resample kernel (bf16 logits and factors) addresses a
  // pass of 256 draft-logit and target rows through buffers below 2^31 bytes,
  // 256 * (K + 1) * V * 2, and its dummy and filler DMA slots read at offset
  // 2^31, past the end of every buffer (Wt included)
  return P.logits_dtype == DSPARK_BF16 && P.weight_dtype == DSPARK_BF16 &&
         (unsigned long long)kRowsPerPass * (P.K + 1) * (unsigned long long)P.V * 2ull < (1ull << 31) &&
         (unsigned long long)P.V * (unsigned long long)P.r * 2ull < (1ull << 31);
}

hipError_t launch_stream_draft(const dspark_problem& P, const StreamArgs& a, int G, hipStream_t s) {
  return launch_stream<MODE_DRAFT>(P, a, G, s);
}

hipError_t launch_stream_verify(const dspark_problem& P, const StreamArgs& a, int G, hipStream_t s) {
  return launch_stream<MODE_VERIFY>(P, a, G, s);
}

hipError_t launch_select(const dspark_problem& P, const SelectArgs& a, hipStream_t s) {
  const bool zb = P.logits_dtype == DSPARK_BF16, wb = P.weight_dtype == DSPARK_BF16;
#define DSPARK_SEL(ZT, WT, R) hipLaunchKernelGGL((k_select<ZT, WT, R>), P.B, 256, 0, s, a)
#define DSPARK_SEL_R32(ZT)                        \
  switch (P.r) {                                  \
    case 16: DSPARK_SEL(ZT, float, 16); break;    \
    case 32: DSPARK_SEL(ZT, float, 32); break;    \
    case 64: DSPARK_SEL(ZT, float, 64); break;    \
    default: return hipErrorInvalidValue;         \
  }
#define DSPARK_SELB(ZT)                                                                 \
  switch (P.r) {                                                                        \
    case 16: hipLaunchKernelGGL((k_select_b16<ZT, 16>), P.B, 256, 0, s, a); break;       \
    case 32: hipLaunchKernelGGL((k_select_b16<ZT, 32>), P.B, 256, 0, s, a); break;       \
    case 64: hipLaunchKernelGGL((k_select_b16<ZT, 64>), P.B, 256, 0, s, a); break;       \
    case 128: hipLaunchKernelGGL((k_select_b16<ZT, 128>), P.B, 256, 0, s, a); break;     \
    case 256: hipLaunchKernelGGL((k_select_b16<ZT, 256>), P.B, 256, 0, s, a); break;     \
    default: return hipErrorInvalidValue;                                               \
  }
  if (zb && wb) { DSPARK_SELB(uint16_t) }
  else if (zb) { DSPARK_SEL_R32(uint16_t) }
  else if (wb) { DSPARK_SELB(float) }
  else { DSPARK_SEL_R32(float) }
#undef DSPARK_SELB
#undef DSPARK_SEL_R32
#undef DSPARK_SEL
  return hipGetLastError();
}

}  // namespace dspark
