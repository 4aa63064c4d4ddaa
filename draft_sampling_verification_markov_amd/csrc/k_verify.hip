// Rejection-sampling verification of the scheduled draft prefix.
//
// DSpark page, Overview and Background: the target scores all scheduled draft
// positions in one pass, keeps the longest prefix consistent with its own
// distribution, drops everything after the first rejection, and the
// rejection-sampling rule keeps the output distributed exactly as the target.
// The rule (speculative sampling): accept x_k iff u_k <= min(1, p_k(x_k) /
// q_k(x_k)); at the first rejection draw from max(0, p - q) normalised; if all
// scheduled positions pass, draw a bonus token from the next target row.
//
//   k_rowlist  one workgroup: compact list of the rows (b, k <= n_b) to test
//              (batches up to 1,024 requests and 8,192 candidates: every k_vlse
//              workgroup builds it in LDS instead)
//   k_vlse     (row, 8192-entry segment) items: base-2 (max, sum) of target/T_s
//   k_accept   one wave per request: log-partition of each tested row,
//              log p_k(x_k), the accept draw, the first rejection
//   (k_stream in verify mode: chunk scores of the residual or bonus row)
//   k_finish   one workgroup per request: winning chunk, entry draw, emission
#include "dspark_internal.hpp"

namespace dspark {
namespace {

constexpr int kListThreads = 1024;

__global__ __launch_bounds__(kListThreads) void k_rowlist(const int32_t* n_sched, int B, int K, int32_t* rows,
                                                          int32_t* nrows) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_wsum[kListThreads / 64];
  __shared__ int s_base;
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int base = 0; base < B; base += kListThreads) {
    const int b = base + tid;
    int nb = b < B ? n_sched[b] : 0;
    nb = nb < 0 ? 0 : (nb > K ? K : nb);
    int incl = nb;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int off = s_base;
    for (int w = 0; w < wave; ++w) off += s_wsum[w];
    off += incl - nb;
    for (int j = 0; j < nb; ++j) rows[off + j] = b * 64 + j;
    __syncthreads();
    if (tid == 0) {
      int t = 0;
      for (int w = 0; w < kListThreads / 64; ++w) t += s_wsum[w];
      s_base += t;
    }
    __syncthreads();
  }
  if (tid == 0) *nrows = s_base;
}

template <typename ZT>
struct Vec16;  // one 16-byte load of logits
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void load(const uint16_t* p, float* o) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    o[0] = bf16_lo(u.x);
    o[1] = bf16_hi(u.x);
    o[2] = bf16_lo(u.y);
    o[3] = bf16_hi(u.y);
    o[4] = bf16_lo(u.z);
    o[5] = bf16_hi(u.z);
    o[6] = bf16_lo(u.w);
    o[7] = bf16_hi(u.w);
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void load(const float* p, float* o) {
    const float4 f = *reinterpret_cast<const float4*>(p);
    o[0] = f.x;
    o[1] = f.y;
    o[2] = f.z;
    o[3] = f.w;
  }
};

// Raw 16-byte pieces of one (row, segment) item, through a buffer descriptor
// over the row: entries past V, and every piece when the item does not exist
// (a zero-sized descriptor), read as zeros without a memory access, so the
// next item's loads need no branch.  (Behind a branch the compiler made the
// reduction wait for them too, and nothing overlapped.)
template <typename ZT>
struct VlseItem {
  static constexpr int kLoads = kVlseSeg / 256 / Vec16<ZT>::N;  // 16-byte loads per thread
  u32x4_t raw[kLoads];
  __device__ __forceinline__ void load(const ZT* row, bool valid, int lo, int V, int tid) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(row, valid ? (uint32_t)V * (uint32_t)sizeof(ZT) : 0u);
#pragma unroll
    for (int l = 0; l < kLoads; ++l)
      raw[l] = __builtin_amdgcn_raw_buffer_load_b128(rs, (lo + (l * 256 + tid) * Vec16<ZT>::N) * (int)sizeof(ZT), 0, 0);
  }
};

// Row code of item w: from the list in LDS (LOCAL) or the one k_rowlist wrote.
template <typename ZT, bool LOCAL>
__device__ __forceinline__ const ZT* vlse_row(const VerifyArgs& a, const int* s_rows, int w, int& b, int& k0,
                                              int& seg) {
  const int j = w / a.nseg;
  seg = w - j * a.nseg;
  const int code = __builtin_amdgcn_readfirstlane(LOCAL ? s_rows[j] : a.rows[j]);  // uniform: scalar row base
  b = code >> 6;
  k0 = code & 63;
  return static_cast<const ZT*>(a.Zt) + ((size_t)b * (a.K + 1) + k0) * a.V;
}

// With LOCAL (B <= kVlseListB, B*K <= kVlseListMax) every workgroup builds the
// compact list of the rows to test in LDS from n_sched (request b's positions
// 1..n_b, requests in order: the list k_rowlist writes), so no separate launch
// precedes this pass.
constexpr int kVlseListMax = 8192;
constexpr int kVlseListB = 1024;

// (row, segment) items, round-robin over the workgroups; the loads of the next
// item are in flight while the current one is reduced (the workgroup joins its
// waves with LDS-only barriers, which leave those loads in flight).
template <typename ZT, bool LOCAL>
__global__ __launch_bounds__(256) void k_vlse(VerifyArgs a) {
  using Vec = Vec16<ZT>;
  using It = VlseItem<ZT>;
  constexpr int kPer = kVlseSeg / 256;  // entries per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float s_m[4], s_s[4];
  __shared__ int s_rows[LOCAL ? kVlseListMax : 1];
  __shared__ int s_wsum[4];
  int M;
  if (LOCAL) {
    // n_b of requests tid, tid + 256, ... (at most four per thread), then one
    // scan per 256 requests: wave inclusive scans, the waves' totals in LDS
    const int B = a.B, K = a.K;
    int nbv[kVlseListB / 256];
#pragma unroll
    for (int q = 0; q < kVlseListB / 256; ++q) {
      const int b = tid + 256 * q;
      const int v = a.n_sched[b < B ? b : 0];
      nbv[q] = b < B ? (v < 0 ? 0 : (v > K ? K : v)) : 0;
    }
    int base = 0;
#pragma unroll
    for (int q = 0; q < kVlseListB / 256; ++q) {
      if (256 * q >= B) break;
      const int nb = nbv[q];
      int incl = nb;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      if (lane == 63) s_wsum[wave] = incl;
      __syncthreads();
      int off = base;
      for (int w2 = 0; w2 < wave; ++w2) off += s_wsum[w2];
      off += incl - nb;
      const int b = tid + 256 * q;
      for (int j = 0; j < nb; ++j) s_rows[off + j] = b * 64 + j;
      base += s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
      __syncthreads();
    }
    M = base;
  } else {
    M = *a.nrows;
  }
  const int items = __builtin_amdgcn_readfirstlane(M) * a.nseg;  // the same in every lane
  int w = blockIdx.x;
  if (w >= items) return;
  int b, k0, seg;
  const ZT* row = vlse_row<ZT, LOCAL>(a, s_rows, w, b, k0, seg);
  It cur;
  __builtin_amdgcn_sched_barrier(0);
  cur.load(row, true, seg * kVlseSeg, a.V, tid);
  __builtin_amdgcn_sched_barrier(0);
  for (; w < items; w += gridDim.x) {
    const int wn = w + gridDim.x;
    const bool vn = wn < items;
    int bn, kn, segn;
    It nxt;
    const ZT* rown = vlse_row<ZT, LOCAL>(a, s_rows, vn ? wn : w, bn, kn, segn);
    __builtin_amdgcn_sched_barrier(0);
    nxt.load(rown, vn, segn * kVlseSeg, a.V, tid);
    __builtin_amdgcn_sched_barrier(0);
    // VALU-bound (one transcendental per entry): the max is taken on the raw
    // logits, the temperature folds into one fma per entry, and only the last
    // segment of a row masks entries past V (V is a multiple of 8: a 16-byte
    // piece is wholly inside or outside)
    // The exponential is the hardware's v_exp_f32: terms below 2^-126 of the
    // segment maximum flush to zero, far below the sum's own rounding, and the
    // library exp2f's denormal range handling (a fifth of this kernel's time)
    // is gone.  (Four items in flight per workgroup instead of one: slower.)
    const int lo = seg * kVlseSeg;
    const bool full = lo + kVlseSeg <= a.V;
    float x[kPer];
    float m = -INFINITY;
#pragma unroll
    for (int l = 0; l < It::kLoads; ++l) {
      Vec::load(reinterpret_cast<const ZT*>(&cur.raw[l]), x + l * Vec::N);
      if (!full && lo + (l * 256 + tid) * Vec::N >= a.V) {
#pragma unroll
        for (int i = 0; i < Vec::N; ++i) x[l * Vec::N + i] = -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < Vec::N; ++i) m = fmaxf(m, x[l * Vec::N + i]);
    }
    m = wave_max(m);
    if (lane == 0) s_m[wave] = m;
    barrier_lds_only();
    m = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3])) * a.scale2;  // base-2 units
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) s += __builtin_amdgcn_exp2f(fmaf(x[i], a.scale2, -m));
    s = wave_sum(s);
    if (lane == 0) s_s[wave] = s;
    barrier_lds_only();
    if (tid == 0) a.vlse[((size_t)b * a.K + k0) * a.nseg + seg] = make_float2(m, s_s[0] + s_s[1] + s_s[2] + s_s[3]);
    barrier_lds_only();
    cur = nxt;
    b = bn;
    k0 = kn;
    seg = segn;
  }
}

template <typename ZT>
__global__ __launch_bounds__(64) void k_accept(VerifyArgs a) {
  const int b = blockIdx.x, k0 = threadIdx.x;
  const int K = a.K;
  int nb = a.n_sched[b];
  const int anc = a.anchor[b];
  nb = nb < 0 ? 0 : (nb > K ? K : nb);
  const bool tested = k0 < nb;
  float logp = __int_as_float(0x7fc00000);  // NaN where not verified
  bool rej = false;
  int x = 0;  // draft token of position k0 + 1 (tested positions)
  if (tested) {
    float m = -INFINITY, s = 0.f;
    const float2* part = a.vlse + ((size_t)b * K + k0) * a.nseg;
    // the segment partials in batches of loads issued together (one round trip
    // per batch: 152K entries are 19 segments), merged in segment order
    constexpr int kBatch = 20;
    for (int i0 = 0; i0 < a.nseg; i0 += kBatch) {
      float2 pv[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) pv[u] = part[i0 + u < a.nseg ? i0 + u : 0];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (i0 + u < a.nseg) lse2_merge(m, s, pv[u].x, pv[u].y);
    }
    const float lse_p = (m + log2f(s)) * kLn2;
    x = clamp_id(a.tok[(size_t)b * K + k0], a.V);
    const ZT* row = static_cast<const ZT*>(a.Zt) + ((size_t)b * (K + 1) + k0) * a.V;
    logp = logit_at<ZT>(row, x) * a.inv_T - lse_p;
    a.lse_p[(size_t)b * K + k0] = lse_p;
    const float u = uniform01(draw_word(a.key, 0u, (uint32_t)b, (uint32_t)(k0 + 1), kAccept));
    const float ratio = expf(fminf(0.f, logp - a.logq[(size_t)b * K + k0]));
    rej = !(u <= ratio);
  }
  if (k0 < K) a.logp[(size_t)b * K + k0] = logp;
  const unsigned long long mask = __ballot(rej);
  const int ks = mask ? __ffsll((long long)mask) : 0;
  if (k0 == 0) a.job[b] = ks;
  // x_{k*-1}: the anchor, or the token lane k* - 2 holds (k* <= n_b, so it was tested)
  const int prev = ks > 0 ? (ks == 1 ? clamp_id(anc, a.V) : __builtin_amdgcn_readlane(x, ks - 2)) : -1;
  if (a.efrag && k0 < (a.r >> 3)) {
    // B fragments of the resample pass: E[x_{k*-1}] for a rejection at k*, zeros for a bonus row
    if (a.state) {  // RNN head: the state of position k*
      efrag_store_piece_f32(a.efrag, ks > 0 ? a.state + ((size_t)b * K + ks - 1) * a.r : nullptr, b, a.r, k0);
    } else {
      efrag_store_piece(a.efrag, static_cast<const uint16_t*>(a.E), prev, b, a.r, k0);
    }
  }
}

// Two-level Gumbel-max over a whole row of x / T_s inside one workgroup (used
// only when a residual has no mass left after rounding: the draw falls back to p).
template <typename ZT>
__device__ int full_row_draw(const ZT* row, int V, float inv_T, Key key, int b, int k, uint32_t pc, uint32_t pe,
                             float* s_best, int* s_idx) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nc = (V + kChunk - 1) / kChunk;
  float best = -INFINITY;
  int bc = 0x7fffffff;
  for (int c = wave; c < nc; c += 4) {
    const int v0 = c * kChunk + lane, v1 = v0 + 64;
    const float x0 = v0 < V ? logit_at<ZT>(row, v0) * inv_T : -INFINITY;
    const float x1 = v1 < V ? logit_at<ZT>(row, v1) * inv_T : -INFINITY;
    const float m = wave_max(fmaxf(x0, x1));
    const float s = wave_sum(expf(x0 - m) + expf(x1 - m));
    const float score = m + logf(s) + gumbel_from_word(draw_word(key, (uint32_t)c, (uint32_t)b, (uint32_t)k, pc));
    if (better(score, c, best, bc)) {
      best = score;
      bc = c;
    }
  }
  if (lane == 0) {
    s_best[wave] = best;
    s_idx[wave] = bc;
  }
  __syncthreads();
  float B0 = s_best[0];
  int C0 = s_idx[0];
  for (int w = 1; w < 4; ++w)
    if (better(s_best[w], s_idx[w], B0, C0)) {
      B0 = s_best[w];
      C0 = s_idx[w];
    }
  // a row without any finite chunk score (non-finite logits) keeps the sentinel
  // id: chunk 0 (compared with the chunk count: C0 * kChunk could wrap)
  const int cs = (C0 >= 0 && C0 < nc) ? C0 : 0;
  __syncthreads();
  float sc = -INFINITY;
  int idx = 0x7fffffff;
  if (tid < kChunk) {
    const int v = cs * kChunk + tid;
    if (v < V) {
      sc = logit_at<ZT>(row, v) * inv_T + gumbel_from_word(draw_word(key, (uint32_t)v, (uint32_t)b, (uint32_t)k, pe));
      idx = v;
    }
  }
  wave_argmax(sc, idx);
  if (lane == 0) {
    s_best[wave] = sc;
    s_idx[wave] = idx;
  }
  __syncthreads();
  float B1 = s_best[0];
  int X = s_idx[0];
  for (int w = 1; w < 4; ++w)
    if (better(s_best[w], s_idx[w], B1, X)) {
      B1 = s_best[w];
      X = s_idx[w];
    }
  __syncthreads();
  return (X >= 0 && X < V) ? X : cs * kChunk;  // no finite score: the chunk's first entry
}

template <typename ZT, typename WT>
__global__ __launch_bounds__(256) void k_finish(VerifyArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, V = a.V;
  __shared__ float s_best[4];
  __shared__ int s_idx[4];
  __shared__ double s_d[4][4];
  __shared__ int s_y;
  __shared__ double s_R, s_mass;
  __shared__ int s_cstar;

  // merge the partials of the resample pass: residual sums (float64), winning chunk
  double R = 0.0, QA = 0.0, Zp = 0.0, Zq = 0.0;
  float best = -INFINITY;
  int bc = 0x7fffffff;
  for (int i = tid; i < a.G; i += 256) {
    const float4 p = a.part[(size_t)b * a.G + i];
    const float2 z = a.zpart[(size_t)b * a.G + i];
    R += (double)p.x;
    QA += (double)p.y;
    Zp += (double)z.x;
    Zq += (double)z.y;
    const int pc = __float_as_int(p.w);
    if (better(p.z, pc, best, bc)) {
      best = p.z;
      bc = pc;
    }
  }
  R = wave_sum_d(R);
  QA = wave_sum_d(QA);
  Zp = wave_sum_d(Zp);
  Zq = wave_sum_d(Zq);
  wave_argmax(best, bc);
  if (lane == 0) {
    s_d[wave][0] = R;
    s_d[wave][1] = QA;
    s_d[wave][2] = Zp;
    s_d[wave][3] = Zq;
    s_best[wave] = best;
    s_idx[wave] = bc;
  }
  __syncthreads();
  if (tid == 0) {
    float Bm = s_best[0];
    int C0 = s_idx[0];
    for (int w = 1; w < 4; ++w)
      if (better(s_best[w], s_idx[w], Bm, C0)) {
        Bm = s_best[w];
        C0 = s_idx[w];
      }
    double t[4];
    for (int j = 0; j < 4; ++j) t[j] = (s_d[0][j] + s_d[1][j]) + (s_d[2][j] + s_d[3][j]);
    s_R = t[0];
    s_mass = resid_mass_normalised(t[0], t[1], t[2], t[3]);
    s_cstar = (Bm == -INFINITY || C0 < 0 || C0 >= (V + kChunk - 1) / kChunk) ? -1 : C0;
  }
  __syncthreads();
  const int cstar = s_cstar;
  const int kstar = a.job[b];
  int nb = a.n_sched[b];
  nb = nb < 0 ? 0 : (nb > K ? K : nb);
  const ZT* Zt = static_cast<const ZT*>(a.Zt);

  int y = -1;
  if (kstar > 0) {
    const int k0 = kstar - 1;
    const ZT* trow = Zt + ((size_t)b * (K + 1) + k0) * V;
    if (s_R > 0.0 && cstar >= 0) {
      const ZT* zrow = static_cast<const ZT*>(a.Z) + ((size_t)b * K + k0) * V;
      const int prev = clamp_id(k0 == 0 ? a.anchor[b] : a.tok[(size_t)b * K + k0 - 1], V);
      const int j = tid >> 1, h = tid & 1;
      const int v = cstar * kChunk + j;
      const bool inside = v < V;
      float dot = 0.f;
      if (inside) {
        if constexpr (sizeof(WT) == 2) {
          dot = a.state ? half_dot_state(a.state + ((size_t)b * K + k0) * a.r, static_cast<const uint16_t*>(a.Wt), v,
                                         a.r, h)
                        : half_dot<WT>(static_cast<const WT*>(a.E), static_cast<const WT*>(a.Wt), prev, v, a.r, h);
        } else {
          dot = half_dot<WT>(static_cast<const WT*>(a.E), static_cast<const WT*>(a.Wt), prev, v, a.r, h);
        }
      }
      dot += dpp_f<kDppXor1>(dot);
      float sc = -INFINITY;
      int idx = 0x7fffffff;
      if (h == 0 && inside) {
        const float lq2 = a.lse_q[(size_t)b * K + k0] * kLog2e, lp2 = a.lse_p[(size_t)b * K + k0] * kLog2e;
        const float r = resid_entry(logit_at<ZT>(trow, v), logit_at<ZT>(zrow, v), dot, a.scale2, lp2, lq2, lp2 - lq2).r;
        if (r > 0.f) {
          sc = logf(r) + gumbel_from_word(draw_word(a.key, (uint32_t)v, (uint32_t)b, (uint32_t)kstar, kResidElem));
          idx = v;
        }
      }
      wave_argmax(sc, idx);
      if (lane == 0) {
        s_best[wave] = sc;
        s_idx[wave] = idx;
      }
      __syncthreads();
      if (tid == 0) {
        float B1 = s_best[0];
        int X = s_idx[0];
        for (int w = 1; w < 4; ++w)
          if (better(s_best[w], s_idx[w], B1, X)) {
            B1 = s_best[w];
            X = s_idx[w];
          }
        s_y = (B1 == -INFINITY) ? -1 : X;
      }
      __syncthreads();
      y = s_y;
    }
    if (y < 0) y = full_row_draw<ZT>(trow, V, a.inv_T, a.key, b, kstar, kResidChunk, kResidElem, s_best, s_idx);
  } else {
    const ZT* trow = Zt + ((size_t)b * (K + 1) + nb) * V;
    float sc = -INFINITY;
    int idx = 0x7fffffff;
    if (tid < kChunk && cstar >= 0) {
      const int v = cstar * kChunk + tid;
      if (v < V) {
        sc = logit_at<ZT>(trow, v) * a.inv_T +
             gumbel_from_word(draw_word(a.key, (uint32_t)v, (uint32_t)b, (uint32_t)(nb + 1), kBonusElem));
        idx = v;
      }
    }
    wave_argmax(sc, idx);
    if (lane == 0) {
      s_best[wave] = sc;
      s_idx[wave] = idx;
    }
    __syncthreads();
    if (tid == 0) {
      float B1 = s_best[0];
      int X = s_idx[0];
      for (int w = 1; w < 4; ++w)
        if (better(s_best[w], s_idx[w], B1, X)) {
          B1 = s_best[w];
          X = s_idx[w];
        }
      s_y = (B1 == -INFINITY) ? -1 : X;
    }
    __syncthreads();
    y = s_y;
    if (y < 0) y = full_row_draw<ZT>(trow, V, a.inv_T, a.key, b, nb + 1, kBonusChunk, kBonusElem, s_best, s_idx);
  }

  const int acc = kstar > 0 ? kstar - 1 : nb;
  for (int j = tid; j <= K; j += 256) {
    int t = -1;
    if (j < acc) t = a.tok[(size_t)b * K + j];
    else if (j == acc) t = y;
    a.out_tok[(size_t)b * (K + 1) + j] = t;
  }
  if (tid == 0) {
    a.n_acc[b] = acc;
    a.next_anchor[b] = y;
    a.resid_mass[b] = kstar > 0 ? (float)s_mass : __int_as_float(0x7fc00000);
  }
}

// Finishing kernel for bf16 logits and factors with the fragment-ordered
// operands of the resample pass: the same draw as k_finish with the loads laid
// out as in the selection kernel.  The first rejection, the schedule and this
// thread's 16-byte piece of the residual's Markov operand (which k_accept
// stored in B-fragment order: E[x_{k*-1}], the RNN state, or zeros for a bonus
// row) are requested with the partials; the winning chunk's 128 Wt rows are
// one contiguous block read with consecutive threads on consecutive pieces,
// and the partial dot products are summed through LDS (entry r by thread r).
template <int R>
__global__ __launch_bounds__(256) void k_finish_b16(VerifyArgs a) {
  constexpr int PR = R / 8, NP = PR / 2, RG = 256 / PR;
  constexpr int STR = PR % 4 == 0 ? PR + 4 : PR;
  static_assert(NP * RG == kChunk, "one chunk of rows over the workgroup");
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, V = a.V;
  __shared__ float s_best[4];
  __shared__ int s_idx[4];
  __shared__ double s_d[4][4];
  __shared__ __attribute__((aligned(16))) float s_part[kChunk * STR];
  const int c = tid % PR, grp = tid / PR;

  const int kstar = a.job[b];
  int nb = a.n_sched[b];
  nb = nb < 0 ? 0 : (nb > K ? K : nb);
  float4 p = a.part[(size_t)b * a.G + (tid < a.G ? tid : 0)];
  float2 zs = a.zpart[(size_t)b * a.G + (tid < a.G ? tid : 0)];
  if (tid >= a.G) {
    p = make_float4(0.f, 0.f, -INFINITY, 0.f);
    zs = make_float2(0.f, 0.f);
  }
  const uint4 ep = a.efrag[((size_t)(b >> 5) * (R >> 4) + (c >> 1)) * 64 + (b & 31) + 32 * (c & 1)];

  // merge the partials of the resample pass: residual sums (float64), winning chunk
  const double Rw = wave_sum_d((double)p.x), QAw = wave_sum_d((double)p.y);
  const double Zpw = wave_sum_d((double)zs.x), Zqw = wave_sum_d((double)zs.y);
  float best = p.z;
  int bc = __float_as_int(p.w);
  if (tid >= a.G) bc = 0x7fffffff;
  wave_argmax(best, bc);
  if (lane == 0) {
    s_d[wave][0] = Rw;
    s_d[wave][1] = QAw;
    s_d[wave][2] = Zpw;
    s_d[wave][3] = Zqw;
    s_best[wave] = best;
    s_idx[wave] = bc;
  }
  __syncthreads();
  float Bm = s_best[0];
  int C0 = s_idx[0];
  for (int w = 1; w < 4; ++w)
    if (better(s_best[w], s_idx[w], Bm, C0)) {
      Bm = s_best[w];
      C0 = s_idx[w];
    }
  double tot[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) tot[j] = (s_d[0][j] + s_d[1][j]) + (s_d[2][j] + s_d[3][j]);
  const int cstar = (Bm == -INFINITY || C0 < 0 || C0 >= (V + kChunk - 1) / kChunk) ? -1 : C0;
  __syncthreads();  // s_best / s_idx are reused below (and by full_row_draw)
  const uint16_t* Zt = static_cast<const uint16_t*>(a.Zt);
  const int r = tid & (kChunk - 1);
  const int v0 = cstar >= 0 ? cstar * kChunk : 0;
  const int v = v0 + r;
  const bool inside = cstar >= 0 && tid < kChunk && v < V;

  int y = -1;
  __shared__ int s_y;
  if (kstar > 0) {
    const int k0 = kstar - 1;
    const uint16_t* trow = Zt + ((size_t)b * (K + 1) + k0) * V;
    if (tot[0] > 0.0 && cstar >= 0) {
      const int nrow = V - v0 < kChunk ? V - v0 : kChunk;
      const uint16_t* blk = static_cast<const uint16_t*>(a.Wt) + (size_t)v0 * R;
      uint4 w[NP];
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int row = i * RG + grp;
        w[i] = *reinterpret_cast<const uint4*>(blk + (size_t)(row < nrow ? row : 0) * R + 8 * c);
      }
      const uint16_t* zrow = static_cast<const uint16_t*>(a.Z) + ((size_t)b * K + k0) * V;
      const float z = bf16_to_f32(zrow[r < nrow ? v : v0]);
      const float zt = bf16_to_f32(trow[r < nrow ? v : v0]);
      const float lq2 = a.lse_q[(size_t)b * K + k0] * kLog2e, lp2 = a.lse_p[(size_t)b * K + k0] * kLog2e;
      const float gum = gumbel_from_word(draw_word(a.key, (uint32_t)v, (uint32_t)b, (uint32_t)kstar, kResidElem));
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        float acc = 0.f;
        const uint4 e = ep, x = w[i];
        acc = fmaf(bf16_lo(e.x), bf16_lo(x.x), acc);
        acc = fmaf(bf16_hi(e.x), bf16_hi(x.x), acc);
        acc = fmaf(bf16_lo(e.y), bf16_lo(x.y), acc);
        acc = fmaf(bf16_hi(e.y), bf16_hi(x.y), acc);
        acc = fmaf(bf16_lo(e.z), bf16_lo(x.z), acc);
        acc = fmaf(bf16_hi(e.z), bf16_hi(x.z), acc);
        acc = fmaf(bf16_lo(e.w), bf16_lo(x.w), acc);
        acc = fmaf(bf16_hi(e.w), bf16_hi(x.w), acc);
        s_part[(i * RG + grp) * STR + c] = acc;
      }
      __syncthreads();
      float sc = -INFINITY;
      int idx = 0x7fffffff;
      if (inside) {
        float dot = 0.f;
        if constexpr (STR != PR) {
          const float4* q = reinterpret_cast<const float4*>(s_part + r * STR);
#pragma unroll
          for (int j = 0; j < PR / 4; ++j) {
            const float4 xx = q[j];
            dot += xx.x;
            dot += xx.y;
            dot += xx.z;
            dot += xx.w;
          }
        } else {
#pragma unroll
          for (int j = 0; j < PR; ++j) dot += s_part[r * STR + j];
        }
        const float rr = resid_entry(zt, z, dot, a.scale2, lp2, lq2, lp2 - lq2).r;
        if (rr > 0.f) {
          sc = logf(rr) + gum;
          idx = v;
        }
      }
      wave_argmax(sc, idx);
      if (lane == 0) {
        s_best[wave] = sc;
        s_idx[wave] = idx;
      }
      __syncthreads();
      if (tid == 0) {
        float B1 = s_best[0];
        int X = s_idx[0];
        for (int ww = 1; ww < 4; ++ww)
          if (better(s_best[ww], s_idx[ww], B1, X)) {
            B1 = s_best[ww];
            X = s_idx[ww];
          }
        s_y = (B1 == -INFINITY) ? -1 : X;
      }
      __syncthreads();
      y = s_y;
    }
    if (y < 0) y = full_row_draw<uint16_t>(trow, V, a.inv_T, a.key, b, kstar, kResidChunk, kResidElem, s_best, s_idx);
  } else {
    const uint16_t* trow = Zt + ((size_t)b * (K + 1) + nb) * V;
    float sc = -INFINITY;
    int idx = 0x7fffffff;
    if (inside) {
      sc = bf16_to_f32(trow[v]) * a.inv_T +
           gumbel_from_word(draw_word(a.key, (uint32_t)v, (uint32_t)b, (uint32_t)(nb + 1), kBonusElem));
      idx = v;
    }
    wave_argmax(sc, idx);
    if (lane == 0) {
      s_best[wave] = sc;
      s_idx[wave] = idx;
    }
    __syncthreads();
    if (tid == 0) {
      float B1 = s_best[0];
      int X = s_idx[0];
      for (int ww = 1; ww < 4; ++ww)
        if (better(s_best[ww], s_idx[ww], B1, X)) {
          B1 = s_best[ww];
          X = s_idx[ww];
        }
      s_y = (B1 == -INFINITY) ? -1 : X;
    }
    __syncthreads();
    y = s_y;
    if (y < 0) y = full_row_draw<uint16_t>(trow, V, a.inv_T, a.key, b, nb + 1, kBonusChunk, kBonusElem, s_best, s_idx);
  }

  const int acc = kstar > 0 ? kstar - 1 : nb;
  for (int j = tid; j <= K; j += 256) {
    int t = -1;
    if (j < acc) t = a.tok[(size_t)b * K + j];
    else if (j == acc) t = y;
    a.out_tok[(size_t)b * (K + 1) + j] = t;
  }
  if (tid == 0) {
    a.n_acc[b] = acc;
    a.next_anchor[b] = y;
    a.resid_mass[b] = kstar > 0 ? (float)resid_mass_normalised(tot[0], tot[1], tot[2], tot[3]) : __int_as_float(0x7fc00000);
  }
}

}  // namespace

hipError_t launch_verify_pre(const dspark_problem& P, const VerifyArgs& a, hipStream_t s) {
  const bool local = P.B <= kVlseListB && (long long)P.B * P.K <= kVlseListMax;
  hipError_t e;
  if (!local) {
    hipLaunchKernelGGL(k_rowlist, 1, kListThreads, 0, s, a.n_sched, P.B, P.K, a.rows, a.nrows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool zb = P.logits_dtype == DSPARK_BF16;
  if (zb && local) hipLaunchKernelGGL((k_vlse<uint16_t, true>), kVlseGrid, 256, 0, s, a);
  else if (zb) hipLaunchKernelGGL((k_vlse<uint16_t, false>), kVlseGrid, 256, 0, s, a);
  else if (local) hipLaunchKernelGGL((k_vlse<float, true>), kVlseGrid, 256, 0, s, a);
  else hipLaunchKernelGGL((k_vlse<float, false>), kVlseGrid, 256, 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (zb) hipLaunchKernelGGL(k_accept<uint16_t>, P.B, 64, 0, s, a);
  else hipLaunchKernelGGL(k_accept<float>, P.B, 64, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_verify_finish(const dspark_problem& P, const VerifyArgs& a, hipStream_t s) {
  const bool zb = P.logits_dtype == DSPARK_BF16, wb = P.weight_dtype == DSPARK_BF16;
  if (zb && wb && a.efrag) {
    switch (P.r) {
      case 16: hipLaunchKernelGGL(k_finish_b16<16>, P.B, 256, 0, s, a); break;
      case 32: hipLaunchKernelGGL(k_finish_b16<32>, P.B, 256, 0, s, a); break;
      case 64: hipLaunchKernelGGL(k_finish_b16<64>, P.B, 256, 0, s, a); break;
      case 128: hipLaunchKernelGGL(k_finish_b16<128>, P.B, 256, 0, s, a); break;
      case 256: hipLaunchKernelGGL(k_finish_b16<256>, P.B, 256, 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  else if (zb && wb) hipLaunchKernelGGL((k_finish<uint16_t, uint16_t>), P.B, 256, 0, s, a);
  else if (zb) hipLaunchKernelGGL((k_finish<uint16_t, float>), P.B, 256, 0, s, a);
  else if (wb) hipLaunchKernelGGL((k_finish<float, uint16_t>), P.B, 256, 0, s, a);
  else hipLaunchKernelGGL((k_finish<float, float>), P.B, 256, 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
