// RNN head: the gated recurrent sequential block (DSpark page, Method >
// Semi-autoregressive generation, the RNN head).
//
// A GRU cell (gate order reset, update, new; the reset gate scales the
// recurrent product of the new gate) runs over the block:
//   a = W_ih [h_k; E[x_{k-1}]] + b_ih,  c = W_hh s_{k-1} + b_hh,  s_0 = 0
//   rho = sigmoid(a_r + c_r), z = sigmoid(a_z + c_z), n = tanh(a_n + rho * c_n)
//   s_k = (1 - z) * n + z * s_{k-1}
// and bf16(s_k) takes the place of E[x_{k-1}] as the operand of the logit
// projection at position k.
//
// The hidden-state part of a does not depend on the drafted tokens, so one
// MFMA GEMM computes it for all B*K positions before the first step
// (k_rnn_gemm); each step then adds the embedding part and the recurrent part
// on MFMA (k_rnn_step), finishes the cell in fp32, stores s_k and writes
// bf16(s_k) in the B-fragment order the draft-step kernel reads.
#include "dspark_internal.hpp"

namespace dspark {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// ------------------------------------------------------------------ GEMM
// Gh[m][n] = sum_i H[m][i] * W[n][i] + bias[n] for m < M, n < N, i < D; W rows
// have stride ldw.  Tile 128 x 128 per workgroup, K-chunk 64, four waves of
// 64 x 64 (2 x 2 MFMA 32x32x16 tiles).  Global -> registers -> LDS with the
// global loads kGemmAhead chunks ahead (a register ring) and two LDS stages.
constexpr int kTM = 128, kTN = 128, kTK = 64, kLd = kTK + 8;  // LDS row: 144 bytes
constexpr int kGemmAhead = 2;
constexpr int kPieces = kTM * kTK / 8 / 256;                   // 16-byte pieces per thread per operand

struct GemmTiles {
  uint16_t a[2][kTM * kLd];
  uint16_t b[2][kTN * kLd];
};

struct GemmRegs {
  uint4 a[kPieces], b[kPieces];
};

__device__ __forceinline__ void gemm_fetch(const uint16_t* H, const uint16_t* W, int M, int N, int D, int ldw,
                                           int m0, int n0, int k0, int tid, GemmRegs& r) {
#pragma unroll
  for (int u = 0; u < kPieces; ++u) {
    const int idx = tid + 256 * u, row = idx / (kTK / 8), piece = idx % (kTK / 8);
    const int m = m0 + row, n = n0 + row, kk = k0 + 8 * piece;  // a last chunk past D reads zeros
    r.a[u] = m < M && kk < D ? *reinterpret_cast<const uint4*>(H + (size_t)m * D + kk) : make_uint4(0, 0, 0, 0);
    r.b[u] = n < N && kk < D ? *reinterpret_cast<const uint4*>(W + (size_t)n * ldw + kk) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void gemm_store(GemmTiles& t, int st, int tid, const GemmRegs& r) {
#pragma unroll
  for (int u = 0; u < kPieces; ++u) {
    const int idx = tid + 256 * u, row = idx / (kTK / 8), piece = idx % (kTK / 8);
    *reinterpret_cast<uint4*>(&t.a[st][row * kLd + 8 * piece]) = r.a[u];
    *reinterpret_cast<uint4*>(&t.b[st][row * kLd + 8 * piece]) = r.b[u];
  }
}

__global__ __launch_bounds__(256) void k_rnn_gemm(const uint16_t* __restrict__ H, const uint16_t* __restrict__ W,
                                                  const float* __restrict__ bias, float* __restrict__ Gh, int M, int N,
                                                  int D, int ldw) {
  __shared__ GemmTiles t;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * kTM, n0 = blockIdx.y * kTN;
  const int wm = 64 * (wave >> 1), wn = 64 * (wave & 1);
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
  const int nk = (D + kTK - 1) / kTK;  // D is a multiple of 8
  GemmRegs ring[kGemmAhead];
#pragma unroll
  for (int q = 0; q < kGemmAhead; ++q)
    if (q < nk) gemm_fetch(H, W, M, N, D, ldw, m0, n0, q * kTK, tid, ring[q]);
  gemm_store(t, 0, tid, ring[0]);
  __syncthreads();
  // chunk kc sits in LDS stage kc & 1; chunk kc + q (q < kGemmAhead) in ring[(kc + q) % kGemmAhead]
  for (int kc = 0; kc < nk; ++kc) {
    const int st = kc & 1;
    if (kc + kGemmAhead < nk) {
#pragma unroll
      for (int q = 0; q < kGemmAhead; ++q)  // the slot chunk kc held (its registers went to LDS)
        if ((kc % kGemmAhead) == q) gemm_fetch(H, W, M, N, D, ldw, m0, n0, (kc + kGemmAhead) * kTK, tid, ring[q]);
    }
#pragma unroll
    for (int ks = 0; ks < kTK / 16; ++ks) {
      bf16x8_t af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8_t*>(&t.a[st][(wm + 32 * i + (lane & 31)) * kLd + 16 * ks + 8 * (lane >> 5)]);
        bf[i] = *reinterpret_cast<const bf16x8_t*>(&t.b[st][(wn + 32 * i + (lane & 31)) * kLd + 16 * ks + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kc + 1 < nk) {
#pragma unroll
      for (int q = 0; q < kGemmAhead; ++q)
        if (((kc + 1) % kGemmAhead) == q) gemm_store(t, st ^ 1, tid, ring[q]);
      __syncthreads();
    }
  }
  // accumulator: lane l holds column l % 32 and rows 8*(e/4) + 4*(l/32) + e%4 of each 32 x 32 tile
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn + 32 * j + (lane & 31);
    if (n >= N) continue;
    const float bn = bias[n];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m < M) Gh[(size_t)m * N + n] = acc[i][j][e] + bn;
      }
  }
}

// ------------------------------------------------------------------ one step
// One workgroup of four waves per (32 requests, 32 state entries).  Three MFMA
// tiles per product (gates r, z, n of the same 32 entries): A = rows of W
// (bf16), B = the requests' operands.  The embedding operand E[x_{k-1}] is exact
// in bf16; the fp32 state enters the recurrent product as hi + lo, two bf16
// terms (hi = bf16(s), lo = bf16(s - hi)), which leaves a relative error of at
// most 2^-18 per entry.  Wave w takes a quarter of the K-steps; the partial
// accumulators are summed through LDS in wave order, and wave w then finishes
// the cell for accumulator entries 4w..4w+3 (four of the 16 entries of each lane).
constexpr int kStepWaves = 4;
constexpr int kStepUnroll = 4;  // K-steps per wave at r = 256, all loads in flight together

struct RnnStepArgs {
  const float* Gh;          // [B*K][3r]: hidden-state part of a, with b_ih
  const uint16_t* W_ih;     // [3r][d + r] (columns d.. hold the embedding part)
  const uint16_t* W_hh;     // [3r][r]
  const float* b_hh;        // [3r]
  const uint16_t* E;        // [V][r]
  const int32_t* anchor;    // [B]
  const int32_t* tok;       // [B][K]
  float* state;             // [B][K][r]
  uint4* efrag;             // B fragments of bf16(s_k) for the draft step
  int B, K, V, d, r, k;     // k: 1-based position
};

__device__ __forceinline__ void split_bf16x8(const float4 x0, const float4 x1, bf16x8_t& hi, bf16x8_t& lo) {
  const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t h0 = f32_to_bf16_bits(v[2 * q]), h1 = f32_to_bf16_bits(v[2 * q + 1]);
    h[q] = h0 | (h1 << 16);
    l[q] = pack_bf16x2(v[2 * q] - __uint_as_float(h0 << 16), v[2 * q + 1] - __uint_as_float(h1 << 16));
  }
  const uint4 hv = make_uint4(h[0], h[1], h[2], h[3]), lv = make_uint4(l[0], l[1], l[2], l[3]);
  hi = *reinterpret_cast<const bf16x8_t*>(&hv);
  lo = *reinterpret_cast<const bf16x8_t*>(&lv);
}

struct StepLds {
  float acc[kStepWaves][6][16][64];  // partial accumulators: [wave][a_r a_z a_n c_r c_z c_n][entry][lane]
  float sk[32][33];                  // s_k of the block: [request][entry]
};

__global__ __launch_bounds__(256) void k_rnn_step(RnnStepArgs a) {
  __shared__ StepLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 31, half = lane >> 5;
  const int b0 = blockIdx.x * 32, j0 = blockIdx.y * 32;
  const int R = a.r, K = a.K, k = a.k, ldw = a.d + R;
  const int b = b0 + col;
  const bool live = b < a.B;
  const bool has_prev_state = live && k >= 2;

  // the epilogue's operands first (they do not depend on the products): entries
  // jj = 8*(e/4) + 4*half + e%4 for e = 4*wave .. 4*wave + 3, i.e. 8*wave + 4*half + 0..3
  const int jb = j0 + 8 * wave + 4 * half;
  float ghv[3][4], bhv[3][4], spv[4];
  if (live) {
    const float* gh = a.Gh + ((size_t)b * K + (k - 1)) * (3 * R);
    const float* sp = a.state + ((size_t)b * K + (k >= 2 ? k - 2 : 0)) * R;
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      const float4 x = *reinterpret_cast<const float4*>(gh + g * R + jb);
      const float4 y = *reinterpret_cast<const float4*>(a.b_hh + g * R + jb);
      ghv[g][0] = x.x; ghv[g][1] = x.y; ghv[g][2] = x.z; ghv[g][3] = x.w;
      bhv[g][0] = y.x; bhv[g][1] = y.y; bhv[g][2] = y.z; bhv[g][3] = y.w;
    }
    const float4 z = k >= 2 ? *reinterpret_cast<const float4*>(sp + jb) : make_float4(0.f, 0.f, 0.f, 0.f);
    spv[0] = z.x; spv[1] = z.y; spv[2] = z.z; spv[3] = z.w;
  }

  // products over this wave's K-steps
  const int prev = live ? clamp_id(k == 1 ? a.anchor[b] : a.tok[(size_t)b * K + k - 2], a.V) : 0;
  const uint16_t* erow = a.E + (size_t)prev * R + 8 * half;  // its loads are issued after the weights'
  const float* srow = a.state + ((size_t)(live ? b : 0) * K + (k >= 2 ? k - 2 : 0)) * R + 8 * half;
  const uint16_t* wi[3];
  const uint16_t* wh[3];
#pragma unroll
  for (int g = 0; g < 3; ++g) {
    const size_t row = (size_t)g * R + j0 + col;
    wi[g] = a.W_ih + row * ldw + a.d + 8 * half;
    wh[g] = a.W_hh + row * R + 8 * half;
  }
  f32x16_t acc_a[3], acc_c[3];
#pragma unroll
  for (int g = 0; g < 3; ++g) { acc_a[g] = f32x16_t{}; acc_c[g] = f32x16_t{}; }
  const int nt = R / 16, per = (nt + kStepWaves - 1) / kStepWaves;
  const int t_begin = wave * per, t_end = min(nt, t_begin + per);
  for (int t0 = t_begin; t0 < t_end; t0 += kStepUnroll) {
    bf16x8_t be[kStepUnroll], bh[kStepUnroll], bl[kStepUnroll], aw[kStepUnroll][3], hw[kStepUnroll][3];
#pragma unroll
    for (int u = 0; u < kStepUnroll; ++u) {  // weights and states: independent of the previous token
      const int t = t0 + u;
      if (t >= t_end) break;
#pragma unroll
      for (int g = 0; g < 3; ++g) {
        aw[u][g] = *reinterpret_cast<const bf16x8_t*>(wi[g] + 16 * t);
        hw[u][g] = *reinterpret_cast<const bf16x8_t*>(wh[g] + 16 * t);
      }
      float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
      if (has_prev_state) {
        x0 = *reinterpret_cast<const float4*>(srow + 16 * t);
        x1 = *reinterpret_cast<const float4*>(srow + 16 * t + 4);
      }
      split_bf16x8(x0, x1, bh[u], bl[u]);
    }
#pragma unroll
    for (int u = 0; u < kStepUnroll; ++u) {
      const int t = t0 + u;
      if (t >= t_end) break;
      be[u] = live ? *reinterpret_cast<const bf16x8_t*>(erow + 16 * t) : bf16x8_t{};
    }
#pragma unroll
    for (int u = 0; u < kStepUnroll; ++u)
#pragma unroll
      for (int g = 0; g < 3; ++g) {
        if (t0 + u >= t_end) break;
        acc_a[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[u][g], be[u], acc_a[g], 0, 0, 0);
        acc_c[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hw[u][g], bh[u], acc_c[g], 0, 0, 0);
        acc_c[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hw[u][g], bl[u], acc_c[g], 0, 0, 0);
      }
  }
#pragma unroll
  for (int g = 0; g < 3; ++g)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      L.acc[wave][g][e][lane] = acc_a[g][e];
      L.acc[wave][3 + g][e][lane] = acc_c[g][e];
    }
  __syncthreads();

  // wave w: entries e = 4w..4w+3 of every lane, partials summed in wave order
  if (live) {
    float* so = a.state + ((size_t)b * K + (k - 1)) * R;
    float sv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * wave + q;
      float v[6];
#pragma unroll
      for (int m = 0; m < 6; ++m) {
        float t = L.acc[0][m][e][lane];
#pragma unroll
        for (int w = 1; w < kStepWaves; ++w) t += L.acc[w][m][e][lane];
        v[m] = t;
      }
      const float ar = ghv[0][q] + v[0], az = ghv[1][q] + v[1], an = ghv[2][q] + v[2];
      const float cr = bhv[0][q] + v[3], cz = bhv[1][q] + v[4], cn = bhv[2][q] + v[5];
      const float rho = 1.f / (1.f + expf(-(ar + cr)));
      const float z = 1.f / (1.f + expf(-(az + cz)));
      const float n = tanhf(an + rho * cn);
      sv[q] = (1.f - z) * n + z * spv[q];
      L.sk[col][jb - j0 + q] = sv[q];
    }
    *reinterpret_cast<float4*>(so + jb) = make_float4(sv[0], sv[1], sv[2], sv[3]);
  }
  if (!a.efrag) return;
  __syncthreads();
  // bf16(s_k) in B-fragment order: per request of the block 4 pieces of 8 entries
  if (tid < 128) {
    const int qq = tid >> 2, piece = tid & 3, bb = b0 + qq;
    if (bb < a.B) {
      const float* src = &L.sk[qq][8 * piece];
      const uint4 v = make_uint4(pack_bf16x2(src[0], src[1]), pack_bf16x2(src[2], src[3]),
                                 pack_bf16x2(src[4], src[5]), pack_bf16x2(src[6], src[7]));
      const int p = (j0 >> 3) + piece;  // 8-entry piece index within the row
      a.efrag[((size_t)(bb >> 5) * (R >> 4) + (p >> 1)) * 64 + (bb & 31) + 32 * (p & 1)] = v;
    }
  }
}

}  // namespace

size_t rnn_extra_bytes(const dspark_problem& P) {
  return ((size_t)P.B * P.K * 3 * P.r * sizeof(float) + 255) & ~(size_t)255;
}

bool rnn_supported(const dspark_problem& P) {
  // bf16 h for the MFMA GEMM, state blocks of 32 entries, and the fragment-fed
  // draft and resample kernels, which take the state as their operand
  return P.hidden_dtype == DSPARK_BF16 && P.r % 32 == 0 && draft_uses_efrag(P) && verify_uses_efrag(P);
}

hipError_t launch_rnn_gemm(const dspark_problem& P, const void* h, const void* W_ih, const float* b_ih, float* Gh,
                           hipStream_t s) {
  const int M = P.B * P.K, N = 3 * P.r;
  dim3 grid((M + kTM - 1) / kTM, (N + kTN - 1) / kTN);
  hipLaunchKernelGGL(k_rnn_gemm, grid, 256, 0, s, static_cast<const uint16_t*>(h),
                     static_cast<const uint16_t*>(W_ih), b_ih, Gh, M, N, P.d, P.d + P.r);
  return hipGetLastError();
}

hipError_t launch_rnn_step(const dspark_problem& P, const float* Gh, const void* W_ih, const void* W_hh,
                           const float* b_hh, const void* E, const int32_t* anchor, const int32_t* tok, float* state,
                           uint4* efrag, int k, hipStream_t s) {
  RnnStepArgs a;
  a.Gh = Gh;
  a.W_ih = static_cast<const uint16_t*>(W_ih);
  a.W_hh = static_cast<const uint16_t*>(W_hh);
  a.b_hh = b_hh;
  a.E = static_cast<const uint16_t*>(E);
  a.anchor = anchor;
  a.tok = tok;
  a.state = state;
  a.efrag = efrag;
  a.B = P.B; a.K = P.K; a.V = P.V; a.d = P.d; a.r = P.r; a.k = k;
  dim3 grid((P.B + 31) / 32, P.r / 32);
  hipLaunchKernelGGL(k_rnn_step, grid, 64 * kStepWaves, 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
