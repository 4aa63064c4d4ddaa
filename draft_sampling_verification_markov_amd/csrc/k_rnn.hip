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
// One workgroup of four waves per (16 requests, 16 state entries): 256
// workgroups at B = r = 256, so each CU takes in only its 48 weight rows and
// 16 requests' operands.  v_mfma_f32_16x16x32_bf16 tiles, three per product
// (gates r, z, n of the same 16 entries): A = rows of W (bf16), B = the
// requests' operands.  The embedding operand E[x_{k-1}] is exact in bf16; the
// fp32 state enters the recurrent product as hi + lo, two bf16 terms
// (hi = bf16(s), lo = bf16(s - hi)), which leaves a relative error of at most
// 2^-18 per entry.  Wave w takes a quarter of the K-steps of each product; the
// partial accumulators are summed through LDS in wave order, and wave w then
// finishes the cell for accumulator row w of every lane (one entry per lane).
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
constexpr int kStepWaves = 4;
constexpr int kStepTile = 16;   // requests and state entries per workgroup
constexpr int kStepMaxK = 2;    // K-steps of 32 per wave and product at r = 256 (held in registers)

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
  float acc[kStepWaves][6][4][64];      // partials: [wave][a_r a_z a_n c_r c_z c_n][row][lane]
  float sk[kStepTile][kStepTile + 1];   // s_k of the block: [request][entry]
};

__global__ __launch_bounds__(64 * kStepWaves) void k_rnn_step(RnnStepArgs a) {
  __shared__ StepLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;  // MFMA column (request) and k-group
  const int b0 = blockIdx.x * kStepTile, j0 = blockIdx.y * kStepTile;
  const int R = a.r, K = a.K, k = a.k, ldw = a.d + R;
  const int b = b0 + col;
  const bool live = b < a.B;
  const bool has_prev_state = live && k >= 2;

  // the epilogue's operands first (they do not depend on the products):
  // accumulator row `wave` of this lane is state entry j0 + 4*quad + wave
  const int je = j0 + 4 * quad + wave;
  float ghv[3] = {0.f, 0.f, 0.f}, bhv[3] = {0.f, 0.f, 0.f}, spv = 0.f;
  if (live) {
    const float* gh = a.Gh + ((size_t)b * K + (k - 1)) * (3 * R);
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      ghv[g] = gh[g * R + je];
      bhv[g] = a.b_hh[g * R + je];
    }
    if (k >= 2) spv = a.state[((size_t)b * K + (k - 2)) * R + je];
  }

  // products over this wave's K-steps (32 wide): weights and states first, the
  // token-dependent embedding row last
  const int nt = R / 32, per = (nt + kStepWaves - 1) / kStepWaves;
  const int t0 = wave * per, t1 = min(nt, t0 + per);
  const float* srow = a.state + ((size_t)(live ? b : 0) * K + (k >= 2 ? k - 2 : 0)) * R + 8 * quad;
  bf16x8_t aw[kStepMaxK][3], hw[kStepMaxK][3], bh[kStepMaxK], bl[kStepMaxK], be[kStepMaxK];
#pragma unroll
  for (int u = 0; u < kStepMaxK; ++u) {
    const int t = t0 + u;
    if (t >= t1) break;
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      const size_t row = (size_t)g * R + j0 + col;
      aw[u][g] = *reinterpret_cast<const bf16x8_t*>(a.W_ih + row * ldw + a.d + 32 * t + 8 * quad);
      hw[u][g] = *reinterpret_cast<const bf16x8_t*>(a.W_hh + row * R + 32 * t + 8 * quad);
    }
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (has_prev_state) {
      x0 = *reinterpret_cast<const float4*>(srow + 32 * t);
      x1 = *reinterpret_cast<const float4*>(srow + 32 * t + 4);
    }
    split_bf16x8(x0, x1, bh[u], bl[u]);
  }
  const int prev = live ? clamp_id(k == 1 ? a.anchor[b] : a.tok[(size_t)b * K + k - 2], a.V) : 0;
  const uint16_t* erow = a.E + (size_t)prev * R + 8 * quad;
#pragma unroll
  for (int u = 0; u < kStepMaxK; ++u) {
    const int t = t0 + u;
    if (t >= t1) break;
    be[u] = live ? *reinterpret_cast<const bf16x8_t*>(erow + 32 * t) : bf16x8_t{};
  }
  f32x4_t acc_a[3], acc_c[3];
#pragma unroll
  for (int g = 0; g < 3; ++g) { acc_a[g] = f32x4_t{}; acc_c[g] = f32x4_t{}; }
#pragma unroll
  for (int u = 0; u < kStepMaxK; ++u) {
    if (t0 + u >= t1) break;
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      acc_a[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[u][g], be[u], acc_a[g], 0, 0, 0);
      acc_c[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hw[u][g], bh[u], acc_c[g], 0, 0, 0);
      acc_c[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hw[u][g], bl[u], acc_c[g], 0, 0, 0);
    }
  }
#pragma unroll
  for (int g = 0; g < 3; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      L.acc[wave][g][e][lane] = acc_a[g][e];
      L.acc[wave][3 + g][e][lane] = acc_c[g][e];
    }
  __syncthreads();

  // wave w: accumulator row w of every lane, partials summed in wave order
  if (live) {
    float v[6];
#pragma unroll
    for (int m = 0; m < 6; ++m) {
      float t = L.acc[0][m][wave][lane];
#pragma unroll
      for (int q = 1; q < kStepWaves; ++q) t += L.acc[q][m][wave][lane];
      v[m] = t;
    }
    const float ar = ghv[0] + v[0], az = ghv[1] + v[1], an = ghv[2] + v[2];
    const float cr = bhv[0] + v[3], cz = bhv[1] + v[4], cn = bhv[2] + v[5];
    const float rho = 1.f / (1.f + expf(-(ar + cr)));
    const float z = 1.f / (1.f + expf(-(az + cz)));
    const float n = tanhf(an + rho * cn);
    const float sv = (1.f - z) * n + z * spv;
    a.state[((size_t)b * K + (k - 1)) * R + je] = sv;
    L.sk[col][je - j0] = sv;
  }
  if (!a.efrag) return;
  __syncthreads();
  // bf16(s_k) in B-fragment order: per request of the block 2 pieces of 8 entries
  if (tid < kStepTile * 2) {
    const int qq = tid >> 1, piece = tid & 1, bb = b0 + qq;
    if (bb < a.B) {
      const float* src = &L.sk[qq][8 * piece];
      const uint4 val = make_uint4(pack_bf16x2(src[0], src[1]), pack_bf16x2(src[2], src[3]),
                                   pack_bf16x2(src[4], src[5]), pack_bf16x2(src[6], src[7]));
      const int p = (j0 >> 3) + piece;  // 8-entry piece index within the row
      a.efrag[((size_t)(bb >> 5) * (R >> 4) + (p >> 1)) * 64 + (bb & 31) + 32 * (p & 1)] = val;
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
  dim3 grid((P.B + kStepTile - 1) / kStepTile, P.r / kStepTile);
  hipLaunchKernelGGL(k_rnn_step, grid, 64 * kStepWaves, 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
