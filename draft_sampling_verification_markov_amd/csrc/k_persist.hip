// Persistent Markov draft: every position of a cycle in one cooperative launch,
// each CU's slice of the logit projection Wt held on chip for the whole cycle.
//
// DSpark page, Method > Semi-autoregressive generation: the sequential stage
// adds a rank-r transition bias E[prev] . Wt^T to the base logits and samples
// position after position; the low rank is what keeps the per-position work
// small.  A launch per position re-reads all of Wt (r x V) at every position;
// here it is read once per cycle, which pays where that re-read dominates: at
// small batches, where the base logits of a position are a small fraction of
// Wt's bytes.
//
// Every workgroup (one per CU: four waves, one per SIMD) owns a contiguous
// range of at most 5 vocabulary chunks of 128 entries, 20 M-tiles of 32,
// five per wave.  A wave keeps the MFMA A fragments of its first four M-tiles
// in registers for the whole cycle (4 x 16 K-steps x 16 bytes per lane: 256
// registers) and those of its fifth in LDS (64 KB for the workgroup).
// Per position k:
//  1. the previous tokens of all rows into LDS (each awaited as in 6);
//  2. per N-tile of 32 rows: the E rows of its previous tokens arrive in LDS
//     by DMA one N-tile ahead (two buffers, rows padded by 16 bytes); per
//     M-tile the wave chains 16 MFMAs starting from the base logits (requested
//     into registers one N-tile ahead), so the chain ends at the logits, while
//     its vector unit finishes the previous M-tile: (max, sum of 2^(x - max))
//     in base 2 per (row, M-tile), into LDS;
//  3. per 128 rows: chunk log-masses, chunk Gumbels, the best chunk and the
//     running log-partition, one partial record per (row, workgroup), stored
//     past the L2 as four tagged words;
//  4. selection: workgroup g takes rows g, g + G, ...: thread t waits for
//     workgroup t's record of the row, then the row's G records are merged,
//     the winning chunk's Wt block read, its 128 logits recomputed, the entry
//     drawn, and the token, log q and the log-partition written;
//  5. the token, tagged, into each group's replica (16 groups of workgroups);
//  6. while the next position's first base logits are requested, every
//     workgroup waits for the B tokens in its group's replica.
// No grid barrier: each wait is for the tagged words it needs (a tag is the
// launch generation and the position, so a word left by an earlier position or
// launch never satisfies it), read past the L2 (an XCD's L2 is not kept coherent
// with another's).  A workgroup writes position k + 1's records only after
// every token of position k, each written after its row's records of position
// k were read, and so on: no word is overwritten before it is read.  Every wait
// is bounded: past the limit the time-out flag is set and the waits that follow
// return at once, so the kernel always ends (its results are then unspecified).
#include "dspark_internal.hpp"

namespace dspark {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kPThreads = 256;
constexpr int kPWaves = kPThreads / 64;
constexpr int kPMt = 5;                  // M-tiles of 32 entries per wave
constexpr int kPMtWg = kPWaves * kPMt;   // per workgroup: 5 chunks
constexpr int kPRows = 256;              // rows of the batch at most
constexpr int kPHalf = 128;              // rows whose M-tile partials are merged at once

// MFMA row rho of an M-tile -> vocabulary entry within it: in the 32x32
// accumulator layout lane l then holds 16 consecutive entries 16*(l/32)..+15
// of its column (request) l % 32.
__device__ __forceinline__ int prow_entry(int rho) { return ((rho >> 2) & 1) * 16 + (rho >> 3) * 4 + (rho & 3); }

// Chunks [c_begin, c_end) of workgroup g of G: an even split, the first
// nchunks % G workgroups one more (the draft step's split).
__device__ __forceinline__ void persist_chunk_range(int g, int G, int nchunks, int& c_begin, int& c_end) {
  const unsigned q = (unsigned)nchunks / (unsigned)G, rem = (unsigned)nchunks - q * (unsigned)G;
  const unsigned ug = (unsigned)g;
  c_begin = (int)(ug * q + (ug < rem ? ug : rem));
  c_end = c_begin + (int)q + (ug < rem ? 1 : 0);
}

// Word i (0..3) of a Philox quad without indexing (an indexed pick can become a scratch access).
__device__ __forceinline__ uint32_t quad_pick(const Words4& q, int i) {
  const uint32_t lo = (i & 1) ? q.w[1] : q.w[0], hi = (i & 1) ? q.w[3] : q.w[2];
  return (i & 2) ? hi : lo;
}

// Word i (0..3, a constant after unrolling) of a 16-byte piece.
__device__ __forceinline__ uint32_t u4get(const uint4& q, int i) { return i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w; }

// ZT: the base logits' type (uint16_t: bf16; float: fp32)
template <int R, typename ZT>
__global__ __launch_bounds__(kPThreads, 1) void k_draft_persist(PersistArgs a) {
  static_assert(R == 256, "one factor row per 32 lanes of a gather instruction");
  // fp32 base logits: one register set of 16-byte pieces per M-tile, refilled
  // in place as each M-tile's epilogue has read it (two sets would not fit
  // beside the 256 registers of Wt); bf16: two sets, the next N-tile's loaded whole
  constexpr bool kF32 = sizeof(ZT) == 4;
  constexpr int ZP = (int)sizeof(ZT);             // 16-byte pieces of a lane's 16 entries: 2 (bf16) or 4 (fp32)
  constexpr int EPP = 16 / (int)sizeof(ZT);      // entries per piece
  constexpr int S = R / 16;          // MFMA K-steps (16 ranks each)
  constexpr int ROWB = R * 2;        // bytes of a factor row
  constexpr int PR = R / 8;          // 16-byte pieces of a factor row
  constexpr int RG = kPThreads / PR; // selection: rows per piece step
  constexpr int NP = kChunk / RG;    // selection: Wt pieces per thread
  constexpr int STR = PR + 4;        // selection: LDS row stride of the dot partials (floats)
  constexpr int RS = PR + 1;         // LDS row stride of the E rows, in 16-byte slots (one of padding)
  constexpr int NSLOT = 32 * RS;     // slots of an N-tile's E rows
  constexpr int JR = kPMt - 1;       // M-tiles whose fragments stay in registers
  static_assert(kChunk * STR * 4 <= kPHalf * kPMtWg * 8, "the selection's partials fit the merge area");
  // A fragments of each wave's last M-tile ([wave][K-step][lane], 16 bytes each)
  __shared__ __attribute__((aligned(1024))) bf16x8_t s_a[kPWaves][S][64];
  // E rows of two N-tiles, even and odd (row rho's piece p at slot rho * RS +
  // p: the padding slot makes each K-step's fragment read one base address plus
  // a constant, and spreads the 32 rows of a read over distinct banks)
  __shared__ __attribute__((aligned(1024))) unsigned char s_b0[(NSLOT + 63) / 64 * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char s_b1[(NSLOT + 63) / 64 * 1024];
  __shared__ __attribute__((aligned(16))) float2 s_tp[kPHalf * kPMtWg];
  __shared__ int s_tok[kPRows];
  __shared__ float s_ell[kChunk], s_bm[kPWaves], s_bs[kPWaves], s_best[kPWaves];
  __shared__ int s_bi[kPWaves], s_x;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int G = gridDim.x, g = blockIdx.x;
  int c_begin, c_end;
  persist_chunk_range(g, G, a.nchunks, c_begin, c_end);
  const int nct = 4 * (c_end - c_begin);
  const int V = a.V, K = a.K, B = a.B;
  const uint16_t* Wt = static_cast<const uint16_t*>(a.Wt);
  const uint16_t* E = static_cast<const uint16_t*>(a.E);
  const ZT* Z = static_cast<const ZT*>(a.Z);
  const float scale2 = a.scale2;
  const int vbase = c_begin * kChunk;
  // hand-offs: tags are generation * 128 + position (positions are at most 64,
  // so no tag is 127 modulo 128 and 0xFFFFFFFF is an expectation no word ever
  // meets: every wait then times out)
  unsigned* const flag = a.sync + kSyncFlag * kSyncStride;
  const uint32_t gen = ld_agent(a.sync + kSyncGen * kSyncStride);
  const int ng = G < kSyncGroups ? G : kSyncGroups;
  auto tag_of = [&](int kk) { return gen * 128u + (uint32_t)kk; };
  auto expect_of = [&](int kk) { return a.unreachable ? 0xFFFFFFFFu : tag_of(kk); };

  // 0. this wave's A fragments (Wt rows of its M-tiles) for the whole cycle:
  // the first JR in registers, the last in LDS; a missing M-tile (past the
  // workgroup's chunks or past V) is zero
  bf16x8_t af[JR][S];
#pragma unroll
  for (int j = 0; j < kPMt; ++j) {
    const int mtg = wave * kPMt + j;
    const int v = vbase + mtg * 32 + prow_entry(l32);
    const bool ok = mtg < nct && v < V;
    const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(Wt + (size_t)(ok ? v : 0) * R + 8 * h);
#pragma unroll
    for (int t = 0; t < S; ++t) {
      const bf16x8_t x = ok ? src[2 * t] : bf16x8_t{};
      if (j < JR)
        af[j < JR ? j : 0][t] = x;
      else
        s_a[wave][t][lane] = x;
    }
  }

  // base logits of this lane's 16 entries of M-tile j of N-tile nt at position
  // kk: ZP 16-byte buffer loads, always issued (rows past B read row B - 1).
  // A piece past V (wholly past it, as V % 8 == 0) is read at an offset past
  // the end of Z, where the buffer returns zeros; its bits are set to -inf
  // where it is used.
  const int NT = (B + 31) / 32;
  const __amdgpu_buffer_rsrc_t zrs = make_rsrc(Z, a.z_bytes);
  const __amdgpu_buffer_rsrc_t ers = make_rsrc(E, (uint32_t)V * ROWB);
  const int vlane = vbase + wave * kPMt * 32 + 16 * h;  // this lane's first entry of the wave's M-tiles
  const int vleft = V - vlane;
  auto zload_one = [&](int kk, int nt, int j, uint4 (&zj)[ZP]) {
    const int row = nt * 32 + l32;
    const int zr = row < B ? row : B - 1;
    const uint32_t off = (uint32_t)((((size_t)zr * K + (kk - 1)) * V + vlane) * sizeof(ZT));
#pragma unroll
    for (int p = 0; p < ZP; ++p) {
      const bool in = j * 32 + EPP * p < vleft;
      const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(
          zrs, (int)(in ? off + (uint32_t)(j * 32 * (int)sizeof(ZT) + 16 * p) : a.z_bytes), 0, 0);
      zj[p] = make_uint4(x[0], x[1], x[2], x[3]);
    }
  };
  auto zload = [&](int kk, int nt, uint4 (&z)[kPMt][ZP]) {
#pragma unroll
    for (int j = 0; j < kPMt; ++j) zload_one(kk, nt, j, z[j]);
  };
  // entry e (0..15) of M-tile j from its pieces, -inf past V
  auto zval = [&](int j, const uint4 (&zj)[ZP], int e) -> float {
    const int p = e / EPP;
    if (kF32) return __uint_as_float(u4get(zj[p], e & 3) | (j * 32 + EPP * p < vleft ? 0u : 0xFF800000u));
    const uint32_t w = u4get(zj[p], (e >> 1) & 3) | (j * 32 + EPP * p < vleft ? 0u : 0xFF80FF80u);
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  };
  // E rows of N-tile nt's previous tokens into dst, by LDS DMA: instruction q
  // fills slots 64q .. 64q + 63, lane i slot 64q + i (a padding slot loads
  // piece 0; lanes past the last slot are off)
  // (the instruction index passes through an empty asm statement so that the
  // slot and destination arithmetic stays where the request is issued: hoisted
  // out of the N-tile loop it would hold registers per stage)
  auto gather_one = [&](int nt, unsigned char* dst, int q) {
    int qs = __builtin_amdgcn_readfirstlane(q);
    __asm__ volatile("" : "+s"(qs));
    const int sl = qs * 64 + lane;
    const int row = sl / RS, piece = sl - row * RS;
    if (sl < NSLOT)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ers, (__attribute__((address_space(3))) void*)(dst + qs * 1024), 16,
          (int)((uint32_t)s_tok[nt * 32 + row] * ROWB + (uint32_t)(piece < PR ? piece : 0) * 16), 0, 0, 0);
  };
  auto gather = [&](int nt, unsigned char* dst) {
    for (int q = wave; q * 64 < NSLOT; q += kPWaves) gather_one(nt, dst, q);
  };
  // per-row merge of the M-tile partials of N-tiles 4*half .. 4*half+3:
  // chunk log-masses, chunk Gumbels, best chunk, running log-partition, as one
  // record per (row, workgroup) stored past the L2.  Two threads per row: the
  // workgroup's at most five consecutive chunks span at most two Philox quads,
  // and thread p takes the chunks of quad (c_begin / 4) + p (one draw each);
  // the pair then combines over a lane swap.  Sums are taken against the
  // maximum, so every exponent is at most 0 (the hardware exp2).
  auto merge = [&](int k, int half) {
    barrier_lds_only();
    const int r = tid >> 1, p = tid & 1;
    const int prow = half * kPHalf + r;
    const int qd = (c_begin >> 2) + p;
    const int cb = c_begin > 4 * qd ? c_begin : 4 * qd;
    const int ce = c_end < 4 * qd + 4 ? c_end : 4 * qd + 4;
    float rm = -INFINITY, rs = 0.f, best = -INFINITY;
    int best_c = 0x7fffffff;
    if (prow < B && cb < ce) {
      // (the counter words pass through an empty asm statement: the draw's
      // arithmetic that does not depend on the position would otherwise be
      // hoisted out of the position loop, where its registers spill)
      int prow_v = prow, quad_v = qd * 4;
      __asm__ volatile("" : "+v"(prow_v), "+v"(quad_v));
      const Words4 w4 = draw_quad(a.key, (uint32_t)quad_v, (uint32_t)prow_v, (uint32_t)k, kDraftChunk);
      for (int c = cb; c < ce; ++c) {
        {
          const float2* pt = &s_tp[r * kPMtWg + 4 * (c - c_begin)];
          const float2 p0 = pt[0], p1 = pt[1], p2 = pt[2], p3 = pt[3];
          const float m = fmaxf(fmaxf(p0.x, p1.x), fmaxf(p2.x, p3.x));
          const float o = m == -INFINITY ? 0.f : m;
          const float sm = p0.y * __builtin_amdgcn_exp2f(p0.x - o) + p1.y * __builtin_amdgcn_exp2f(p1.x - o) +
                           p2.y * __builtin_amdgcn_exp2f(p2.x - o) + p3.y * __builtin_amdgcn_exp2f(p3.x - o);
          const float gc = gumbel_from_word(quad_pick(w4, c & 3));
          const float score = sm > 0.f ? (m + __builtin_amdgcn_logf(sm)) * kLn2 + gc : -INFINITY;
          if (score > best) {
            best = score;
            best_c = c;
          }
          // running log-partition (base 2), online
          const float mm = fmaxf(rm, m);
          const float mo = mm == -INFINITY ? 0.f : mm;
          rs = rs * __builtin_amdgcn_exp2f(rm - mo) + sm * __builtin_amdgcn_exp2f(m - mo);
          rm = mm;
        }
      }
    }
    // the partner's (quad q0 + 1 - p) results
    const float om = dpp_f<kDppXor1>(rm), os = dpp_f<kDppXor1>(rs), ob = dpp_f<kDppXor1>(best);
    const int oc = dpp_i<kDppXor1>(best_c);
    if (p == 0 && prow < B) {
      const float mm = fmaxf(rm, om);
      const float mo = mm == -INFINITY ? 0.f : mm;
      const float ss = rs * __builtin_amdgcn_exp2f(rm - mo) + os * __builtin_amdgcn_exp2f(om - mo);
      if (better(ob, oc, best, best_c)) {
        best = ob;
        best_c = oc;
      }
      unsigned long long* rp = a.rec + ((size_t)prow * G + g) * 4;
      const uint32_t tg = tag_of(k);
      st_tagged(rp + 0, __float_as_uint(mm), tg);
      st_tagged(rp + 1, __float_as_uint(ss), tg);
      st_tagged(rp + 2, __float_as_uint(best), tg);
      st_tagged(rp + 3, (uint32_t)best_c, tg);
    }
    barrier_lds_only();
  };
  // the reduction of one (N-tile, M-tile) accumulator (the logits: the
  // chain started from the base logits): (max, sum of 2^(x - max)) in base 2
  // into LDS
  auto epilogue = [&](int nt, int j, const f32x16_t& acc) {
    float ell[16];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ell[2 * i] = acc[2 * i];
      ell[2 * i + 1] = acc[2 * i + 1];
      m = fmaxf(m, fmaxf(ell[2 * i], ell[2 * i + 1]));
    }
    m = halves32_max(m);
    const float off = m == -INFINITY ? 0.f : -m * scale2;
    float sm = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sm += __builtin_amdgcn_exp2f(fmaf(ell[i], scale2, off));
    sm = halves32_sum(sm);
    // both halves of the column hold the same pair: a duplicate store of equal values
    s_tp[((nt & 3) * 32 + l32) * kPMtWg + wave * kPMt + j] = make_float2(m * scale2, sm);
  };
  // N-tile nt of position k: its E rows are in cur and its base logits in
  // zc; the next N-tile's rows (into nxt; bf16: gather instruction wave + 4j in
  // stage j; fp32: all at the start, ahead of every refill, which the
  // end-of-tile wait counts on) and its base logits are requested one M-tile
  // per stage (bf16: into zn; fp32: into zc, each M-tile's as
  // soon as its stage has taken them into the accumulator, always issued) well
  // ahead of their use.
  // Requesting all of them at once would stall the wave at issue while the
  // earlier requests drain at the workgroup's share of the memory bandwidth.
  auto tile = [&](int k, int nt, uint4 (&zc)[kPMt][ZP], uint4 (&zn)[kPMt][ZP], const unsigned char* cur,
                  unsigned char* nxt) {
    const bool more = nt + 1 < NT;
    if (kF32 && more) gather(nt + 1, nxt);
    const unsigned char* brow = cur + (l32 * RS + h) * 16;
    auto bfrag = [&](int t) { return *reinterpret_cast<const bf16x8_t*>(brow + 32 * t); };
    // Every M-tile is computed (a missing one has zero fragments and its
    // result is never read).  Stage j chains M-tile j's 16 MFMAs from its base
    // logits (so the chain ends at the logits; entries past V start at -inf),
    // its LDS fragments read D K-steps ahead, and gives each K-step a fixed
    // slice of M-tile j-1's epilogue: steps 0-7 the maximum, step 8 merges the
    // column halves, steps 9-15 the exponentials and sums.  Scheduling barriers
    // keep the slices where they are written.
    auto stage = [&](int j, int pj, const f32x16_t& pacc) {
      f32x16_t acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = zval(j, zc[j], i);
      constexpr int D = kF32 ? 2 : 3;  // fp32: a shorter ring leaves the registers the refills need
      bf16x8_t bq[D + 1], aq[D + 1];
#pragma unroll
      for (int t = 0; t < D; ++t) {
        bq[t] = bfrag(t);
        if (j >= JR) aq[t] = s_a[wave][t][lane];
      }
      float ell[16], m = -INFINITY, off = 0.f, s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int t = 0; t < S; ++t) {
        if (t + D < S) {
          bq[(t + D) % (D + 1)] = bfrag(t + D);
          if (j >= JR) aq[(t + D) % (D + 1)] = s_a[wave][t + D][lane];
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(j < JR ? af[j < JR ? j : 0][t] : aq[t % (D + 1)],
                                                      bq[t % (D + 1)], acc, 0, 0, 0);
        if (pj >= 0) {
          if (t < 8) {
            ell[2 * t] = pacc[2 * t];
            ell[2 * t + 1] = pacc[2 * t + 1];
            m = fmaxf(m, fmaxf(ell[2 * t], ell[2 * t + 1]));
          } else if (t == 8) {
            m = halves32_max(m);
            off = m == -INFINITY ? 0.f : -m * scale2;
          } else {
            // steps 9..14 two entries each, step 15 the last four
            const int e0 = 2 * (t - 9), e1 = t == 15 ? 16 : e0 + 2;
#pragma unroll
            for (int e = e0; e < e1; ++e) {
              const float x = __builtin_amdgcn_exp2f(fmaf(ell[e], scale2, off));
              if (e & 1)
                s1 += x;
              else
                s0 += x;
            }
          }
        }
        // the next N-tile's base logits of M-tile j (fp32: in place, read by the
        // accumulator's start above)
        if (!kF32 && t == 1 && more && (wave + kPWaves * j) * 64 < NSLOT) gather_one(nt + 1, nxt, wave + kPWaves * j);
        if (t == 2 && (kF32 || more)) zload_one(k, nt + 1, j, kF32 ? zc[j] : zn[j]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (pj >= 0) {
        const float sm = halves32_sum(s0 + s1);
        // both halves of the column hold the same pair: a duplicate store of equal values
        s_tp[((nt & 3) * 32 + l32) * kPMtWg + wave * kPMt + pj] = make_float2(m * scale2, sm);
      }
      return acc;
    };
    const f32x16_t zero = {};
    f32x16_t a0 = stage(0, -1, zero);
    f32x16_t a1 = stage(1, 0, a0);
    a0 = stage(2, 1, a1);
    a1 = stage(3, 2, a0);
    a0 = stage(4, 3, a1);
    epilogue(nt, 4, a0);
    // this wave's gather of N-tile nt + 1 is complete (bf16: and the base
    // logits loaded with it; fp32: the kPMt * ZP refills, all issued after the
    // gather, may still be in flight); after the barrier every wave's rows are
    // in and no wave reads cur any more
    if (kF32) {
      wait_vmem_n<kPMt * ZP>();
    } else {
      wait_vmem();
    }
    barrier_lds_only();
    if ((nt & 3) == 3 || !more) merge(k, nt >> 2);
  };

  uint4 zA[kPMt][ZP], zB[kPMt][kF32 ? 1 : ZP];
  zload(1, 0, zA);

  for (int k = 1; k <= K; ++k) {
    // 1. the previous tokens of all 256 rows (rows past B: token 0): the
    // anchors, or this group's replica of the tokens of position k - 1 as each
    // arrives (the wait for the previous position); then the E rows of N-tile 0
    {
      int x = 0;
      if (tid < B) {
        if (k == 1) {
          x = a.anchor[tid];
        } else {
          uint32_t v[1];
          poll_tagged<1>(a.tokrep + (size_t)(g % ng) * kTokRepSlots + tid, expect_of(k - 1), flag, a.spin_limit, v);
          x = (int)v[0];
        }
      }
      s_tok[tid] = clamp_id(x, V);
    }
    __syncthreads();
    gather(0, s_b0);
    wait_vmem();
    __syncthreads();

    // 2-3. the vocabulary stream, N-tile after N-tile (bf16: base-logit
    // registers alternating between zA and zB; fp32: zA refilled in place)
    for (int nt = 0; nt < NT; nt += 2) {
      if constexpr (kF32) {
        tile(k, nt, zA, zA, s_b0, s_b1);
        if (nt + 1 < NT) tile(k, nt + 1, zA, zA, s_b1, s_b0);
      } else {
        tile(k, nt, zA, zB, s_b0, s_b1);
        if (nt + 1 < NT) tile(k, nt + 1, zB, zA, s_b1, s_b0);
      }
    }

    // 4-5. selection of rows g, g + G, ...: thread t < G waits for workgroup
    // t's record of the row (its tags name position k)
    for (int b = g; b < B; b += G) {
      const int c = tid % PR, grp = tid / PR;
      float4 p = make_float4(-INFINITY, 0.f, -INFINITY, 0.f);
      if (tid < G) {
        uint32_t v[4];
        poll_tagged<4>(a.rec + ((size_t)b * G + tid) * 4, expect_of(k), flag, a.spin_limit, v);
        p = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
      }
      // the winning chunk: argmax of the chunk scores, smallest chunk id on ties
      float best = -INFINITY;
      int bc = 0x7fffffff;
      if (tid < G && better(p.z, __float_as_int(p.w), best, bc)) {
        best = p.z;
        bc = __float_as_int(p.w);
      }
      wave_argmax(best, bc);
      float lm = -INFINITY, ls = 0.f;
      if (tid < G) lse2_merge(lm, ls, p.x, p.y);
      wave_lse2_merge(lm, ls);
      if (lane == 0) {
        s_best[wave] = best;
        s_bi[wave] = bc;
        s_bm[wave] = lm;
        s_bs[wave] = ls;
      }
      __syncthreads();
      float B0 = s_best[0];
      int C0 = s_bi[0];
      for (int w = 1; w < kPWaves; ++w)
        if (better(s_best[w], s_bi[w], B0, C0)) {
          B0 = s_best[w];
          C0 = s_bi[w];
        }
      // a row without any finite chunk score keeps the sentinel id: chunk 0
      // (compared with the chunk count: C0 * kChunk could wrap)
      const int cstar = (C0 >= 0 && C0 < a.nchunks) ? C0 : 0;
      const int v0 = cstar * kChunk;
      const int nrow = V - v0 < kChunk ? V - v0 : kChunk;
      // the chunk's Wt block (consecutive threads on consecutive 16-byte
      // pieces), this thread's piece of E[prev], the entry's base logit and Gumbel
      const uint16_t* blk = Wt + (size_t)v0 * R;
      uint4 w[NP];
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int rr = i * RG + grp;
        w[i] = *reinterpret_cast<const uint4*>(blk + (size_t)(rr < nrow ? rr : 0) * R + 8 * c);
      }
      const uint4 ep = *reinterpret_cast<const uint4*>(E + (size_t)s_tok[b] * R + 8 * c);
      const int r = tid & (kChunk - 1);
      const int v = v0 + r;
      const bool inside = tid < kChunk && r < nrow;
      const ZT zraw = Z[((size_t)b * K + (k - 1)) * V + (r < nrow ? v : v0)];
      const float zb = kF32 ? (float)zraw : bf16_to_f32((uint16_t)zraw);
      const float gum = gumbel_from_word(draw_word(a.key, (uint32_t)v, (uint32_t)b, (uint32_t)k, kDraftElem));
      __syncthreads();  // s_tp is reused for the dot partials
      float* s_part = reinterpret_cast<float*>(s_tp);
#pragma unroll
      for (int i = 0; i < NP; ++i) s_part[(i * RG + grp) * STR + c] = dot_bf16x8(ep, w[i]);
      __syncthreads();
      float score = -INFINITY;
      int idx = 0x7fffffff;
      if (inside) {
        float dot = 0.f;
        const float4* q4 = reinterpret_cast<const float4*>(s_part + r * STR);
#pragma unroll
        for (int j = 0; j < PR / 4; ++j) {
          const float4 x = q4[j];
          dot += x.x;
          dot += x.y;
          dot += x.z;
          dot += x.w;
        }
        const float ell = (zb + dot) * a.inv_T;
        s_ell[r] = ell;
        score = ell + gum;
        idx = v;
      }
      wave_argmax(score, idx);
      __syncthreads();  // every wave's LDS reads of the maxima above are done
      if (lane == 0) {
        s_best[wave] = score;
        s_bi[wave] = idx;
      }
      __syncthreads();
      if (tid == 0) {
        float B1 = s_best[0];
        int X = s_bi[0];
        for (int ww = 1; ww < kPWaves; ++ww)
          if (better(s_best[ww], s_bi[ww], B1, X)) {
            B1 = s_best[ww];
            X = s_bi[ww];
          }
        float M = s_bm[0], Sm = s_bs[0];
        for (int ww = 1; ww < kPWaves; ++ww) lse2_merge(M, Sm, s_bm[ww], s_bs[ww]);
        const float lse = (M + log2f(Sm)) * kLn2;
        if (X < v0 || X >= v0 + kChunk || X >= V) X = v0;  // no finite score
        const size_t o = (size_t)b * K + (k - 1);
        a.tok[o] = X;
        a.logq[o] = s_ell[X - v0] - lse;
        a.lse[o] = lse;
        s_x = X;
      }
      __syncthreads();
      // the token, tagged, into every group's replica
      if (tid < ng) st_tagged(a.tokrep + (size_t)tid * kTokRepSlots + b, (uint32_t)s_x, tag_of(k));
      __syncthreads();
    }

    // 6. the next position's first base logits (they do not depend on the
    // tokens), in flight while its tokens are awaited
    if (k < K) zload(k + 1, 0, zA);
  }
}

// Before each launch: clear the time-out flag, advance the launch generation
// (every tag of the launch carries it) and clear every record and token word
// (a cleared word's tag, 0, is no position's), so that no word left by an
// earlier launch, or by other data in a reused workspace, satisfies a wait.
__global__ __launch_bounds__(256) void k_persist_init(unsigned* sync, unsigned long long* rec, int n_rec,
                                                      unsigned long long* tokrep, int n_tok) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0) {
    sync[kSyncFlag * kSyncStride] = 0u;
    sync[kSyncGen * kSyncStride] += 1u;
  }
  for (int j = i; j < n_rec; j += gridDim.x * 256) rec[j] = 0ull;
  for (int j = i; j < n_tok; j += gridDim.x * 256) tokrep[j] = 0ull;
}

}  // namespace

int persist_grid(int V) {
  const int nc = n_chunks(V);
  return nc < kStreamGridMax ? nc : kStreamGridMax;
}

bool draft_persistent_supported(const dspark_problem& P) {
  if ((P.logits_dtype != DSPARK_BF16 && P.logits_dtype != DSPARK_F32) || P.weight_dtype != DSPARK_BF16 ||
      P.r != 256 || P.B > kPRows)
    return false;
  const size_t zsize = P.logits_dtype == DSPARK_F32 ? 4 : 2;
  if ((size_t)P.B * P.K * P.V * zsize > 0xFFFFFFFFull || (size_t)P.V * 512 > 0xFFFFFFFFull) return false;  // 32-bit buffer offsets
  const int nc = n_chunks(P.V);
  const int G = persist_grid(P.V);
  if ((nc + G - 1) / G > kPMtWg / 4) return false;
  static int capable = -1;  // whether one workgroup per CU fits and the device launches cooperatively
  if (capable < 0) {
    int dev = 0, coop = 0, ncu = 0, per_cu16 = 0, per_cu32 = 0;
    capable = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu16, reinterpret_cast<const void*>(k_draft_persist<256, uint16_t>), kPThreads, 0) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu32, reinterpret_cast<const void*>(k_draft_persist<256, float>), kPThreads, 0) == hipSuccess)
      capable = coop && per_cu16 >= 1 && per_cu32 >= 1 && ncu >= kStreamGridMax ? 1 : 0;
    (void)hipGetLastError();
  }
  return capable == 1;
}

hipError_t launch_draft_persistent(const dspark_problem& P, const PersistArgs& a, hipStream_t s) {
  const int n_rec = P.B * persist_grid(P.V) * 4;  // B <= 256: at most 256 x 256 x 4 words
  const int n_tok = kSyncGroups * kTokRepSlots;
  const int blocks = (n_rec + 256 * 8 - 1) / (256 * 8);  // about 8 words per thread
  hipLaunchKernelGGL(k_persist_init, blocks, 256, 0, s, a.sync, a.rec, n_rec, a.tokrep, n_tok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PersistArgs arg = a;
  void* args[] = {&arg};
  const void* kernel = P.logits_dtype == DSPARK_F32 ? reinterpret_cast<const void*>(k_draft_persist<256, float>)
                                                    : reinterpret_cast<const void*>(k_draft_persist<256, uint16_t>);
  return hipLaunchCooperativeKernel(kernel, dim3(persist_grid(P.V)), dim3(kPThreads), args, 0, s);
}

}  // namespace dspark
