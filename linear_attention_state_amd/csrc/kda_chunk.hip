// kda_chunk.hip -- chunked prefill of Kimi delta attention (KDA) on gfx950 MFMA.
//
// Recurrence (Kimi Linear technical report, 2025; the tracker page "Continuous
// batching: model support tracker" lists KDA among the layers whose per-request
// states the cache holds), per sequence and value head, state S [d_k][d_v]:
//     S_t = (I - b_t k_t k_t^T) diag(a_t) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t,
// with a_t = exp(g_t) one decay per key channel.  In delta form
// S_t = diag(a_t) S_{t-1} + k_t u_t^T, u_t = b_t (v_t - (diag(a_t) S_{t-1})^T k_t).
// Over a chunk of 64 rows, with gamma_t = sum_{s<=t} g_s per channel (<= 0 and
// non-increasing) and S the state entering the chunk, unrolling gives the WY / UT
// form with the decay inside the channel sums:
//     A_tj = b_t sum_c k_t[c] k_j[c] e^{gamma_t[c]-gamma_j[c]}   (j < t),  T = (I + A)^-1
//     U    = T diag(b) (V - Kt S),                 Kt_t = e^{gamma_t} o k_t
//     O    = Qt S + P U,  P_tj = sum_c q_t[c] k_j[c] e^{gamma_t[c]-gamma_j[c]} (j <= t),  Qt_t = e^{gamma_t} o q_t
//     S   <- diag(e^{gamma_last}) S + Kh^T U,      Kh_t = e^{gamma_last - gamma_t} o k_t
// (with a decay equal on every channel this is the gated delta rule's chunk form).
//
// The channel sums of A and P are dense products of 16 x 16 blocks.  For a block
// pair (bi, bj), bi > bj, the decay splits at the end e = 16 bj + 15 of block bj
// and at the row 16 bi - 1 before block bi, so that no factor exceeds 1:
//     e^{gamma_t - gamma_j} = e^{gamma_t - gamma_{16bi-1}} e^{gamma_{16bi-1} - gamma_e} e^{gamma_e - gamma_j}
// i.e. rows of block bi of Kb = e^{gamma_t - gamma_{16bi-1}} o k (A side), rows of
// block bj of Kr = e^{gamma_e - gamma_j} o k (B side), times a channel factor for
// pairs two or more blocks apart.  On a diagonal block the B side is Kr times
// e^{gamma_{16b-1} - gamma_{16b+15}} >= 1, the block's own decay: bounded by the
// decay over 16 rows, and computed exactly in fp32 instead (exact_diag) for a
// block where that factor would leave the range of fp32.  Only differences of
// running sums are exponentiated.
//
// Work split: one 512-thread workgroup (8 waves) per (sequence, value head),
// chunk by chunk in three phases separated by workgroup barriers:
//   1. all waves: thread (block b, channel c) loads its 16 rows of q, k, v (the
//      conv output, normalised) and g, forms gamma within the block and across
//      the blocks, and writes the decay-scaled tiles Kb, Qb, Kr, Kt, Qt, Kh and V;
//   2. all waves: the ten A blocks and ten P blocks (MFMA), then T = (I + A)^-1
//      (diagonal blocks by fp32 forward substitution, the others by block
//      products) written as T2^T = (T diag(b))^T;
//   3. waves 0-3: wave w owns d_v columns [32w, 32w+32) of the fp32 state in
//      registers and computes Kt S, U = T2 (V - Kt S), (Qt S)^T, O^T and the
//      state update (each state row scaled by its channel's e^{gamma_last}).
// All products are v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulate).
#include "gdn_device.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int KNT = 512;            // threads per workgroup
constexpr int KNS = 4;              // state waves
constexpr int KNB = D / 16 / KNS;   // 16-column tiles per state wave
constexpr int KPS = D + 4;          // fp32 pitch of the state staged in LDS
// a diagonal block whose own decay exceeds this (natural log) on some channel
// is computed in fp32 (its B-side growth factor would pass e^kMaxGrowth)
constexpr float kMaxGrowth = 80.f;

// LDS.  The [64][128] bf16 tiles use the swizzled row-major layout of swz_off.
struct alignas(16) KSmem {
  uint16_t kb[BT * D];   // e^{gamma_t - gamma_{16b-1}} o k_t: A side of the A blocks (t in block b)
  uint16_t qb[BT * D];   // e^{gamma_t - gamma_{16b-1}} o q_t: A side of the P blocks
  uint16_t kr[BT * D];   // e^{gamma_{16b+15} - gamma_t} o k_t: B side of the A and P blocks
  uint16_t kt[BT * D];   // e^{gamma_t} o k_t: K S
  uint16_t qt[BT * D];   // e^{gamma_t} o q_t: Q S
  uint16_t kh[BT * D];   // e^{gamma_last - gamma_t} o k_t: the state update
  uint16_t v[BT * D];
  uint16_t p[BT * PP];         // P [t][j in pair order]; blocks above the diagonal stay zero
  uint16_t t2[11][16 * PB];    // (T diag(b))^T as 16 x 16 blocks, and the zero block (slot 10)
  uint16_t ab[6][16 * PB];     // A^T blocks below the diagonal
  uint16_t tb[5][16 * PB];     // T^T blocks 00, 11, 22, 33 and 32
  float at[4 * 16 * PA];       // diagonal blocks of A, fp32, [block][j][t]
  float beta[BT];
  float btot[4][D];            // per block and channel: the sum of g over its rows (<= 0)
  float fac[7][D];             // B-side channel factors: pairs (2,0), (3,1), (3,0); diagonal blocks 0..3
  float glast[D];              // e^{gamma_last} per channel
  float gex[16 * D];           // exact_diag: gamma within the block, per row and channel
  int diag_exact;              // bit b: diagonal block b computed in fp32
};
static_assert(sizeof(KSmem) <= 160 * 1024, "LDS");
static_assert(D * KPS * 4 <= 5 * BT * D * 2, "state staging fits the first five tiles");

struct KSeq {
  int s, r0, L, N, m, h;
};

// B-side factor slot of block pair (bi, bj), bi >= bj: -1 none, 0..2 the pairs two
// or more blocks apart, 3 + b the diagonal block b
__device__ __forceinline__ constexpr int fac_slot(int bi, int bj) {
  return bi == bj ? 3 + bi : bi - bj == 1 ? -1 : (bi == 2 ? 0 : bj == 1 ? 1 : 2);
}

// A row operand (16 rows, 8 channels per lane) of a tile, scaled per channel by
// a factor vector and rounded back to bf16.
__device__ __forceinline__ bf16x8 scaled8(bf16x8 x, const float* f) {
  const f32x4 f0 = *reinterpret_cast<const f32x4*>(f);
  const f32x4 f1 = *reinterpret_cast<const f32x4*>(f + 4);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (__bf16)((float)x[e] * f0[e]);
    r[4 + e] = (__bf16)((float)x[4 + e] * f1[e]);
  }
  return r;
}

// ---- phase 1: the decay-scaled tiles of chunk c, by the 256 producer threads:
// thread (bp, c) owns channel c of the 32 rows of blocks 2bp and 2bp+1; rows past
// the sequence's end are zero with g = 0 and b = 0, so they change nothing.
// Pass 1 (before the barrier the caller places): each block's total decay.
__device__ __forceinline__ void kda_totals(KSmem& sm, const ScanArgs& a, const KSeq& q, int chunk, int tp) {
  const int bp = tp >> 7, ch = tp & 127, Hv = a.num_v_heads;
#pragma unroll 1
  for (int hb = 0; hb < 2; ++hb) {
    const int b = 2 * bp + hb;
    const int64_t rb = (int64_t)q.r0 + chunk * BT + 16 * b;
    const int nv = max(0, min(16, q.L - chunk * BT - 16 * b));
    const float* gp = a.g + ((rb * Hv + q.m) * D + ch);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += i < nv ? gp[i * (int64_t)Hv * D] : 0.f;
    sm.btot[b][ch] = acc;
    if (-acc > kMaxGrowth) atomicOr(&sm.diag_exact, 1 << b);
  }
  if (tp < BT) {
    const int t = tp, in = chunk * BT + t < q.L;
    sm.beta[t] = in ? a.beta[((int64_t)q.r0 + chunk * BT + t) * Hv + q.m] : 0.f;
  }
}

// Pass 2 (after it): the tiles, four rows at a time (g read again, now from the caches).
__device__ __forceinline__ void kda_tiles(KSmem& sm, const ScanArgs& a, const KSeq& q, int chunk, int tp) {
  const int bp = tp >> 7, ch = tp & 127;
  const int Hv = a.num_v_heads, C = a.channels, Hk = a.num_k_heads;
  const uint16_t* y = reinterpret_cast<const uint16_t*>(a.y);
  float tot[4], glast = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    tot[j] = sm.btot[j][ch];
    glast += tot[j];
  }
  // rows are walked with rolled loops: unrolled, their addresses (hoisted out of
  // the chunk loop) would not fit the registers
#pragma unroll 1
  for (int hb = 0; hb < 2; ++hb) {
    const int b = 2 * bp + hb;
    const int64_t rb = (int64_t)q.r0 + chunk * BT + 16 * b;
    const int nv = max(0, min(16, q.L - chunk * BT - 16 * b));
    const float acc = tot[b];
    const float off = b == 0 ? 0.f : b == 1 ? tot[0] : b == 2 ? tot[0] + tot[1] : tot[0] + tot[1] + tot[2];
    const float* gp = a.g + ((rb * Hv + q.m) * D + ch);
    const uint16_t* kp = y + rb * C + (int64_t)Hk * D + q.h * D + ch;
    const uint16_t* qp = y + rb * C + (int64_t)q.h * D + ch;
    const uint16_t* vp = y + rb * C + 2 * (int64_t)Hk * D + (int64_t)q.m * D + ch;
    float gl = 0.f;
#pragma unroll 1
    for (int i0 = 0; i0 < 16; i0 += 4) {
      float g[4], k[4], qq[4], v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        const bool in = i < nv;
        const int64_t ro = in ? i : 0;  // a clamped row for the loads past the end
        g[e] = gp[ro * (int64_t)Hv * D];
        k[e] = bf16_bits_to_f32(kp[ro * C]);
        qq[e] = bf16_bits_to_f32(qp[ro * C]);
        v[e] = bf16_bits_to_f32(vp[ro * C]);
        if (!in) g[e] = k[e] = qq[e] = v[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gl += g[e];
        const int o = swz_off(16 * b + i0 + e, ch);
        const float e1 = __expf(gl);                 // e^{gamma_t - gamma_{16b-1}}
        const float e2 = __expf(acc - gl);           // e^{gamma_{16b+15} - gamma_t}
        const float e3 = __expf(off + gl);           // e^{gamma_t}
        const float e4 = __expf(glast - off - gl);   // e^{gamma_last - gamma_t}
        sm.kb[o] = f32_to_bf16_bits(k[e] * e1);
        sm.qb[o] = f32_to_bf16_bits(qq[e] * e1);
        sm.kr[o] = f32_to_bf16_bits(k[e] * e2);
        sm.kt[o] = f32_to_bf16_bits(k[e] * e3);
        sm.qt[o] = f32_to_bf16_bits(qq[e] * e3);
        sm.kh[o] = f32_to_bf16_bits(k[e] * e4);
        sm.v[o] = f32_to_bf16_bits(v[e]);
      }
    }
    // diagonal block b: e^{-(sum of g over the block)} >= 1, kept finite (a block
    // past the bound is computed exactly instead)
    sm.fac[3 + b][ch] = __expf(fminf(-acc, kMaxGrowth));
  }
  if (bp == 0) {
    sm.fac[0][ch] = __expf(tot[1]);           // pair (2,0): e^{gamma_31 - gamma_15}
    sm.fac[1][ch] = __expf(tot[2]);           // pair (3,1): e^{gamma_47 - gamma_31}
    sm.fac[2][ch] = __expf(tot[1] + tot[2]);  // pair (3,0): e^{gamma_47 - gamma_15}
    sm.glast[ch] = __expf(glast);
  }
}

// ---- phase 2a: A and P blocks.  Producer wave w (0..3): row block bi = w of A
// and of P; both share the B-side operands of the blocks bj <= bi.
__device__ __forceinline__ void kda_blocks(KSmem& sm, int bi, const Lane& ln) {
  int roff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) roff[kk] = swz_off(ln.r, 32 * kk + 8 * ln.g);
  for (int bj = 0; bj <= bi; ++bj) {
    const int fs = fac_slot(bi, bj);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, pacc = acc;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 yr = lds8(sm.kr + roff[kk] + 16 * bj * D);
      if (fs >= 0) yr = scaled8(yr, &sm.fac[fs][32 * kk + 8 * ln.g]);
      const bf16x8 ka = lds8(sm.kb + roff[kk] + 16 * bi * D);
      const bf16x8 qa = lds8(sm.qb + roff[kk] + 16 * bi * D);
      // A: lane holds A[16bi + 4g + i][16bj + r]; P transposed: P[16bi + r][16bj + 4g + i]
      acc = mfma(ka, yr, acc);
      pacc = mfma(yr, qa, pacc);
    }
    {
      const int j = 16 * bj + ln.r;
      const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[16 * bi + 4 * ln.g]);
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (j < 16 * bi + 4 * ln.g + i) ? bt[i] * acc[i] : 0.f;
      if (bi == bj)
        *reinterpret_cast<float4*>(&sm.at[(16 * bi + ln.r) * PA + 4 * ln.g]) = make_float4(v[0], v[1], v[2], v[3]);
      else
        st4bf(&sm.ab[low_slot(bi, bj)][ln.r * PB + 4 * ln.g], v[0], v[1], v[2], v[3]);
    }
    {
      // lane holds P[t = 16bi + r][j = 16bj + 4g + i]
      const int t = 16 * bi + ln.r;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (16 * bj + 4 * ln.g + i <= t) ? pacc[i] : 0.f;
      st4bf(&sm.p[t * PP + perm(16 * bj + 4 * ln.g)], v[0], v[1], v[2], v[3]);
    }
  }
}

// ---- phase 2b (only for a diagonal block whose own decay leaves the fp32 range):
// its A and P entries from the channel sums themselves, with every
// e^{gamma_t - gamma_j} formed from the difference of running sums (<= 0).  All
// threads; block b's gamma (relative to the row before it) is first put in gex.
__device__ void exact_diag(KSmem& sm, const ScanArgs& a, const KSeq& q, int chunk, int b, int tid) {
  const int Hv = a.num_v_heads, C = a.channels, Hk = a.num_k_heads;
  const int64_t rb = (int64_t)q.r0 + chunk * BT + 16 * b;
  const int nv = max(0, min(16, q.L - chunk * BT - 16 * b));
  const uint16_t* y = reinterpret_cast<const uint16_t*>(a.y);
  if (tid < D) {
    float acc = 0.f;
    for (int i = 0; i < 16; ++i) {
      if (i < nv) acc += a.g[((rb + i) * Hv + q.m) * D + tid];
      sm.gex[i * D + tid] = acc;
    }
  }
  __syncthreads();  // (every wave of the workgroup meets it: see the main loop)
  // 136 pairs (j <= t) x 4 channel quarters; the quarters of a pair are adjacent lanes
  for (int w = tid; w < 136 * 4; w += KNT / 2) {
    const int pr = w >> 2, qd = w & 3;
    int t = 0, rem = pr;  // pair index -> (t, j), j <= t
    while (rem > t) { rem -= t + 1; ++t; }
    const int j = rem;
    float sa = 0.f, sp = 0.f;
    if (t < nv && j < nv) {
      for (int c = 32 * qd; c < 32 * qd + 32; ++c) {
        const float kt = bf16_bits_to_f32(y[(rb + t) * C + (int64_t)Hk * D + q.h * D + c]);
        const float kj = bf16_bits_to_f32(y[(rb + j) * C + (int64_t)Hk * D + q.h * D + c]);
        const float qt = bf16_bits_to_f32(y[(rb + t) * C + (int64_t)q.h * D + c]);
        const float e = __expf(sm.gex[t * D + c] - sm.gex[j * D + c]);
        sa = fmaf(kt * kj, e, sa);
        sp = fmaf(qt * kj, e, sp);
      }
    }
    sa += __shfl_xor(sa, 1);
    sa += __shfl_xor(sa, 2);
    sp += __shfl_xor(sp, 1);
    sp += __shfl_xor(sp, 2);
    if (qd == 0) {
      const int tt = 16 * b + t, jj = 16 * b + j;
      if (j < t) sm.at[(16 * b + j) * PA + t] = sm.beta[tt] * sa;
      sm.p[tt * PP + perm(jj)] = f32_to_bf16_bits(sp);
    }
  }
}

// ---- phase 3: the state pass of one chunk for d_v columns [32 wv, 32 wv + 32)
// (the arithmetic of the gated-delta-rule state pass with the decays in the tiles).
struct StateLanes {
  int roff[4], toff[4][2], voffs[KNB], col[KNB], t2off, poff, olane;
};

__device__ __forceinline__ void kda_state_step(KSmem& sm, f32x4 (&sacc)[8][KNB], const StateLanes& sl,
                                               const ScanArgs& a, const KSeq& q, int chunk, const Lane& ln) {
  const int lg = ln.g;
  // ---- Kt S (rows t, columns n)
  f32x4 ks[4][KNB];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) ks[tb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // operands of step kk + 1 are read during the products of step kk (the
  // scheduling fences keep the compiler from hoisting every step's reads)
  bf16x8 ka[2][4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) ka[0][tb] = lds8(sm.kt + sl.roff[0] + 16 * tb * D);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int cur = kk & 1;
    fence();
    if (kk < 3) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) ka[cur ^ 1][tb] = lds8(sm.kt + sl.roff[kk + 1] + 16 * tb * D);
    }
    fence();
    bf16x8 sb[KNB];
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) sb[nb] = pair_operand(sacc[2 * kk][nb], sacc[2 * kk + 1][nb]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int nb = 0; nb < KNB; ++nb) ks[tb][nb] = mfma(ka[cur][tb], sb[nb], ks[tb][nb]);
  }
  fence();
  // ---- X = V - Kt S (in place of Kt S),  U = T2 X
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) {
      const bf16x4 vv = ldtr(sm.v + sl.voffs[nb] + 16 * tb * D);
#pragma unroll
      for (int i = 0; i < 4; ++i) ks[tb][nb][i] = (float)vv[i] - ks[tb][nb][i];
    }
  f32x4 u[4][KNB];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) u[tb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    bf16x8 xb[KNB];
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) xb[nb] = pair_operand(ks[2 * kk][nb], ks[2 * kk + 1][nb]);
#pragma unroll
    for (int tb = 2 * kk; tb < 4; ++tb) {
      const bf16x8 a2 = cat(ldtr(&sm.t2[t2_slot(tb, 2 * kk)][0] + sl.t2off),
                            ldtr(&sm.t2[t2_slot(tb, 2 * kk + 1)][0] + sl.t2off));
#pragma unroll
      for (int nb = 0; nb < KNB; ++nb) u[tb][nb] = mfma(a2, xb[nb], u[tb][nb]);
    }
  }
  // ---- (Qt S)^T (rows n, columns t), then O^T = (Qt S)^T + U^T P^T
  f32x4 ot[KNB][4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) ot[nb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 qa[2][4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) qa[0][tb] = lds8(sm.qt + sl.roff[0] + 16 * tb * D);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int cur = kk & 1;
    fence();
    if (kk < 3) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) qa[cur ^ 1][tb] = lds8(sm.qt + sl.roff[kk + 1] + 16 * tb * D);
    }
    fence();
    bf16x8 sb[KNB];
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) sb[nb] = pair_operand(sacc[2 * kk][nb], sacc[2 * kk + 1][nb]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int nb = 0; nb < KNB; ++nb) ot[nb][tb] = mfma(sb[nb], qa[cur][tb], ot[nb][tb]);
  }
  fence();
  bf16x8 ub[2][KNB];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) ub[k2][nb] = pair_operand(u[2 * k2][nb], u[2 * k2 + 1][nb]);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int tb = 2 * kk; tb < 4; ++tb) {
      const bf16x8 pa = lds8(sm.p + sl.poff + 16 * tb * PP + 32 * kk);
#pragma unroll
      for (int nb = 0; nb < KNB; ++nb) ot[nb][tb] = mfma(ub[kk][nb], pa, ot[nb][tb]);
    }
  // ---- S <- diag(e^{gamma_last}) S + Kh^T U (register row d holds state row sigma(d))
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const f32x4 f = *reinterpret_cast<const f32x4*>(&sm.glast[sigma(16 * db + 4 * lg)]);
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) sacc[db][nb] *= f;
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    fence();
    bf16x8 kt[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint16_t* src = sm.kh + sl.toff[db >> 1][db & 1] + 32 * half * D;
      kt[db] = cat(ldtr(src), ldtr(src + 16 * D));
    }
    fence();
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int nb = 0; nb < KNB; ++nb) sacc[db][nb] = mfma(kt[db], ub[half][nb], sacc[db][nb]);
  }
  fence();
  // ---- O rows: lane holds O[16 tb + r][n0 + 8 g .. +7]; rows past the end dropped
  const int nv = min(BT, q.L - chunk * BT), Hv = a.num_v_heads;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(reinterpret_cast<uint16_t*>(a.out) + ((int64_t)q.r0 + chunk * BT + 16 * tb) * Hv * D,
                  (uint32_t)max(nv - 16 * tb, 0) * Hv * D * 2);
    const u32x4 o = {pack_bf16x2(ot[0][tb][0], ot[0][tb][1]), pack_bf16x2(ot[0][tb][2], ot[0][tb][3]),
                     pack_bf16x2(ot[1][tb][0], ot[1][tb][1]), pack_bf16x2(ot[1][tb][2], ot[1][tb][3])};
    __builtin_amdgcn_raw_buffer_store_b128(o, ro, sl.olane, 0, 0);
  }
}

__global__ __launch_bounds__(KNT) void kda_chunk_kernel(ScanArgs a, SeqOrder ord) {
  __shared__ KSmem sm;
  const int Hv = a.num_v_heads;
  const int rank = blockIdx.x / Hv;
  KSeq q;
  q.m = blockIdx.x % Hv;
  q.s = ord.n > 0 ? (rank < ord.n ? (int)ord.seq[rank] : a.num_seqs) : rank;
  if (q.s >= a.num_seqs) return;
  q.r0 = a.cu[q.s];
  q.L = a.cu[q.s + 1] - q.r0;
  if (q.L < a.min_len || q.L > a.max_len) return;
  if (!seq_active(a.read_idx, a.write_idx, q.s, a.num_blocks)) return;
  q.N = (q.L + BT - 1) / BT;
  q.h = q.m / (Hv / a.num_k_heads);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lane ln{lane & 15, lane >> 4, lane & 3, (lane >> 2) & 3};

  // the state [d][n] staged through the first tiles (free before the first chunk)
  float* sst = reinterpret_cast<float*>(&sm.kb[0]);
  const int64_t head_off = (int64_t)q.m * D * D;
  {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(
        reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.ssm_pool) +
                                       (int64_t)a.read_idx[q.s] * a.ssm_stride) + head_off, D * D * 4);
#pragma unroll
    for (int it = 0; it < D * D / 4 / KNT; ++it) {
      const int f = tid + KNT * it, row = f >> 5, c4 = f & 31;
      *reinterpret_cast<u32x4*>(&sst[row * KPS + 4 * c4]) = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * f, 0, 0);
    }
  }
  // the zero block of T2 and the P blocks above the diagonal are read by the
  // full-width products and never written (p lies outside the staging area)
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int i = tid; i < BT * PP / 8; i += KNT) reinterpret_cast<u32x4*>(&sm.p[0])[i] = zero;
    for (int i = tid; i < 16 * PB / 8; i += KNT) reinterpret_cast<u32x4*>(&sm.t2[10][0])[i] = zero;
  }
  __syncthreads();
  // Two roles with the same sequence of workgroup barriers per chunk:
  //   [1] diag_exact cleared  [2] block totals  [3] tiles  [4] A and P blocks
  //   (2 per diagonal block computed exactly)  [5] diagonal solve  [6] block solve
  //   [7] state pass done, the tiles are free again.
  if (wv < KNS) {
    // ---- state waves: the fp32 state of their columns in registers
    StateLanes sl;
    f32x4 sacc[8][KNB];
    const int n0 = 16 * KNB * wv, li = ln.r, lg = ln.g;
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) sl.col[nb] = n0 + 8 * (li >> 2) + 4 * nb + (li & 3);
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int nb = 0; nb < KNB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[db][nb][i] = sst[sigma(16 * db + 4 * lg + i) * KPS + sl.col[nb]];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) sl.roff[kk] = swz_off(li, 32 * kk + 8 * lg);
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int e = 0; e < 2; ++e) sl.toff[h][e] = swz_off(4 * lg + ln.i, 32 * h + 8 * ln.a) + 4 * e;
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) sl.voffs[nb] = swz_off(4 * lg + ln.i, n0 + 8 * ln.a + 4 * nb);
    sl.t2off = (4 * lg + ln.i) * PB + 4 * ln.a;
    sl.poff = li * PP + 8 * lg;
    sl.olane = 2 * (li * Hv * D + 8 * lg + q.m * D + n0);
    __syncthreads();  // the staged state has been read
    for (int c = 0; c < q.N; ++c) {
      __syncthreads();  // [1]
      __syncthreads();  // [2]
      __syncthreads();  // [3]
      __syncthreads();  // [4]
      const int ex = sm.diag_exact;  // uniform
      for (int b = 0; b < 4; ++b)
        if (ex & (1 << b)) {
          __syncthreads();
          __syncthreads();
        }
      __syncthreads();  // [5]
      __syncthreads();  // [6]
      kda_state_step(sm, sacc, sl, a, q, c, ln);
      __syncthreads();  // [7]
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int nb = 0; nb < KNB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sst[sigma(16 * db + 4 * lg + i) * KPS + sl.col[nb]] = sacc[db][nb][i];
  } else {
    // ---- producer waves: tiles, A and P blocks, T
    const int tp = tid - 64 * KNS;
    __syncthreads();  // the state waves have read the staged state
    for (int c = 0; c < q.N; ++c) {
      if (tp == 0) sm.diag_exact = 0;
      __syncthreads();  // [1]
      kda_totals(sm, a, q, c, tp);
      __syncthreads();  // [2]
      kda_tiles(sm, a, q, c, tp);
      __syncthreads();  // [3]
      kda_blocks(sm, wv - KNS, ln);
      __syncthreads();  // [4]
      const int ex = sm.diag_exact;  // uniform
      for (int b = 0; b < 4; ++b)
        if (ex & (1 << b)) {
          exact_diag(sm, a, q, c, b, tp);  // one barrier inside
          __syncthreads();
        }
      if (wv == KNS) solve_diag(sm.at, sm.tb, &sm.t2[0][0], sm.beta, lane);
      __syncthreads();  // [5]
      if (wv == KNS) solve_blocks(sm.ab, sm.tb, &sm.t2[0][0], sm.beta, ln);
      __syncthreads();  // [6]
      __syncthreads();  // [7]
    }
  }
  __syncthreads();
  {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(
        reinterpret_cast<float*>(reinterpret_cast<char*>(a.ssm_pool) + (int64_t)a.write_idx[q.s] * a.ssm_stride) +
            head_off, D * D * 4);
#pragma unroll
    for (int it = 0; it < D * D / 4 / KNT; ++it) {
      const int f = tid + KNT * it, row = f >> 5, c4 = f & 31;
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(&sst[row * KPS + 4 * c4]), rs, 16 * f, 0, 0);
    }
  }
}

}  // namespace

bool kda_chunk_supported(int dk, int dv) { return dk == D && dv == D; }

hipError_t launch_kda_chunk(const ScanArgs& a, const SeqOrder& order, hipStream_t st) {
  if (!kda_chunk_supported(D, D) || !a.y) return hipErrorInvalidValue;
  const int rows = order.n > 0 ? order.n : a.num_seqs;
  hipLaunchKernelGGL(kda_chunk_kernel, dim3(rows * a.num_v_heads), dim3(KNT), 0, st, a, order);
  return hipGetLastError();
}

GDN_STATUS_ACCESSOR(status_kda)

}  // namespace gdn
