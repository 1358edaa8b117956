// gdn_chunk.hip -- chunked prefill of the gated delta rule on gfx950 MFMA.
//
// Recurrence (Gated Delta Networks, Yang et al., ICLR 2025), state of a value
// head stored [d_k][d_v], carried per request in its cache block (page
// "Continuous batching for linear attention layers", PR description):
//     S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t.
// It is evaluated 64 tokens at a time in the WY / UT-transform form (chunkwise
// DeltaNet, Yang et al., NeurIPS 2024).  Inside a chunk, gamma is the running sum
// of g, Gamma = exp(gamma), and with K, Q, V the chunk's rows:
//     A  = strictly-lower( b_t e^{gamma_t-gamma_j} k_t.k_j ),   T = (I + A)^-1
//     U  = T diag(b) V - T diag(b Gamma) K S = T2 (V - diag(Gamma) K S),  T2 = T diag(b)
//     O  = diag(Gamma) Q S + (M o Q K^T) U,   M_tj = e^{gamma_t-gamma_j} (j <= t)
//     S <- Gamma_c S + K^T diag(e^{gamma_c-gamma}) U
// Only differences of running sums are exponentiated, so every factor is <= 1.
// (U is the usual U~ - W S with W = T diag(b Gamma) K, U~ = T diag(b) V, with
// T factored out, so W is never formed.)
//
// Work split: one 512-thread workgroup (8 waves, two per SIMD) per (sequence,
// value head), walking the sequence's chunks as a software pipeline with one
// workgroup barrier per step.  In step i:
//   waves 0-3 (state)  chunk i: wave w owns d_v columns [32w, 32w+32) of the
//                      128 x 128 fp32 state, in registers; it computes K S,
//                      (Q S)^T, U, O^T and the state update for its columns;
//                      its two 16-column tiles interleave in groups of 4
//                      columns, so each lane ends with 8 adjacent outputs;
//   wave 4 (gram)      chunk i+2: the Gram products and A from K rows loaded
//                      straight into registers, diagonal blocks first;
//   wave 6 (loads)     chunk i+1: Q, K and V rows copied from global memory
//                      straight into LDS (no registers), whole rows per load,
//                      and gamma, e^gamma, e^(gamma_c - gamma);
//                      chunk i+2: fp32 forward substitution on the four 16x16
//                      diagonal blocks of T, as soon as wave 4 has published
//                      the diagonal blocks of A;
//   wave 5 (blocks)    chunk i+1: the blocks of T below the diagonal by block
//                      products (two levels), written as T2^T, then rows
//                      48-63 of P = M o Q K^T;
//   wave 7 (P)         chunk i+1: once wave 6 has published the Q and K rows
//                      and gamma, rows 0-47 of P.
// Within a step, a consumer waits for its producer on an LDS flag (the rows of
// the next chunk, the diagonal blocks of A); everything else is read one or two
// steps after it is written (double-buffered Q/K/V and P, triple-buffered T2),
// across the barrier that ends each step.  Global pointers are address
// space 1 and the barriers wait for LDS traffic only, so loads and the output
// stores stay in flight across them.  All products are
// v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulate).  Sequences are
// launched longest first.
//
// Before the scans, the workgroups can also run the depthwise conv + SiLU +
// q/k normalisation of the launch's rows themselves, as tasks claimed from a
// global counter (conv_phase below): the workgroups of the longest sequences
// start their scans as soon as their own rows are done, while the others go
// on converting, so most of the conv is hidden behind the long scans.  The
// host picks this when every workgroup is resident at once (one per CU) and
// its time model says it pays; otherwise a separate conv kernel runs first.
//
// MFMA 16x16x32 bf16 operand layout (lane l, r = l & 15, grp = l >> 4):
//   A: row r, 8 values of k;  B: column r, the same 8 values of k;
//   D: column r, rows 4*grp + {0,1,2,3}.
// The MFMA sums over k, so any k order shared by both operands gives the same
// product.  A D tile X can be used as the B operand X or as the A operand X^T
// of a later product; a pair of D tiles (row blocks 2kk and 2kk+1) is then an
// operand over the 32 k values {4grp..4grp+3, 16+4grp..16+4grp+3} of step kk
// ("pair order").  The state rows are kept in registers relabelled so that
// pair order over d is natural order over the columns of K and Q: register
// row d = 32kk + 16h + 4g + i holds state row sigma(d) = 32kk + 8g + 4h + i, so
// a pair operand over d is one natural 16-byte chunk of a K or Q row, and K
// and Q rows can stay in natural column order in LDS.
#include "gdn_device.h"
#include "gdn_mfma.h"
#include "gdn_convtask.h"

namespace gdn {
namespace {

constexpr int NS = 4;             // state waves
constexpr int NT = 512;           // threads per workgroup (8 waves)
constexpr int NB = D / 16 / NS;   // 16-column state tiles per state wave
constexpr int PS = D + 4;         // fp32 pitch of the state staged in LDS (start and end)

// LDS.  The [64][128] bf16 tiles keep natural row-major order with the 16-byte
// chunk c of row t stored at chunk c ^ f(t) (swz_f): every pass of a row-operand
// read then falls on distinct banks, and a transposed read on each bank twice.
struct ChunkBuf {
  uint16_t q[BT * D];
  uint16_t k[BT * D];
  uint16_t v[BT * D];
  float gam[BT];              // running sum of g
  float eg[BT];               // e^gamma
  float ed[BT];               // e^(gamma_last - gamma)
};
struct alignas(16) Smem {
  ChunkBuf cb[2];             // chunk i & 1: written by wave 6, read by the state waves and waves 5, 7
  uint16_t p[2][BT * PP];     // P of chunk i & 1, [t][j in pair order]; blocks above the diagonal stay zero
  uint16_t t2[3][11][16 * PB]; // (T diag(b))^T of chunk i % 3 as 16 x 16 blocks [j][t] (t2_slot), and a zero block
  uint16_t ab[2][6][16 * PB]; // A^T blocks below the diagonal (gram wave -> blocks wave)
  uint16_t tb[2][5][16 * PB]; // T^T blocks 00, 11, 22, 33 (gram wave) and 32 (blocks wave)
  float at[4 * 16 * PA];      // diagonal blocks of A, fp32, [block][j][t] (gram wave -> wave 6)
  float bsc[2][BT];           // beta of the chunk (gram wave -> blocks wave)
  float gw[BT];               // gamma, gram wave
  int dflag;                  // chunks whose Q / K / V rows are in LDS
  int aflag;                  // chunks whose diagonal blocks of A are in `at`
  int task, task2, task3, task4;  // conv tasks claimed for the workgroup
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS");
static_assert(offsetof(Smem, task) >= 16 * 8 * 1024, "the conv row staging (16 rows x 8 KiB) stays clear of the task slot");
static_assert(NT == kConvThreads, "the conv tasks assume 8 waves");
static_assert(D * PS * 4 <= sizeof(ChunkBuf) * 2, "state staging");

// Buffer offsets below are passed whole as the vector offset: the range check
// that zeroes loads and drops stores past the end applies to that offset.

// Per-workgroup constants.
struct Seq {
  int s, r0, L, N, m, qoff, koff, voff;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rows(const ScanArgs& a, const Seq& q, int c) {
  const int nv = min(BT, q.L - c * BT);
  return make_rsrc(reinterpret_cast<const uint16_t*>(a.y) + (int64_t)(q.r0 + c * BT) * a.channels,
                   (uint32_t)nv * a.channels * 2);
}
__device__ __forceinline__ void load_gb(const ScanArgs& a, const Seq& q, int c, int lane, float& g, float* b) {
  const int nv = min(BT, q.L - c * BT), Hv = a.num_v_heads;
  const int64_t rb = q.r0 + c * BT;
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.g + rb * Hv, (uint32_t)nv * Hv * 4);
  g = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, 4 * (lane * Hv + q.m), 0, 0));
  if (b) {
    const __amdgpu_buffer_rsrc_t rbt = make_rsrc(a.beta + rb * Hv, (uint32_t)nv * Hv * 4);
    *b = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbt, 4 * (lane * Hv + q.m), 0, 0));
  }
}

// Rows 16 B0 .. 16 B1 + 15 of P = M o Q K^T for one chunk, into a P buffer:
// blocks (bi, bj), bj <= bi, as D tiles of K_bj Q_bi^T, chains interleaved, each
// step's operand rows read one step ahead.
template <int B0, int B1>
__device__ __forceinline__ void p_rows(uint16_t* p, const ChunkBuf& cb, const Lane& ln) {
  constexpr int NBLK = (B1 + 1) * (B1 + 2) / 2 - B0 * (B0 + 1) / 2;
  int roff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) roff[kk] = swz_off(ln.r, 32 * kk + 8 * ln.g);
  f32x4 acc[NBLK];
#pragma unroll
  for (int e = 0; e < NBLK; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 kr[2][B1 + 1], qr[2][B1 + 1];
#pragma unroll
  for (int b = 0; b <= B1; ++b) {
    kr[0][b] = lds8(cb.k + roff[0] + 16 * b * D);
    if (b >= B0) qr[0][b] = lds8(cb.q + roff[0] + 16 * b * D);
  }
  float gt[B1 + 1];
  f32x4 gj[B1 + 1];
#pragma unroll
  for (int b = 0; b <= B1; ++b) {
    gt[b] = cb.gam[16 * b + ln.r];
    gj[b] = *reinterpret_cast<const f32x4*>(&cb.gam[16 * b + 4 * ln.g]);
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int cur = kk & 1;
    fence();
    if (kk < 3) {
#pragma unroll
      for (int b = 0; b <= B1; ++b) {
        kr[cur ^ 1][b] = lds8(cb.k + roff[kk + 1] + 16 * b * D);
        if (b >= B0) qr[cur ^ 1][b] = lds8(cb.q + roff[kk + 1] + 16 * b * D);
      }
    }
    fence();
#pragma unroll
    for (int bi = B0, e = 0; bi <= B1; ++bi)
#pragma unroll
      for (int bj = 0; bj <= bi; ++bj, ++e) acc[e] = mfma(kr[cur][bj], qr[cur][bi], acc[e]);
  }
  // lane holds P[t = 16bi + r][j = 16bj + 4g + i]
#pragma unroll
  for (int bi = B0, e = 0; bi <= B1; ++bi)
#pragma unroll
    for (int bj = 0; bj <= bi; ++bj, ++e) {
      const int t = 16 * bi + ln.r;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f = __expf(gt[bi] - gj[bj][i]) * acc[e][i];
        v[i] = (16 * bj + 4 * ln.g + i <= t) ? f : 0.f;
      }
      st4bf(&p[t * PP + perm(16 * bj + 4 * ln.g)], v[0], v[1], v[2], v[3]);
    }
}

// ---- waves 0-3: the state pass of chunk i for d_v columns [n0, n0 + 32).
// Every LDS operand read is a per-lane base offset plus a compile-time constant:
// the swizzle of row t depends on t & 15 only.
__device__ __forceinline__ void state_role(Smem& sm, float* sst, const ScanArgs& a, const Seq& q, int wv,
                                           const Lane& ln) {
  const int n0 = 16 * NB * wv, li = ln.r, lg = ln.g;
  const int Hv = a.num_v_heads;
  // tile nb, lane column r stands for state column n0 + 8 (r >> 2) + 4 nb + (r & 3);
  // register row d = 16 db + 4 lg + i holds state row sigma(d)
  int col[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) col[nb] = n0 + 8 * (li >> 2) + 4 * nb + (li & 3);
  f32x4 sacc[8][NB];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[db][nb][i] = sst[sigma(16 * db + 4 * lg + i) * PS + col[nb]];
  lds_barrier();  // the staged state is dead; P / T2 are cleared next
  lds_barrier();
  // row operands (K, Q): row 16 tb + li, columns 32 kk + 8 lg .. +7
  int roff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) roff[kk] = swz_off(li, 32 * kk + 8 * lg);
  // K^T operand for register rows 16 db..: the transposed-read source lane reads
  // row 4 lg + i (+32 kk, +16), columns sigma(16 db + 4 a) = 32 (db >> 1) + 8 a + 4 (db & 1)
  int toff[4][2];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int e = 0; e < 2; ++e) toff[h][e] = swz_off(4 * lg + ln.i, 32 * h + 8 * ln.a) + 4 * e;
  // V in D layout: source lane reads row 4 lg + i (+16 tb), columns n0 + 8 a + 4 nb .. +3
  int voffs[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) voffs[nb] = swz_off(4 * lg + ln.i, n0 + 8 * ln.a + 4 * nb);
  const int t2off = (4 * lg + ln.i) * PB + 4 * ln.a;  // T2 rows as A operands, within a block
  const int poff = li * PP + 8 * lg;                   // P rows as B operands
  const int olane = 2 * (li * Hv * D + 8 * lg + q.m * D + n0);
  lds_barrier();  // step -2
  lds_barrier();  // step -1
  int b3 = 0;     // i % 3
  for (int it = 0; it < q.N; ++it) {
    const ChunkBuf& cb = sm.cb[it & 1];
    const uint16_t* t2 = &sm.t2[b3][0][0];
    const uint16_t* pb = sm.p[it & 1];
    // The chain K S -> X -> U -> state update is serial; (Q S)^T is only needed
    // for O, so its products run while U and its operand packing complete.
    // ---- K S (rows t, columns n)
    f32x4 ks[4][NB];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) ks[tb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 ka[2][4], a2[2][4];
    bf16x4 vv[4][NB];  // V[16 tb + 4 lg + i][state columns of tile nb]
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) ka[0][tb] = lds8(cb.k + roff[0] + 16 * tb * D);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1;
      fence();
      if (kk < 3) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) ka[cur ^ 1][tb] = lds8(cb.k + roff[kk + 1] + 16 * tb * D);
      } else {  // the operands of X and U
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int tb = 2 * k2; tb < 4; ++tb)  // T2 rows 16 tb + li, j of step k2 in pair order
            a2[k2][tb] = cat(ldtr(t2 + t2_slot(tb, 2 * k2) * 16 * PB + t2off),
                             ldtr(t2 + t2_slot(tb, 2 * k2 + 1) * 16 * PB + t2off));
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) vv[tb][nb] = ldtr(cb.v + voffs[nb] + 16 * tb * D);
      }
      fence();
      bf16x8 sb[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sb[nb] = pair_operand(sacc[2 * kk][nb], sacc[2 * kk + 1][nb]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) ks[tb][nb] = mfma(ka[cur][tb], sb[nb], ks[tb][nb]);
    }
    fence();
    // ---- X = V - diag(Gamma) K S,  U = T2 X
    f32x4 u[4][NB];
    {
      f32x4 x[4][NB];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const f32x4 gv = *reinterpret_cast<const f32x4*>(&cb.eg[16 * tb + 4 * lg]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) x[tb][nb][i] = __builtin_fmaf(-gv[i], ks[tb][nb][i], (float)vv[tb][nb][i]);
          u[tb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 xb[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) xb[nb] = pair_operand(x[2 * kk][nb], x[2 * kk + 1][nb]);
#pragma unroll
        for (int tb = 2 * kk; tb < 4; ++tb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) u[tb][nb] = mfma(a2[kk][tb], xb[nb], u[tb][nb]);
      }
    }
    fence();
    // ---- (Q S)^T (rows n, columns t); U's operands are packed between its steps
    f32x4 ot[NB][4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) ot[nb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 qa[2][4], ub[2][NB], upb[2][NB], kt[8], pa[6];
    float egt[4];
    float gc = 0.f;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) qa[0][tb] = lds8(cb.q + roff[0] + 16 * tb * D);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1;
      fence();
      if (kk < 3) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) qa[cur ^ 1][tb] = lds8(cb.q + roff[kk + 1] + 16 * tb * D);
      }
      if (kk == 3) {  // the operands of O
#pragma unroll
        for (int tb = 0, e = 0; tb < 4; ++tb)
#pragma unroll
          for (int k2 = 0; k2 <= (tb >> 1); ++k2, ++e) pa[e] = lds8(pb + poff + 16 * tb * PP + 32 * k2);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) egt[tb] = cb.eg[16 * tb + li];
        gc = cb.eg[BT - 1];
      }
      fence();
      bf16x8 sb[NB];  // packed again: an empty asm hides that the K S loop packed the same
                      // values, which would otherwise be kept alive (32 registers)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        asm volatile("" : "+v"(sacc[2 * kk][nb]), "+v"(sacc[2 * kk + 1][nb]));
        sb[nb] = pair_operand(sacc[2 * kk][nb], sacc[2 * kk + 1][nb]);
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) ot[nb][tb] = mfma(sb[nb], qa[cur][tb], ot[nb][tb]);
      if (kk == 1) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(&cb.ed[32 * k2 + 4 * lg]);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(&cb.ed[32 * k2 + 16 + 4 * lg]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            ub[k2][nb] = pair_operand(u[2 * k2][nb], u[2 * k2 + 1][nb]);
            upb[k2][nb] = pair_operand(u[2 * k2][nb] * d0, u[2 * k2 + 1][nb] * d1);
          }
        }
      }
    }
    fence();
    // ---- O^T = Gamma-scaled (Q S)^T + U^T P^T;  S <- Gamma_c S + K^T diag(e^{gamma_c - gamma}) U
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint16_t* src = cb.k + toff[db >> 1][db & 1];
      kt[db] = cat(ldtr(src), ldtr(src + 16 * D));
    }
    fence();
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) ot[nb][tb] *= egt[tb];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int tb = 2 * kk; tb < 4; ++tb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          ot[nb][tb] = mfma(ub[kk][nb], pa[kk == 0 ? (tb < 2 ? tb : 2 * tb - 2) : 2 * tb - 1], ot[nb][tb]);
    // tokens 0..31, then 32..63; the second half's operands are read during the
    // first half's products
    bf16x8 kn[8];
    fence();
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint16_t* src = cb.k + toff[db >> 1][db & 1] + 32 * D;
      kn[db] = cat(ldtr(src), ldtr(src + 16 * D));
    }
    fence();
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        sacc[db][nb] *= gc;
        sacc[db][nb] = mfma(kt[db], upb[0][nb], sacc[db][nb]);
      }
    fence();
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sacc[db][nb] = mfma(kn[db], upb[1][nb], sacc[db][nb]);
    fence();
    // ---- O rows: lane holds O[16 tb + li][n0 + 8 lg .. +7]; one buffer range per
    //      16-row block drops the rows past the end
    {
      const int nv = min(BT, q.L - it * BT);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(reinterpret_cast<uint16_t*>(a.out) + (int64_t)(q.r0 + it * BT + 16 * tb) * Hv * D,
                      (uint32_t)max(nv - 16 * tb, 0) * Hv * D * 2);
        const u32x4 o = {pack_bf16x2(ot[0][tb][0], ot[0][tb][1]), pack_bf16x2(ot[0][tb][2], ot[0][tb][3]),
                         pack_bf16x2(ot[1][tb][0], ot[1][tb][1]), pack_bf16x2(ot[1][tb][2], ot[1][tb][3])};
        __builtin_amdgcn_raw_buffer_store_b128(o, ro, olane, 0, 0);
      }
    }
    b3 = b3 == 2 ? 0 : b3 + 1;
    lds_barrier();
  }
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sst[sigma(16 * db + 4 * lg + i) * PS + col[nb]] = sacc[db][nb][i];
}

// ---- wave 4: A for chunk i + 2, its diagonal blocks published first
// ready: the chunk counters of the sequence when the conv runs inside the
// kernel, else NULL (the conv kernel ran before it)
__device__ __forceinline__ void gram_role(Smem& sm, const ScanArgs& a, const Seq& q, int lane, const Lane& ln,
                                          const int32_t* ready, int slices) {
  Blk gk[4];
  float g4, b4;
  int upto = 0;  // chunks below this one are known to be converted
  auto load = [&](int c) {
    if (ready) upto = chunk_wait(ready, slices, q.L, c, upto, lane);
    const __amdgpu_buffer_rsrc_t ry = chunk_rows(a, q, c);
#pragma unroll
    for (int b = 0; b < 4; ++b) gk[b] = ld_blk_g(ry, a.channels, q.koff, b, ln);
    load_gb(a, q, c, lane, g4, &b4);
  };
  load(0);
  for (int it = -2; it < q.N; ++it) {
    const int c = it + 2;
    if (c < q.N) {
      float* beta = sm.bsc[c & 1];
      sm.gw[lane] = wave_prefix_sum(g4);
      beta[lane] = b4;
      // K K^T blocks (b, b), then (bi, bj) with bj < bi; the chains interleaved
      f32x4 ad[4], ao[6];
#pragma unroll
      for (int b = 0; b < 4; ++b) ad[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 6; ++e) ao[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int b = 0; b < 4; ++b) ad[b] = mfma(gk[b].v[kk], gk[b].v[kk], ad[b]);
#pragma unroll
      for (int b = 0; b < 4; ++b) put_a(sm.at, sm.ab[c & 1], sm.gw, beta, b, b, ad[b], ln);
      set_flag(&sm.aflag, c + 1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int bi = 1, e = 0; bi < 4; ++bi)
#pragma unroll
          for (int bj = 0; bj < bi; ++bj, ++e) ao[e] = mfma(gk[bi].v[kk], gk[bj].v[kk], ao[e]);
      if (c + 1 < q.N) load(c + 1);
#pragma unroll
      for (int bi = 1, e = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < bi; ++bj, ++e) put_a(sm.at, sm.ab[c & 1], sm.gw, beta, bi, bj, ao[e], ln);
    }
    lds_barrier();
  }
}

// ---- wave 5: the blocks of T below the diagonal and rows 48-63 of P for chunk i + 1
__device__ __forceinline__ void blocks_role(Smem& sm, const Seq& q, const Lane& ln) {
  int b3 = 2;  // (i + 1) % 3
  for (int it = -2; it < q.N; ++it) {
    const int c = it + 1;
    if (c >= 0 && c < q.N) {
      solve_blocks(sm.ab[c & 1], sm.tb[c & 1], &sm.t2[b3][0][0], sm.bsc[c & 1], ln);
      wait_flag(&sm.dflag, c + 1);  // the chunk's Q and K rows are in LDS
      p_rows<3, 3>(sm.p[c & 1], sm.cb[c & 1], ln);
    }
    b3 = b3 == 2 ? 0 : b3 + 1;
    lds_barrier();
  }
}

// ---- wave 6: Q, K and V rows of chunk i + 1 copied from global memory straight
// into LDS, with the decay vectors; then the diagonal blocks of T for chunk
// i + 2.  Load j writes LDS bytes [1024 j, 1024 j + 1024) of a tile, i.e.
// rows 4j..4j+3; lane l fills chunk slot l & 15 of row 4j + (l >> 4), so it reads
// the natural chunk (l & 15) ^ f(row): every load covers four whole 256-byte rows.
__device__ __forceinline__ void load_role(Smem& sm, const ScanArgs& a, const Seq& q, int lane) {
  const int C = a.channels, t0 = lane >> 4, sl = lane & 15;
  float gv;
  load_gb(a, q, 0, lane, gv, nullptr);
  int b3 = 0;  // (i + 2) % 3
  for (int it = -2; it < q.N; ++it) {
    const int c = it + 1;
    if (c >= 0 && c < q.N) {
      ChunkBuf& cn = sm.cb[c & 1];
      const __amdgpu_buffer_rsrc_t ry = chunk_rows(a, q, c);
      // Q and K first (P waits for them), then V (read next step)
#pragma unroll
      for (int j = 0; j < BT / 4; ++j) {
        const int t = 4 * j + t0;
        const int go = 2 * (t * C + 8 * (sl ^ swz_f(t)));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (__attribute__((address_space(3))) void*)(cn.q + 512 * j), 16,
                                                 go + 2 * q.qoff, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (__attribute__((address_space(3))) void*)(cn.k + 512 * j), 16,
                                                 go + 2 * q.koff, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < BT / 4; ++j) {
        const int t = 4 * j + t0;
        const int go = 2 * (t * C + 8 * (sl ^ swz_f(t)));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (__attribute__((address_space(3))) void*)(cn.v + 512 * j), 16,
                                                 go + 2 * q.voff, 0, 0, 0);
      }
      {
        const float gam = wave_prefix_sum(gv);
        const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gam), 63));
        cn.gam[lane] = gam;
        cn.eg[lane] = __expf(gam);
        cn.ed[lane] = __expf(glast - gam);
      }
      const int nv = min(BT, q.L - c * BT);
      const u32x4 zero = {0u, 0u, 0u, 0u};
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // loads complete in order: Q and K have landed
      if (nv < BT) {  // rows past the end of the sequence become zero
        for (int e = nv * 16 + lane; e < BT * 16; e += 64) {
          reinterpret_cast<u32x4*>(cn.q)[e] = zero;
          reinterpret_cast<u32x4*>(cn.k)[e] = zero;
        }
      }
      set_flag(&sm.dflag, c + 1);
      if (nv < BT) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        for (int e = nv * 16 + lane; e < BT * 16; e += 64) reinterpret_cast<u32x4*>(cn.v)[e] = zero;
      }
      if (c + 1 < q.N) load_gb(a, q, c + 1, lane, gv, nullptr);
    }
    const int cd = it + 2;
    if (cd < q.N) {
      wait_flag(&sm.aflag, cd + 1);  // the gram wave has written the diagonal blocks of A
      solve_diag(sm.at, sm.tb[cd & 1], &sm.t2[b3][0][0], sm.bsc[cd & 1], lane);
    }
    b3 = b3 == 2 ? 0 : b3 + 1;
    // the copies must have landed before the consumers read them next step
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

// ---- wave 7: rows 0-47 of P of chunk i + 1
__device__ __forceinline__ void p_role(Smem& sm, const Seq& q, const Lane& ln) {
  for (int it = -2; it < q.N; ++it) {
    const int c = it + 1;
    if (c >= 0 && c < q.N) {
      wait_flag(&sm.dflag, c + 1);  // the chunk's Q and K rows and gamma are in LDS
      p_rows<0, 2>(sm.p[c & 1], sm.cb[c & 1], ln);
    }
    lds_barrier();
  }
}

// New conv state of the sequence of `rank`: the last W-1 rows of [old state; x],
// once every conv task of the sequence (the readers of the old state) is done.
// Each thread reads all W-1 rows of its 8 channels before it writes, so the
// ordinary in-place case (read block == write block) is safe.
template <bool DP>
__device__ void commit_tail(Smem& sm, const ScanArgs& a, const SeqOrder& ord, const FusedConv& fc, int rank) {
  const int W = a.width;
  if (W < 2) return;
  conv_wait<DP>(fc, rank);  // the tasks of every rank are claimed before the last rank's are
  const int s = plan_seq<DP>(ord, fc, rank);
  if (!seq_active(a.read_idx, a.write_idx, s, a.num_blocks)) return;  // uniform
  const int r0 = a.cu[s], L = a.cu[s + 1] - r0, C = a.channels;
  const gptr<const u32x4> x = as_global(reinterpret_cast<const u32x4*>(a.x));
  const gptr<const u32x4> src = as_global(reinterpret_cast<const u32x4*>(a.conv_pool + (int64_t)a.read_idx[s] * a.conv_stride));
  const gptr<u32x4> dst = as_global(reinterpret_cast<u32x4*>(const_cast<char*>(a.conv_pool) + (int64_t)a.write_idx[s] * a.conv_stride));
  for (int cq = threadIdx.x; cq < C / 8; cq += NT) {  // 16-byte column
    u32x4 v[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int i = L + j;  // row of [old state; x]
      if (j < W - 1) v[j] = i < W - 1 ? src[(int64_t)i * (C / 8) + cq] : x[(int64_t)(r0 + i - (W - 1)) * (C / 8) + cq];
    }
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < W - 1) dst[(int64_t)j * (C / 8) + cq] = v[j];
  }
}

// Plans a launch on the device from cu_seqlens, for calls that leave the
// planning to the device (graph capture): the launch order of the chunked
// sequences (length >= 2; longest first, then lower index), the conv task
// ranges, the choice between the conv inside the chunk kernel and the conv
// kernel, and the makespan target, all by the same rules as the host plan; and
// it zeroes the task counters.  One workgroup of 1024 threads, one thread per
// sequence.
__global__ __launch_bounds__(1024) void plan_kernel(PlanArgs a) {
  __shared__ int len[kMaxPlanSeqs];
  __shared__ int tasks[kMaxPlanSeqs];
  __shared__ int n_long, longest, chunks_sum;
  const int tid = threadIdx.x, N = a.num_seqs;
  if (tid == 0) {
    n_long = 0;
    longest = 0;
    chunks_sum = 0;
  }
  for (int i = tid; i < N; i += blockDim.x) len[i] = a.cu[i + 1] - a.cu[i];
  __syncthreads();
  int rank = -1;
  if (tid < N && len[tid] >= 2) {
    const int L = len[tid];
    rank = 0;
    for (int j = 0; j < N; ++j) rank += (len[j] >= 2 && (len[j] > L || (len[j] == L && j < tid))) ? 1 : 0;
    a.plan[kPlanOrder + rank] = tid;
    atomicAdd(&n_long, 1);
    atomicMax(&longest, L);
    atomicAdd(&chunks_sum, (L + BT - 1) / BT);
  }
  __syncthreads();
  const int n = n_long;
  // the task counters: [0], one per rank, one per chunk of each rank
  for (int i = tid; i < 1 + n + chunks_sum; i += blockDim.x) a.sync[i] = 0;
  if (rank >= 0) tasks[rank] = (len[tid] + a.conv_rows - 1) / a.conv_rows * a.slices;
  __syncthreads();
  // inclusive scan of tasks[0 .. n) (Hillis-Steele; one entry per thread)
  for (int off = 1; off < n; off <<= 1) {
    const int v = (tid < n && tid >= off) ? tasks[tid - off] : 0;
    __syncthreads();
    if (tid < n) tasks[tid] += v;
    __syncthreads();
  }
  int32_t* first = a.plan + kPlanOrder + N;
  if (tid == 0) first[0] = 0;
  if (tid < n) first[tid + 1] = tasks[tid];
  if (tid == 0) {
    const int T = a.cu[N];
    const int total = n > 0 ? tasks[n - 1] : 0;
    const double scans = n * a.scan0_us + a.scan1_us * chunks_sum;
    const double lng = a.scan0_us + a.scan1_us * ((longest + BT - 1) / BT);
    double fused = n > 0 ? (total * a.task_us + a.num_v_heads * scans) / ((double)n * a.num_v_heads) : 0.0;
    fused = fmax(fused, lng + 2.0 * a.task_us);
    const double half = (a.cus > 2 ? a.cus : 2) / 2.0;
    const double crowd = fmin(1.0, fmax(0.0, ((double)n * a.num_v_heads - half) / half));
    const double apart = a.conv_us_per_token * T + a.scan0_us +
                         (a.plain_scan1_us + a.crowd_scan1_us * crowd) * ((longest + BT - 1) / BT) + 3.0;
    const int use = a.fused_allowed && n > 0 &&
                    (a.fused_forced || a.phased_scale * fused < apart || (a.beside_tokens && n < N));
    a.plan[kPlanN] = n;
    a.plan[kPlanFused] = use;
    a.plan[kPlanTarget] = (int32_t)(fused * a.margin);
    a.plan[3] = 0;
  }
}

// New conv state of sequence s (the last W-1 rows of [old state; x]) once no
// conv task reads the old one any more; each thread reads its rows before it
// writes them, so the in-place case is safe.
__device__ void write_tail(const ScanArgs& a, int s) {
  const int W = a.width;
  if (W < 2 || !seq_active(a.read_idx, a.write_idx, s, a.num_blocks)) return;
  const int r0 = a.cu[s], L = a.cu[s + 1] - r0, C = a.channels;
  const gptr<const u32x4> x = as_global(reinterpret_cast<const u32x4*>(a.x));
  const gptr<const u32x4> src = as_global(reinterpret_cast<const u32x4*>(a.conv_pool + (int64_t)a.read_idx[s] * a.conv_stride));
  const gptr<u32x4> dst = as_global(reinterpret_cast<u32x4*>(const_cast<char*>(a.conv_pool) + (int64_t)a.write_idx[s] * a.conv_stride));
  for (int cq = threadIdx.x; cq < C / 8; cq += NT) {
    u32x4 v[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int i = L + j;  // row of [old state; x]
      if (j < W - 1) v[j] = i < W - 1 ? src[(int64_t)i * (C / 8) + cq] : x[(int64_t)(r0 + i - (W - 1)) * (C / 8) + cq];
    }
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < W - 1) dst[(int64_t)j * (C / 8) + cq] = v[j];
  }
}

// Streaming helper workgroup: converts the rows the scans need next, in
// chunk-major order (the tasks of every rank's chunk 0, then of every rank's
// chunk 1, ...), the order in which the scans, which start together and step
// at the same pace, consume them.  Each task (kConvTaskRows rows x
// kConvTaskChannels channels) is counted in its chunk's counter.  As in conv_phase, the next task is claimed
// one task ahead and its rows load into LDS while the current one is
// computed.  Ends when every task is claimed; never waits for anything.
//
// Claims the next task: one atomic on the global counter, decoded over the
// ranks' chunk counts (ranks run longest first, so the ranks that still have
// a chunk c are a prefix of the order).  Returns (rank, task within the rank)
// or (-1, 0) once every task is claimed.  Tasks past a sequence's end in its
// last chunk are skipped; each pass takes a larger index, so the loop ends.
// Called by one wave with no other vector memory operation outstanding.
__device__ __forceinline__ int2 stream_claim(const ScanArgs& a, const SeqOrder& ord, const FusedConv& fc, int lane) {
  const int U = BT / kConvTaskRows * fc.slices;  // tasks per chunk of one rank
  for (;;) {
    int g = 0;
    if (lane == 0) g = __hip_atomic_fetch_add(fc.sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    g = __builtin_amdgcn_readfirstlane(g);
    int c0 = 0, r = -1, t = 0;
    for (int act = fc.n; act >= 1; --act) {  // chunks [c0, c1) are held by ranks 0 .. act-1
      const int c1 = fc.first[act] - fc.first[act - 1];
      const int span = (c1 - c0) * act * U;
      if (g < span) {
        const int c = c0 + g / (act * U), j = g % (act * U);
        r = j / U;
        t = c * U + j % U;
        break;
      }
      g -= span;
      c0 = c1;
    }
    if (r < 0) return int2{-1, 0};  // every task is claimed
    const int s = ord.seq[r];
    if ((t / fc.slices) * kConvTaskRows < a.cu[s + 1] - a.cu[s]) return int2{r, t};
  }
}

__device__ __forceinline__ ConvTask stream_task(const ScanArgs& a, const SeqOrder& ord, const FusedConv& fc, int r, int t) {
  ConvTask k;
  k.rank = r;
  k.s = ord.seq[r];
  k.seq0 = a.cu[k.s];
  conv_part(a, k, t / fc.slices, t % fc.slices);
  return k;
}

template <int W>
__device__ void stream_helper(Smem& sm, const ScanArgs& a, const SeqOrder& ord, const FusedConv& fc) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  int32_t* ready = fc.sync + 1;
  const u32x4* st = conv_stage(sm);
  // the first two tasks
  if (wv == 0) {
    const int2 c0 = stream_claim(a, ord, fc, lane);
    const int2 c1 = c0.x >= 0 ? stream_claim(a, ord, fc, lane) : int2{-1, 0};
    if (lane == 0) {
      sm.task = c0.x;
      sm.task2 = c0.y;
      sm.task3 = c1.x;
      sm.task4 = c1.y;
    }
  }
  lds_barrier();
  int r = sm.task, t = sm.task2, ur = sm.task3, ut = sm.task4;
  lds_barrier();  // read before wave 0 writes them again
  ConvTask k{};
  ConvSide<W> cur, nxt;
  if (r >= 0) {
    k = stream_task(a, ord, fc, r, t);
    conv_prefetch<W>(sm, a, k, nxt);
  }
  u32x4 rx[kConvWaveRows];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  while (r >= 0) {
    // wave 0 claims the task after the next one, with nothing else in flight
    int2 v{-1, 0};
    if (wv == 0 && ur >= 0) v = stream_claim(a, ord, fc, lane);
    cur = nxt;
    if (k.on) {
#pragma unroll
      for (int i = 0; i < kConvWaveRows; ++i) rx[i] = st[(i * kConvWaves + wv) * 64 + lane];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the next rows overwrite them
    ConvTask kn{};
    if (ur >= 0) {
      kn = stream_task(a, ord, fc, ur, ut);
      conv_prefetch<W>(sm, a, kn, nxt);
    }
    conv_compute<W>(a, k, cur, rx);
    if (tid == 0) {
      sm.task = v.x;
      sm.task2 = v.y;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this task's stores, the next task's rows
    lds_barrier();
    if (tid == 0)
      __hip_atomic_fetch_add(&ready[fc.first[k.rank] + k.row], 1,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    k = kn;
    r = ur;
    t = ut;
    ur = __builtin_amdgcn_readfirstlane(sm.task);
    ut = __builtin_amdgcn_readfirstlane(sm.task2);
    lds_barrier();  // read before wave 0 writes them again
  }
}

__device__ __forceinline__ void stream_helper_w(Smem& sm, const ScanArgs& a, const SeqOrder& ord, const FusedConv& fc) {
  switch (a.width) {
    case 1: stream_helper<1>(sm, a, ord, fc); break;
    case 2: stream_helper<2>(sm, a, ord, fc); break;
    case 3: stream_helper<3>(sm, a, ord, fc); break;
    default: stream_helper<4>(sm, a, ord, fc); break;
  }
}

__global__ void zero_sync_kernel(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

template <bool DP, bool STREAM>
__global__ __launch_bounds__(NT) void chunk_scan_kernel(ScanArgs a, SeqOrder ord, FusedConv fc) {
  __shared__ Smem sm;
  const int Hv = a.num_v_heads;
  int bid = blockIdx.x;
  if constexpr (STREAM) {
    // Roles by arrival: the first fc.helpers workgroups to start take a ticket
    // below fc.helpers and convert rows; the later ones scan.  So every helper
    // has started before any scan waits for converted rows, and the waits end
    // without any assumption about which workgroups are resident together.
    if (threadIdx.x == 0)
      sm.task = __hip_atomic_fetch_add(fc.sync + 1 + fc.first[fc.n], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    bid = __builtin_amdgcn_readfirstlane(sm.task);
    __syncthreads();  // read before a helper overwrites it
    if (bid < fc.helpers) {
      stream_helper_w(sm, a, ord, fc);
      return;
    }
    bid -= fc.helpers;
  }
  const int rank = bid / Hv;
  Seq q;
  q.m = bid % Hv;
  const int n_ord = plan_n<DP>(ord, fc);
  const int fused_n = STREAM ? 0 : plan_fused_n<DP>(fc);  // 0, or every rank of the launch order (phased conv)
  const bool lead_wg = q.m == 0;
  if (DP && rank >= n_ord) return;  // device plan: the grid covers every sequence
  q.s = n_ord > 0 ? (rank < n_ord ? plan_seq<DP>(ord, fc, rank) : a.num_seqs) : rank;
  if (fused_n > 0) {
    conv_phase_w<DP>(sm, a, ord, fc, rank);  // every rank < fused_n; waits come later
    // the workgroups of the shortest sequence, which finish long before the
    // others, write the new conv states: workgroup j those of ranks j, j + H_v, ...
    if (rank == fused_n - 1)
      for (int r = q.m; r < fused_n; r += Hv) commit_tail<DP>(sm, a, ord, fc, r);
  }
  if (fused_n > 0 || STREAM) {
    // value heads of one key head on one XCD (workgroups go round-robin over
    // the 8 XCDs), so the second reader of the shared Q and K rows can hit L2
    const int g = Hv / a.num_k_heads, per = Hv / 8;
    if (Hv % 8 == 0 && per % g == 0) {
      const int x = q.m % 8, sl = q.m / 8;
      q.m = g * (x * (per / g) + sl / g) + sl % g;
    }
  }
  if (q.s >= a.num_seqs) return;
  q.r0 = a.cu[q.s];
  q.L = a.cu[q.s + 1] - q.r0;
  if (q.L < a.min_len || q.L > a.max_len) return;
  if (!seq_active(a.read_idx, a.write_idx, q.s, a.num_blocks)) return;
  q.N = (q.L + BT - 1) / BT;
  const int h = q.m / (Hv / a.num_k_heads);
  q.qoff = h * D;
  q.koff = a.num_k_heads * D + h * D;
  q.voff = 2 * a.num_k_heads * D + q.m * D;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
  const Lane ln{lane & 15, lane >> 4, lane & 3, (lane >> 2) & 3};

  // the fp32 state [d][n] is staged through the chunk buffers, which are free
  // before the first step and after the last
  float* sst = reinterpret_cast<float*>(&sm.cb[0]);
  const int64_t head_off = (int64_t)q.m * D * D;
  {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(
        reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.ssm_pool) +
                                       (int64_t)__builtin_amdgcn_readfirstlane(a.read_idx[q.s]) * a.ssm_stride) +
            head_off, D * D * 4);
#pragma unroll
    for (int it = 0; it < D * D / 4 / NT; ++it) {
      const int f = tid + NT * it, row = f >> 5, c4 = f & 31;
      *reinterpret_cast<u32x4*>(&sst[row * PS + 4 * c4]) = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * f, 0, 0);
    }
  }
  // the scan waits for the converted rows chunk by chunk (the gram wave, the
  // first reader of each chunk's rows)
  const int32_t* ready = nullptr;
  if constexpr (STREAM) ready = fc.sync + 1 + fc.first[rank];
  else if (fused_n > 0) ready = fc.sync + 1 + fused_n + plan_first<DP>(fc, rank) / fc.slices;
  lds_barrier();
  if (wv < NS) {
    state_role(sm, sst, a, q, wv, ln);
  } else {
    lds_barrier();  // the state waves have read the staged state
    // blocks above the diagonal of P, and the zero block of T2, are read by the
    // full-width products and never written
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int i = tid - 64 * NS; i < 2 * BT * PP / 8; i += NT - 64 * NS) reinterpret_cast<u32x4*>(&sm.p[0][0])[i] = zero;
    for (int i = tid - 64 * NS; i < 3 * 16 * PB / 8; i += NT - 64 * NS) {
      const int b = i / (16 * PB / 8), e = i % (16 * PB / 8);
      reinterpret_cast<u32x4*>(&sm.t2[b][10][0])[e] = zero;
    }
    if (tid == 64 * NS) {
      sm.dflag = 0;
      sm.aflag = 0;
    }
    lds_barrier();
    if (wv == NS) gram_role(sm, a, q, lane, ln, ready, fc.slices);
    else if (wv == NS + 1) blocks_role(sm, q, ln);
    else if (wv == NS + 2) load_role(sm, a, q, lane);
    else p_role(sm, q, ln);
  }
  lds_barrier();
  {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(
        reinterpret_cast<float*>(reinterpret_cast<char*>(a.ssm_pool) +
                                 (int64_t)__builtin_amdgcn_readfirstlane(a.write_idx[q.s]) * a.ssm_stride) +
            head_off, D * D * 4);
#pragma unroll
    for (int it = 0; it < D * D / 4 / NT; ++it) {
      const int f = tid + NT * it, row = f >> 5, c4 = f & 31;
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(&sst[row * PS + 4 * c4]), rs, 16 * f, 0, 0);
    }
  }
  // streaming: this scan consumed every chunk, so every conv task of the
  // sequence (the readers of its old conv state) is done
  if constexpr (STREAM) {
    if (lead_wg) write_tail(a, q.s);
  }
}

}  // namespace

bool chunk_supported(int dk, int dv) { return dk == D && dv == D; }

// The task counters of a host-planned launch start at zero: a kernel, not a
// memset, so the call stays capturable.
hipError_t launch_zero_sync(int32_t* sync, int n, hipStream_t st) {
  if (!sync || n < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_sync_kernel, dim3(1), dim3(256), 0, st, sync, n);
  return hipGetLastError();
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
  if (a.num_seqs < 1 || a.num_seqs > kMaxPlanSeqs || !a.plan || !a.sync) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_chunk(const ScanArgs& a, const SeqOrder& order, const FusedConv& fc, int dk, int dv,
                        hipStream_t st) {
  if (!chunk_supported(dk, dv)) return hipErrorInvalidValue;
  if (fc.n > 0 && (fc.n != order.n || fc.n > kMaxFusedRanks || !fc.sync || a.width < 1 || a.width > 4))
    return hipErrorInvalidValue;
  if (fc.plan && (fc.plan_seqs != a.num_seqs || !fc.sync || a.width < 1 || a.width > 4)) return hipErrorInvalidValue;
  const int rows = fc.plan ? a.num_seqs : order.n > 0 ? order.n : a.num_seqs;
  if (fc.stream) {
    // scans wait for helpers; roles go by arrival order (a ticket), so a plain
    // launch is enough: no workgroup waits for one that has not started
    if (fc.plan || fc.n != order.n || fc.n < 1 || fc.helpers < 1 || !fc.sync) return hipErrorInvalidValue;
    const int blocks = fc.n * a.num_v_heads + fc.helpers;
    hipLaunchKernelGGL((chunk_scan_kernel<false, true>), dim3(blocks), dim3(NT), 0, st, a, order, fc);
    return hipGetLastError();
  }
  dim3 grid(rows * a.num_v_heads);
  if (fc.plan) hipLaunchKernelGGL((chunk_scan_kernel<true, false>), grid, dim3(NT), 0, st, a, order, fc);
  else hipLaunchKernelGGL((chunk_scan_kernel<false, false>), grid, dim3(NT), 0, st, a, order, fc);
  return hipGetLastError();
}

GDN_STATUS_ACCESSOR(status_chunk)

}  // namespace gdn
