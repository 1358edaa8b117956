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
// decay over 16 rows, and computed exactly in fp32 instead (kda_exact) for a
// block where that factor would leave the range of fp32.  Only differences of
// running sums are exponentiated; the tiles of the state pass take their
// factors as products of two factors <= 1 (e^{gamma_t} = e^{gamma_{16b-1}}
// e^{gamma_t - gamma_{16b-1}}, and likewise for Kh).
//
// Work split: one 512-thread workgroup (8 waves) per (sequence, value head),
// walking the chunks as a two-stage pipeline with one workgroup barrier per
// step.  In step i:
//   waves 0-3 (state)     chunk i: wave w owns d_v columns [32w, 32w+32) of the
//                         fp32 state in registers and computes Kt S, U =
//                         T2 (V - Kt S), (Qt S)^T, O^T and the state update;
//   waves 4-7 (producers) chunk i+1: wave 4+b owns the 16 rows of block b, in
//                         MFMA operand layout (lane (r, g): row 16b + r,
//                         channels 32kk + 8g .. +7), loaded from global memory
//                         one step ahead with 16-byte buffer loads; it forms the
//                         running sums within the block across the lanes of a
//                         DPP row, keeps Kb and Qb in registers as the A
//                         operands of its row of A and P blocks (its diagonal
//                         block first), writes Kr, Kt, Qt, Kh and V;
//   state wave 0          once its pass is done, T of chunk i+1: the diagonal
//                         blocks as soon as the producers have flagged theirs,
//                         the others once every block of A is in.
// The producers wait among themselves on LDS flags.  Kt, V and Qt of chunk i+1
// go into single buffers once the state waves have flagged that they have read
// chunk i's (Kt and V early in the state pass, Qt in its middle); Kh, P, T2 and
// e^{gamma_last} are double-buffered.  The barriers wait for LDS traffic only,
// so the loads of the next chunk and the output stores stay in flight across
// them.  All products are v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32
// accumulate).
#include "gdn_device.h"
#include "gdn_mfma.h"
#include "gdn_convtask.h"

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
  uint16_t kr[BT * D];         // e^{gamma_{16b+15} - gamma_t} o k_t: B side of the A and P blocks
  uint16_t kt[BT * D];         // e^{gamma_t} o k_t: K S
  uint16_t qt[BT * D];         // e^{gamma_t} o q_t: Q S
  uint16_t v[BT * D];
  uint16_t kh[2][BT * D];      // e^{gamma_last - gamma_t} o k_t: the state update, chunk parity
  uint16_t p[2][BT * PP];      // P [t][j in pair order]; blocks above the diagonal stay zero
  uint16_t t2[2][11][16 * PB]; // (T diag(b))^T as 16 x 16 blocks, and the zero block (slot 10)
  uint16_t ab[6][16 * PB];     // A^T blocks below the diagonal
  uint16_t tb[5][16 * PB];     // T^T blocks 00, 11, 22, 33 and 32
  float at[4 * 16 * PA];       // diagonal blocks of A, fp32, [block][j][t]
  float beta[BT];
  float btot[4][D];            // per block and channel: the sum of g over its rows (<= 0)
  float eoff[4][D];            // e^{gamma_{16b-1}}: Kt and Qt from the A-side factor
  float etail[4][D];           // e^{gamma_last - gamma_{16b+15}}: Kh from the B-side factor
  float fac[7][D];             // B-side channel factors: pairs (2,0), (3,1), (3,0); diagonal blocks 0..3
  float glast[2][D];           // e^{gamma_last} per channel, chunk parity
  int c1[KNS];                 // state wave w has read Kt and V of chunks < c1[w]
  int c2[KNS];                 // ... and Qt
  int pf[4];                   // producer sync counters
  int dex[4];                  // block b's diagonal is computed in fp32
  int dflag[4];                // producer wave b: its diagonal block of A is final for chunks < dflag[b]
  int aflag[4];                // ... and all its blocks of A
  int task;                    // conv tasks run by the workgroup (the conv of the rows inside this kernel)
};
static_assert(sizeof(KSmem) <= 160 * 1024, "LDS");
static_assert(offsetof(KSmem, task) >= 16 * 8 * 1024, "the conv row staging (16 rows x 8 KiB) stays clear of the task slot");
static_assert(KNT == kConvThreads, "the conv tasks assume 8 waves");
static_assert(D * KPS * 4 <= 6 * BT * D * 2, "state staging fits the first six tiles");
static_assert(16 * D * 4 <= BT * D * 2, "exact-path running sums fit the Kr tile");

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

// Inclusive prefix sum over the 16 lanes of each DPP row (the 16 rows of a block).
__device__ __forceinline__ float row_scan16(float v) {
  v += dpp_move<0x111, 0xf>(v);  // row_shr:1
  v += dpp_move<0x112, 0xf>(v);  // row_shr:2
  v += dpp_move<0x114, 0xf>(v);  // row_shr:4
  v += dpp_move<0x118, 0xf>(v);  // row_shr:8
  return v;
}

// Compiler-only ordering point: a wave's own LDS writes reach its later reads in
// program order, so cross-lane exchanges within one wave need no hardware wait.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// The four producer waves meet: every LDS write made before it by any of them
// is visible after it.
__device__ __forceinline__ void psync(KSmem& sm, int pw, int& seq) {
  ++seq;
  set_flag(&sm.pf[pw], seq);
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (w != pw) wait_flag(&sm.pf[w], seq);
}

// ---- producers: the raw rows of one 16-row block of chunk c, held in registers
// from one step to the next.  Lane (r, g): row 16 pw + r, channels 32kk + 8g .. +7
// of q, k and v (bf16) and g (fp32), and b of the row.  Rows past the sequence's
// end read as zero (g = 0, b = 0), so they change nothing.
struct KRaw {
  bf16x8 k[4], q[4], v[4];
  f32x4 g[8];  // g[2kk + h]: channels 32kk + 8g + 4h .. +3
  float beta;
};

// part: 1 = g and b, 2 = q, k and v, 3 = both
__device__ __forceinline__ void kda_load(KRaw& x, const ScanArgs& a, const KSeq& q, int c, int pw, const Lane& ln,
                                         int part) {
  const int Hv = a.num_v_heads, C = a.channels, Hk = a.num_k_heads;
  const int row0 = BT * c + 16 * pw;
  // uniform by construction; in scalar registers, so the buffer descriptors are too
  const int nv = __builtin_amdgcn_readfirstlane(max(0, min(16, q.L - row0)));
  const int64_t grow = (int64_t)q.r0 + row0;
  const __amdgpu_buffer_rsrc_t ry =
      make_rsrc(reinterpret_cast<const uint16_t*>(a.y) + grow * C, (uint32_t)(nv * C * 2));
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.g + grow * Hv * D, (uint32_t)(nv * Hv * D * 4));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.beta + grow * Hv, (uint32_t)(nv * Hv * 4));
  const int yo = ln.r * C + 8 * ln.g;
  const int go = (ln.r * Hv + q.m) * D + 8 * ln.g;
  if (part & 1) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      x.g[2 * kk] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, 4 * (go + 32 * kk), 0, 0));
      x.g[2 * kk + 1] =
          __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, 4 * (go + 32 * kk + 4), 0, 0));
    }
    x.beta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, 4 * (ln.r * Hv + q.m), 0, 0));
  }
  if (part & 2) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      x.q[kk] =
          __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ry, 2 * (yo + q.h * D + 32 * kk), 0, 0));
      x.k[kk] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ry, 2 * (yo + (Hk + q.h) * D + 32 * kk), 0, 0));
      x.v[kk] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ry, 2 * (yo + 2 * Hk * D + q.m * D + 32 * kk), 0, 0));
    }
  }
}

// ---- producers: row block bi of A and of P.  Kb and Qb of block bi come from
// registers; the B side (Kr of the blocks bj <= bi) from LDS.
// The diagonal block comes first and is flagged (when no block of the chunk takes
// the exact path), so the solver can start on it while the others are formed.
__device__ __forceinline__ void kda_pairs(KSmem& sm, int bi, const Lane& ln, const bf16x8 (&kb)[4],
                                          const bf16x8 (&qb)[4], uint16_t* pbuf, int flag_val) {
  int roff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) roff[kk] = swz_off(ln.r, 32 * kk + 8 * ln.g);
  for (int jj = 0; jj <= bi; ++jj) {
    const int bj = jj == 0 ? bi : jj - 1;
    const int fs = fac_slot(bi, bj);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, pacc = acc;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 yr = lds8(sm.kr + roff[kk] + 16 * bj * D);
      if (fs >= 0) yr = scaled8(yr, &sm.fac[fs][32 * kk + 8 * ln.g]);
      // A: lane holds A[16bi + 4g + i][16bj + r]; P transposed: P[16bi + r][16bj + 4g + i]
      acc = mfma(kb[kk], yr, acc);
      pacc = mfma(yr, qb[kk], pacc);
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
      st4bf(&pbuf[t * PP + perm(16 * bj + 4 * ln.g)], v[0], v[1], v[2], v[3]);
    }
    if (jj == 0 && flag_val > 0) set_flag(&sm.dflag[bi], flag_val);
  }
}

// ---- producers (only for a diagonal block whose own decay leaves the fp32
// range): its A and P entries from the channel sums themselves, with every
// e^{gamma_t - gamma_j} formed from the difference of running sums (<= 0).
// Block b's running sums (relative to the row before it) are first put over the
// Kr tile, which the A and P blocks no longer read.  tp: producer thread 0..255.
__device__ void kda_exact(KSmem& sm, const ScanArgs& a, const KSeq& q, int chunk, int b, int tp, int pw,
                          uint16_t* pbuf, int& seq) {
  const int Hv = a.num_v_heads, C = a.channels, Hk = a.num_k_heads;
  const int64_t rb = (int64_t)q.r0 + chunk * BT + 16 * b;
  const int nv = max(0, min(16, q.L - chunk * BT - 16 * b));
  const uint16_t* y = reinterpret_cast<const uint16_t*>(a.y);
  float* gex = reinterpret_cast<float*>(sm.kr);
  if (tp < D) {
    float acc = 0.f;
    for (int i = 0; i < 16; ++i) {
      if (i < nv) acc += a.g[((rb + i) * Hv + q.m) * D + tp];
      gex[i * D + tp] = acc;
    }
  }
  psync(sm, pw, seq);
  // 136 pairs (j <= t) x 4 channel quarters; the quarters of a pair are adjacent lanes
  for (int w = tp; w < 136 * 4; w += 256) {
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
        const float e = __expf(gex[t * D + c] - gex[j * D + c]);
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
      pbuf[tt * PP + perm(jj)] = f32_to_bf16_bits(sp);
    }
  }
  psync(sm, pw, seq);  // gex is free again; the exact entries are written
}

// ---- producers: everything the state pass of chunk c reads.  pw: producer wave
// 0..3 (its block); x: the raw rows of chunk c, replaced by those of chunk c + 1.
__device__ __forceinline__ void kda_produce(KSmem& sm, const ScanArgs& a, const KSeq& q, int c, int pw,
                                            const Lane& ln, KRaw& x, int& seq) {
  const int lane = 16 * ln.g + ln.r, par = c & 1;
  // running sums of g within the block (in place), block totals, b
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) x.g[j][e] = row_scan16(x.g[j][e]);
  bool big = false;
  if (ln.r == 15) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      *reinterpret_cast<f32x4*>(&sm.btot[pw][32 * (j >> 1) + 8 * ln.g + 4 * (j & 1)]) = x.g[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) big = big || (-x.g[j][e] > kMaxGrowth);
    }
  }
  if (ln.g == 0) sm.beta[16 * pw + ln.r] = x.beta;
  const bool dex_own = __builtin_amdgcn_ballot_w64(big) != 0;
  if (lane == 0) sm.dex[pw] = dex_own ? 1 : 0;
  psync(sm, pw, seq);  // every block's totals
  // per-channel factors of this block, two channels per lane
  {
    const int ch = 2 * lane;
    float2 t[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) t[b] = *reinterpret_cast<const float2*>(&sm.btot[b][ch]);
    float off0 = 0.f, off1 = 0.f, gl0 = 0.f, gl1 = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < pw) {
        off0 += t[b].x;
        off1 += t[b].y;
      }
      gl0 += t[b].x;
      gl1 += t[b].y;
    }
    const float2 own = *reinterpret_cast<const float2*>(&sm.btot[pw][ch]);
    *reinterpret_cast<float2*>(&sm.eoff[pw][ch]) = make_float2(__expf(off0), __expf(off1));
    *reinterpret_cast<float2*>(&sm.etail[pw][ch]) =
        make_float2(__expf(gl0 - off0 - own.x), __expf(gl1 - off1 - own.y));
    *reinterpret_cast<float2*>(&sm.fac[3 + pw][ch]) =
        make_float2(__expf(fminf(-own.x, kMaxGrowth)), __expf(fminf(-own.y, kMaxGrowth)));
    if (pw == 0) *reinterpret_cast<float2*>(&sm.glast[par][ch]) = make_float2(__expf(gl0), __expf(gl1));
    if (pw == 2) *reinterpret_cast<float2*>(&sm.fac[0][ch]) = make_float2(__expf(t[1].x), __expf(t[1].y));
    if (pw == 3) {
      *reinterpret_cast<float2*>(&sm.fac[1][ch]) = make_float2(__expf(t[2].x), __expf(t[2].y));
      *reinterpret_cast<float2*>(&sm.fac[2][ch]) = make_float2(__expf(t[1].x + t[2].x), __expf(t[1].y + t[2].y));
    }
  }
  lds_order();
  // the tiles of the block's rows (Kt, V and Qt once every state wave has read
  // chunk c - 1's: in the state pass both flags come well before this point)
#pragma unroll
  for (int w = 0; w < KNS; ++w) wait_flag(&sm.c1[w], c);
#pragma unroll
  for (int w = 0; w < KNS; ++w) wait_flag(&sm.c2[w], c);
  bf16x8 kb[4], qb[4];
  const int row = 16 * pw + ln.r;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int cb = 32 * kk + 8 * ln.g;
    const f32x4 tot[2] = {*reinterpret_cast<const f32x4*>(&sm.btot[pw][cb]),
                          *reinterpret_cast<const f32x4*>(&sm.btot[pw][cb + 4])};
    const f32x4 eo[2] = {*reinterpret_cast<const f32x4*>(&sm.eoff[pw][cb]),
                         *reinterpret_cast<const f32x4*>(&sm.eoff[pw][cb + 4])};
    const f32x4 et[2] = {*reinterpret_cast<const f32x4*>(&sm.etail[pw][cb]),
                         *reinterpret_cast<const f32x4*>(&sm.etail[pw][cb + 4])};
    bf16x8 kr, kh, kt, qt;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float gm = x.g[2 * kk + (e >> 2)][e & 3];
      const float e1 = __expf(gm);                        // e^{gamma_t - gamma_{16b-1}}
      const float e2 = __expf(tot[e >> 2][e & 3] - gm);   // e^{gamma_{16b+15} - gamma_t}
      const float e3 = e1 * eo[e >> 2][e & 3];            // e^{gamma_t}
      const float e4 = e2 * et[e >> 2][e & 3];            // e^{gamma_last - gamma_t}
      const float kv = (float)x.k[kk][e], qv = (float)x.q[kk][e];
      kb[kk][e] = (__bf16)(kv * e1);
      qb[kk][e] = (__bf16)(qv * e1);
      kr[e] = (__bf16)(kv * e2);
      kt[e] = (__bf16)(kv * e3);
      qt[e] = (__bf16)(qv * e3);
      kh[e] = (__bf16)(kv * e4);
    }
    const int o = swz_off(row, cb);
    *reinterpret_cast<bf16x8*>(&sm.kr[o]) = kr;
    *reinterpret_cast<bf16x8*>(&sm.kh[par][o]) = kh;
    *reinterpret_cast<bf16x8*>(&sm.kt[o]) = kt;
    *reinterpret_cast<bf16x8*>(&sm.v[o]) = x.v[kk];
    *reinterpret_cast<bf16x8*>(&sm.qt[o]) = qt;
  }
  psync(sm, pw, seq);  // Kr of every block
  const int ex = sm.dex[0] | (sm.dex[1] << 1) | (sm.dex[2] << 2) | (sm.dex[3] << 3);  // uniform
  kda_pairs(sm, pw, ln, kb, qb, sm.p[par], ex ? 0 : c + 1);
  if (ex) {
    psync(sm, pw, seq);  // the A and P blocks no longer read Kr
    for (int b = 0; b < 4; ++b)
      if (ex & (1 << b)) kda_exact(sm, a, q, c, b, 64 * pw + lane, pw, sm.p[par], seq);
    set_flag(&sm.dflag[pw], c + 1);
  }
  set_flag(&sm.aflag[pw], c + 1);  // the solver (state wave 0) takes it from here
  // the next chunk's rows, at the end of the step (not before this point: the
  // compiler would hold both chunks' rows at once); a wave stalls while it
  // issues these loads (each touches 16 rows), so they stay off the path to
  // the A blocks
  lds_order();
  if (c + 1 < q.N) kda_load(x, a, q, c + 1, pw, ln, 3);
}

// ---- T = (I + A)^-1 of chunk c by state wave 0, once its state pass is done:
// the diagonal blocks as soon as every producer has flagged its own, the blocks
// below them once every block of A is in (written as T2 = (T diag(b))^T).
__device__ __forceinline__ void kda_solve(KSmem& sm, int c, int lane, const Lane& ln) {
#pragma unroll
  for (int w = 0; w < 4; ++w) wait_flag(&sm.dflag[w], c + 1);
  uint16_t* t2 = &sm.t2[c & 1][0][0];
  solve_diag(sm.at, sm.tb, t2, sm.beta, lane);
#pragma unroll
  for (int w = 0; w < 4; ++w) wait_flag(&sm.aflag[w], c + 1);
  solve_blocks(sm.ab, sm.tb, t2, sm.beta, ln);
}

// ---- the state pass of one chunk for d_v columns [32 wv, 32 wv + 32)
// (the arithmetic of the gated-delta-rule state pass with the decays in the tiles).
struct StateLanes {
  int roff[4], toff[4][2], voffs[KNB], col[KNB], t2off, poff, olane;
};

__device__ __forceinline__ void kda_state_step(KSmem& sm, f32x4 (&sacc)[8][KNB], const StateLanes& sl,
                                               const ScanArgs& a, const KSeq& q, int chunk, const Lane& ln, int wv) {
  const int lg = ln.g, par = chunk & 1;
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
  set_flag(&sm.c1[wv], chunk + 1);  // Kt and V of this chunk are read
  const uint16_t* t2 = &sm.t2[par][0][0];
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
      const bf16x8 a2 = cat(ldtr(t2 + t2_slot(tb, 2 * kk) * 16 * PB + sl.t2off),
                            ldtr(t2 + t2_slot(tb, 2 * kk + 1) * 16 * PB + sl.t2off));
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
  set_flag(&sm.c2[wv], chunk + 1);  // Qt of this chunk is read
  const uint16_t* pb = sm.p[par];
  bf16x8 ub[2][KNB];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) ub[k2][nb] = pair_operand(u[2 * k2][nb], u[2 * k2 + 1][nb]);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int tb = 2 * kk; tb < 4; ++tb) {
      const bf16x8 pa = lds8(pb + sl.poff + 16 * tb * PP + 32 * kk);
#pragma unroll
      for (int nb = 0; nb < KNB; ++nb) ot[nb][tb] = mfma(ub[kk][nb], pa, ot[nb][tb]);
    }
  // ---- S <- diag(e^{gamma_last}) S + Kh^T U (register row d holds state row sigma(d))
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const f32x4 f = *reinterpret_cast<const f32x4*>(&sm.glast[par][sigma(16 * db + 4 * lg)]);
#pragma unroll
    for (int nb = 0; nb < KNB; ++nb) sacc[db][nb] *= f;
  }
  const uint16_t* kh = sm.kh[par];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    fence();
    bf16x8 kt[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint16_t* src = kh + sl.toff[db >> 1][db & 1] + 32 * half * D;
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

// fc.n > 0: the conv of the rows runs inside the kernel, as tasks every
// workgroup claims before its scan (gdn_convtask.h); the producers then wait
// for each chunk's rows before they load them.
__global__ __launch_bounds__(KNT) void kda_chunk_kernel(ScanArgs a, SeqOrder ord, FusedConv fc) {
  __shared__ KSmem sm;
  const int Hv = a.num_v_heads;
  const int rank = blockIdx.x / Hv;
  KSeq q;
  q.m = blockIdx.x % Hv;
  const int32_t* ready = nullptr;  // the chunk counters of the sequence, with the conv inside
  if (fc.n > 0) {
    conv_phase_w<false>(sm, a, ord, fc, rank);
    ready = fc.sync + 1 + fc.n + fc.first[rank] / fc.slices;
    // value heads of one key head on one XCD (workgroups go round-robin over
    // the 8 XCDs), so the second reader of the shared q and k rows can hit L2
    const int g = Hv / a.num_k_heads, per = Hv / 8;
    if (Hv % 8 == 0 && per % g == 0) {
      const int x = q.m % 8, sl = q.m / 8;
      q.m = g * (x * (per / g) + sl / g) + sl % g;
    }
  }
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
  float* sst = reinterpret_cast<float*>(&sm.kr[0]);
  const int64_t head_off = (int64_t)q.m * D * D;
  {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(
        reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.ssm_pool) +
                                       (int64_t)__builtin_amdgcn_readfirstlane(a.read_idx[q.s]) * a.ssm_stride) +
            head_off, D * D * 4);
#pragma unroll
    for (int it = 0; it < D * D / 4 / KNT; ++it) {
      const int f = tid + KNT * it, row = f >> 5, c4 = f & 31;
      *reinterpret_cast<u32x4*>(&sst[row * KPS + 4 * c4]) = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * f, 0, 0);
    }
  }
  // the zero blocks of T2 and the P blocks above the diagonal are read by the
  // full-width products and never written (they lie outside the staging area)
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int i = tid; i < 2 * BT * PP / 8; i += KNT) reinterpret_cast<u32x4*>(&sm.p[0][0])[i] = zero;
    for (int i = tid; i < 2 * 16 * PB / 8; i += KNT)
      reinterpret_cast<u32x4*>(&sm.t2[i / (16 * PB / 8)][10][0])[i % (16 * PB / 8)] = zero;
    if (tid < KNS) {
      sm.c1[tid] = 0;
      sm.c2[tid] = 0;
      sm.pf[tid] = 0;
      sm.dflag[tid] = 0;
      sm.aflag[tid] = 0;
    }
  }
  __syncthreads();
  // Per step, one workgroup barrier: the state waves run chunk i while the
  // producers prepare chunk i + 1 (step -1: chunk 0 alone).
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
    lds_barrier();  // the staged state has been read
    if (wv == 0) kda_solve(sm, 0, lane, ln);
    lds_barrier();  // step -1
    for (int c = 0; c < q.N; ++c) {
      kda_state_step(sm, sacc, sl, a, q, c, ln, wv);
      if (wv == 0 && c + 1 < q.N) {
        // the solve's lane addresses are formed here each step (hoisted out of
        // the loop they would push the state wave's registers into scratch)
        int l = lane;
        asm volatile("" : "+v"(l));
        kda_solve(sm, c + 1, l, Lane{l & 15, l >> 4, l & 3, (l >> 2) & 3});
      }
      lds_barrier();  // step c
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int nb = 0; nb < KNB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sst[sigma(16 * db + 4 * lg + i) * KPS + sl.col[nb]] = sacc[db][nb][i];
  } else {
    // ---- producer waves
    const int pw = wv - KNS;
    KRaw x;
    int upto = 0;  // chunks below this one are known to be converted
    if (ready) upto = chunk_wait(ready, fc.slices, q.L, 0, upto, lane);
    kda_load(x, a, q, 0, pw, ln, 3);
    int seq = 0;
    lds_barrier();  // the state waves have read the staged state
    for (int c = 0; c < q.N; ++c) {
      // the rows of chunk c + 1, loaded at the end of this step
      if (ready && c + 1 < q.N) upto = chunk_wait(ready, fc.slices, q.L, c + 1, upto, lane);
      // the lane's addresses are recomputed every step: hoisted out of the
      // loop, they would not fit the registers beside the rows and operands
      int l = lane, w = pw;
      asm volatile("" : "+v"(l), "+s"(w));
      kda_produce(sm, a, q, c, w, Lane{l & 15, l >> 4, l & 3, (l >> 2) & 3}, x, seq);
      lds_barrier();  // step c - 1
    }
    lds_barrier();  // step N - 1
  }
  __syncthreads();
  {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(
        reinterpret_cast<float*>(reinterpret_cast<char*>(a.ssm_pool) +
                                 (int64_t)__builtin_amdgcn_readfirstlane(a.write_idx[q.s]) * a.ssm_stride) +
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

hipError_t launch_kda_chunk(const ScanArgs& a, const SeqOrder& order, const FusedConv& fc, hipStream_t st) {
  if (!kda_chunk_supported(D, D) || !a.y) return hipErrorInvalidValue;
  if (fc.n > 0 && (fc.n != order.n || fc.n > kMaxFusedRanks || !fc.sync || fc.plan || fc.stream || a.width < 1 ||
                   a.width > 4 || fc.slices < 1))
    return hipErrorInvalidValue;
  const int rows = order.n > 0 ? order.n : a.num_seqs;
  hipLaunchKernelGGL(kda_chunk_kernel, dim3(rows * a.num_v_heads), dim3(KNT), 0, st, a, order, fc);
  return hipGetLastError();
}

GDN_STATUS_ACCESSOR(status_kda)

}  // namespace gdn
