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
//     W  = T diag(b Gamma) K,   U~ = T diag(b) V,   U = U~ - W S
//     O  = diag(Gamma) Q S + (M o Q K^T) U,   M_tj = e^{gamma_t-gamma_j} (j <= t)
//     S <- Gamma_c S + K^T diag(e^{gamma_c-gamma}) U
// Only differences of running sums are exponentiated, so every factor is <= 1.
//
// Work split: one 256-thread workgroup (4 waves) per (sequence, value head,
// 64-wide slice of d_v); it walks the sequence's chunks in order with its
// 128 x 64 fp32 state slice in registers (the columns of S evolve
// independently, so slicing d_v is exact).  All products are
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation; operands are bf16 tiles in
// LDS.  T is built from fp32 forward substitution on its four 16x16 diagonal
// blocks and two levels of block products for the rest.  W is kept in
// registers between the product that makes it and the one that uses it: its
// accumulator rows are exactly the A operand rows the next product needs,
// taken in a permuted k order (the MFMA sums over k, so any order shared by both
// operands gives the same result).
//
// MFMA 16x16x32 bf16 operand layout (lane l, r = l & 15, grp = l >> 4):
//   A: row r, 8 values of k;  B: column r, the same 8 values of k;
//   D: column r, rows 4*grp + {0,1,2,3}.
#include "gdn_device.h"

namespace gdn {
namespace {

constexpr int BT = 64;    // chunk length
constexpr int D = 128;    // d_k = d_v
constexpr int NS = 64;    // d_v columns per workgroup
constexpr int PQ = D + 8; // LDS pitch (elements) of [*][128] bf16 tiles
constexpr int PT = BT + 8;// LDS pitch of [*][64] bf16 tiles
constexpr int PY = 40;    // LDS pitch of the [*][32] temporaries
constexpr int PA = 17;    // fp32 pitch of the diagonal blocks of A

struct alignas(16) Smem {
  uint16_t q[BT * PQ];        // Q rows [t][d]
  uint16_t k[BT * PQ];        // K rows [t][d]
  uint16_t kt[D * PT];        // K^T [d][t]
  uint16_t vt[NS * PT];       // V^T slice [n][t]
  uint16_t st[NS * PQ];       // S^T slice [n][d] (bf16 operand copy of the state)
  uint16_t p[BT * PT];        // M o Q K^T [t][j]
  uint16_t t1[BT * PT];       // T diag(b Gamma) [t][j]
  uint16_t t2[BT * PT];       // T diag(b) [t][j]
  union {
    uint16_t ab[BT * PT];     // A, off-diagonal blocks, bf16 [t][j] (T solve)
    uint16_t ut[NS * PT];     // U^T [n][t] (state pass)
  } u;
  uint16_t tr[BT * PT];       // T bf16 [t][j]; its upper blocks stay zero
  uint16_t upt[NS * PT];      // (diag(e^{gamma_c-gamma}) U)^T [n][t]
  uint16_t tt[BT * PT];       // T^T bf16 [j][t]
  uint16_t yt[BT * PY];       // transposed temporaries of the block products
  float af[4 * 16 * PA];      // diagonal blocks of A, fp32
  float gam[BT];              // running sum of g inside the chunk
  float beta[BT];
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// 4 + 4 values from two 8-byte halves (the permuted k order).
__device__ __forceinline__ bf16x8 lds4x2(const uint16_t* p0, const uint16_t* p1) {
  bf16x4 lo = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 hi = *reinterpret_cast<const bf16x4*>(p1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// k values 8*grp..8*grp+7 of a 16-deep product padded to 32 (groups 2, 3 give zero).
__device__ __forceinline__ bf16x8 lds8_k16(const uint16_t* p, int grp) {
  if (grp < 2) return lds8(p);
  bf16x8 z = {};
  return z;
}

__device__ __forceinline__ uint16_t bfbits(float f) { return f32_to_bf16_bits(f); }

__device__ __forceinline__ void st4bf(uint16_t* p, float a, float b, float c, float d) {
  uint2 u;
  u.x = (uint32_t)bfbits(a) | ((uint32_t)bfbits(b) << 16);
  u.y = (uint32_t)bfbits(c) | ((uint32_t)bfbits(d) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

__device__ __forceinline__ __bf16 tobf(float f) {
  uint16_t b = bfbits(f);
  return __builtin_bit_cast(__bf16, b);
}

__global__ __launch_bounds__(256) void chunk_scan_kernel(ScanArgs a) {
  __shared__ Smem sm;
  constexpr int NSL = D / NS;
  const int bid = blockIdx.x;
  const int slice = bid % NSL;
  const int m = (bid / NSL) % a.num_v_heads;
  const int s = bid / (NSL * a.num_v_heads);
  if (s >= a.num_seqs) return;
  const int r0 = a.cu[s];
  const int L = a.cu[s + 1] - r0;
  if (L < a.min_len || L > a.max_len) return;
  if (!seq_active(a.read_idx, a.write_idx, s, a.num_blocks)) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int h = m / (a.num_v_heads / a.num_k_heads);
  const int n0 = slice * NS;
  const int64_t C = a.channels;
  const int64_t qoff = (int64_t)h * D, koff = (int64_t)a.num_k_heads * D + h * D;
  const int64_t voff = 2 * (int64_t)a.num_k_heads * D + (int64_t)m * D + n0;
  const int64_t head_off = (int64_t)m * D * D;
  const uint16_t* Y = reinterpret_cast<const uint16_t*>(a.y);
  uint16_t* OUT = reinterpret_cast<uint16_t*>(a.out);

  // blocks above the diagonal of T, T diag(.) and P stay zero for the whole run
  for (int i = tid; i < BT * PT; i += 256) {
    sm.t1[i] = 0; sm.t2[i] = 0; sm.p[i] = 0; sm.tt[i] = 0;
    sm.tr[i] = 0;
  }

  // state slice: wave w holds rows d in [32w, 32w+32) as two 16-row blocks
  f32x4 sacc[2][4];
  {
    const float* S0 = reinterpret_cast<const float*>(
        reinterpret_cast<const char*>(a.ssm_pool) + (int64_t)a.read_idx[s] * a.ssm_stride) + head_off;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 32 * w + 16 * db + 4 * lg + i;
          sacc[db][cb][i] = S0[(int64_t)d * D + n0 + 16 * cb + li];
        }
  }
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      st4bf(&sm.st[(16 * cb + li) * PQ + 32 * w + 16 * db + 4 * lg], sacc[db][cb][0], sacc[db][cb][1],
            sacc[db][cb][2], sacc[db][cb][3]);
  __syncthreads();

  for (int c0 = 0; c0 < L; c0 += BT) {
    const int nv = min(BT, L - c0);
    const int64_t rbase = r0 + c0;

    // ---- load Q, K (rows and K^T), V^T slice, g, beta; rows past the end are zero
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int t = (tid >> 4) + 16 * it, c8 = tid & 15;
      uint4 qv = make_uint4(0, 0, 0, 0), kv = qv;
      if (t < nv) {
        qv = *reinterpret_cast<const uint4*>(Y + (rbase + t) * C + qoff + 8 * c8);
        kv = *reinterpret_cast<const uint4*>(Y + (rbase + t) * C + koff + 8 * c8);
      }
      *reinterpret_cast<uint4*>(&sm.q[t * PQ + 8 * c8]) = qv;
      *reinterpret_cast<uint4*>(&sm.k[t * PQ + 8 * c8]) = kv;
      const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.kt[(8 * c8 + 2 * e) * PT + t] = (uint16_t)(kw[e] & 0xffff);
        sm.kt[(8 * c8 + 2 * e + 1) * PT + t] = (uint16_t)(kw[e] >> 16);
      }
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int t = (tid >> 3) + 32 * it, c8 = tid & 7;
      uint4 vv = make_uint4(0, 0, 0, 0);
      if (t < nv) vv = *reinterpret_cast<const uint4*>(Y + (rbase + t) * C + voff + 8 * c8);
      const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.vt[(8 * c8 + 2 * e) * PT + t] = (uint16_t)(vw[e] & 0xffff);
        sm.vt[(8 * c8 + 2 * e + 1) * PT + t] = (uint16_t)(vw[e] >> 16);
      }
    }
    if (w == 0) {
      float gv = 0.f, bv = 0.f;
      if (lane < nv) {
        gv = a.g[(rbase + lane) * a.num_v_heads + m];
        bv = a.beta[(rbase + lane) * a.num_v_heads + m];
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(gv, off);
        if (lane >= off) gv += o;
      }
      sm.gam[lane] = gv;
      sm.beta[lane] = bv;
    }
    __syncthreads();

    // ---- Gram products: K K^T -> A (lower blocks), Q K^T -> P (lower blocks)
#pragma unroll
    for (int e = w; e < 20; e += 4) {
      const int pair = e % 10;
      const int bi = pair == 0 ? 0 : pair < 3 ? 1 : pair < 6 ? 2 : 3;
      const int bj = pair - (bi * (bi + 1)) / 2;
      const bool isq = e >= 10;
      const uint16_t* arow = (isq ? sm.q : sm.k) + (16 * bi + li) * PQ;
      const uint16_t* brow = sm.k + (16 * bj + li) * PQ;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = mfma(lds8(arow + 32 * kk + 8 * lg), lds8(brow + 32 * kk + 8 * lg), acc);
      const int j = 16 * bj + li;
      const float gj = sm.gam[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * bi + 4 * lg + i;
        const float gt = sm.gam[t];
        if (isq) {
          const float v = (j <= t) ? __expf(gt - gj) * acc[i] : 0.f;
          sm.p[t * PT + j] = bfbits(v);
        } else {
          const float v = (j < t) ? sm.beta[t] * __expf(gt - gj) * acc[i] : 0.f;
          if (bi == bj) sm.af[(bi * 16 + 4 * lg + i) * PA + li] = v;
          else sm.u.ab[t * PT + j] = bfbits(v);
        }
      }
    }
    __syncthreads();

    // ---- T = (I + A)^-1, diagonal blocks: fp32 forward substitution, wave w -> block w
    {
      const int c = li;
      const float* ab = &sm.af[(w * 16) * PA];
      float tc[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        float v = (t == c) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < t; ++j) v -= ab[t * PA + j] * tc[j];
        tc[t] = v;
      }
      const int cg = 16 * w + c;
      const float bc = sm.beta[cg];
      const float bgc = bc * __expf(sm.gam[cg]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tl = 4 * lg + i, tg = 16 * w + tl;
        const float v = tc[tl];
        sm.tr[tg * PT + cg] = bfbits(v);
        sm.t1[tg * PT + cg] = bfbits(v * bgc);
        sm.t2[tg * PT + cg] = bfbits(v * bc);
      }
      st4bf(&sm.tt[cg * PT + 16 * w + 4 * lg], tc[4 * lg], tc[4 * lg + 1], tc[4 * lg + 2], tc[4 * lg + 3]);
    }
    __syncthreads();

    // ---- first-level blocks: T10 = -T11 A10 T00 (wave 0), T32 = -T33 A32 T22 (wave 1)
    if (w < 2) {
      const int rb = 16 * (2 * w + 1), cbk = 16 * (2 * w);  // row block, column block
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      y = mfma(lds8_k16(&sm.u.ab[(rb + li) * PT + cbk + 8 * lg], lg),
               lds8_k16(&sm.tt[(cbk + li) * PT + cbk + 8 * lg], lg), y);
      st4bf(&sm.yt[(16 * w + li) * PY + 4 * lg], y[0], y[1], y[2], y[3]);
    }
    __syncthreads();
    if (w < 2) {
      const int rb = 16 * (2 * w + 1), cbk = 16 * (2 * w);
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
      t = mfma(lds8_k16(&sm.tr[(rb + li) * PT + rb + 8 * lg], lg),
               lds8_k16(&sm.yt[(16 * w + li) * PY + 8 * lg], lg), t);
      const int cg = cbk + li;
      const float bc = sm.beta[cg];
      const float bgc = bc * __expf(sm.gam[cg]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tg = rb + 4 * lg + i;
        const float v = -t[i];
        sm.tr[tg * PT + cg] = bfbits(v);
        sm.t1[tg * PT + cg] = bfbits(v * bgc);
        sm.t2[tg * PT + cg] = bfbits(v * bc);
      }
      st4bf(&sm.tt[cg * PT + rb + 4 * lg], -t[0], -t[1], -t[2], -t[3]);
    }
    __syncthreads();

    // ---- second level: T[32:64, 0:32] = -T_BB (A_BA T_AA), one 16x16 tile per wave
    {
      const int tr_ = 2 + (w >> 1), tc_ = w & 1;
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      y = mfma(lds8(&sm.u.ab[(16 * tr_ + li) * PT + 8 * lg]),
               lds8(&sm.tt[(16 * tc_ + li) * PT + 8 * lg]), y);
      st4bf(&sm.yt[(32 + 16 * tc_ + li) * PY + 16 * (tr_ - 2) + 4 * lg], y[0], y[1], y[2], y[3]);
    }
    __syncthreads();
    {
      const int tr_ = 2 + (w >> 1), tc_ = w & 1;
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
      t = mfma(lds8(&sm.tr[(16 * tr_ + li) * PT + 32 + 8 * lg]),
               lds8(&sm.yt[(32 + 16 * tc_ + li) * PY + 8 * lg]), t);
      const int cg = 16 * tc_ + li;
      const float bc = sm.beta[cg];
      const float bgc = bc * __expf(sm.gam[cg]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tg = 16 * tr_ + 4 * lg + i;
        sm.t1[tg * PT + cg] = bfbits(-t[i] * bgc);
        sm.t2[tg * PT + cg] = bfbits(-t[i] * bc);
      }
    }
    __syncthreads();

    // ---- W^T = K^T (T diag(b Gamma))^T for rows t of block w, kept as A operands;
    //      U~ = T diag(b) V for rows t of block w, in the U accumulators
    bf16x8 wa[4];
    f32x4 uacc[4];
    {
      f32x4 wacc[8];
#pragma unroll
      for (int db = 0; db < 8; ++db) wacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int nk = (w < 2) ? 1 : 2;
      for (int kk = 0; kk < nk; ++kk) {
        const bf16x8 bt = lds8(&sm.t1[(16 * w + li) * PT + 32 * kk + 8 * lg]);
#pragma unroll
        for (int db = 0; db < 8; ++db)
          wacc[db] = mfma(lds8(&sm.kt[(16 * db + li) * PT + 32 * kk + 8 * lg]), bt, wacc[db]);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = tobf(-wacc[2 * kk][i]);
          v[4 + i] = tobf(-wacc[2 * kk + 1][i]);
        }
        wa[kk] = v;
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) uacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int kk = 0; kk < nk; ++kk) {
        const bf16x8 at = lds8(&sm.t2[(16 * w + li) * PT + 32 * kk + 8 * lg]);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          uacc[cb] = mfma(at, lds8(&sm.vt[(16 * cb + li) * PT + 32 * kk + 8 * lg]), uacc[cb]);
      }
    }

    // ---- U = U~ - W S  and  Q S  (rows t of block w, all 64 columns of the slice)
    f32x4 oacc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) oacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint16_t* qrow = &sm.q[(16 * w + li) * PQ + 32 * kk + 4 * lg];
      const bf16x8 qa = lds4x2(qrow, qrow + 16);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const uint16_t* srow = &sm.st[(16 * cb + li) * PQ + 32 * kk + 4 * lg];
        const bf16x8 bs = lds4x2(srow, srow + 16);
        uacc[cb] = mfma(wa[kk], bs, uacc[cb]);
        oacc[cb] = mfma(qa, bs, oacc[cb]);
      }
    }
    const float glast = sm.gam[BT - 1];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      float dec[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * w + 4 * lg + i;
        const float gt = sm.gam[t];
        dec[i] = __expf(glast - gt);
        oacc[cb][i] *= __expf(gt);
      }
      uint16_t* ut = &sm.u.ut[(16 * cb + li) * PT + 16 * w + 4 * lg];
      st4bf(ut, uacc[cb][0], uacc[cb][1], uacc[cb][2], uacc[cb][3]);
      uint16_t* upt = &sm.upt[(16 * cb + li) * PT + 16 * w + 4 * lg];
      st4bf(upt, uacc[cb][0] * dec[0], uacc[cb][1] * dec[1], uacc[cb][2] * dec[2], uacc[cb][3] * dec[3]);
    }
    __syncthreads();

    // ---- O += P U ; write the chunk's output rows
    {
      const int nk = (w < 2) ? 1 : 2;
      for (int kk = 0; kk < nk; ++kk) {
        const bf16x8 pa = lds8(&sm.p[(16 * w + li) * PT + 32 * kk + 8 * lg]);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          oacc[cb] = mfma(pa, lds8(&sm.u.ut[(16 * cb + li) * PT + 32 * kk + 8 * lg]), oacc[cb]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * w + 4 * lg + i;
        if (t < nv) {
          uint16_t* orow = OUT + ((rbase + t) * a.num_v_heads + m) * D + n0 + li;
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) orow[16 * cb] = bfbits(oacc[cb][i]);
        }
      }
    }

    // ---- S <- Gamma_c S + K^T U'
    {
      const float gc = __expf(glast);
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) sacc[db][cb] *= gc;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const bf16x8 ka = lds8(&sm.kt[(32 * w + 16 * db + li) * PT + 32 * kk + 8 * lg]);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            sacc[db][cb] = mfma(ka, lds8(&sm.upt[(16 * cb + li) * PT + 32 * kk + 8 * lg]), sacc[db][cb]);
        }
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          st4bf(&sm.st[(16 * cb + li) * PQ + 32 * w + 16 * db + 4 * lg], sacc[db][cb][0], sacc[db][cb][1],
                sacc[db][cb][2], sacc[db][cb][3]);
    }
    __syncthreads();
  }

  {
    float* S1 = reinterpret_cast<float*>(
        reinterpret_cast<char*>(a.ssm_pool) + (int64_t)a.write_idx[s] * a.ssm_stride) + head_off;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 32 * w + 16 * db + 4 * lg + i;
          S1[(int64_t)d * D + n0 + 16 * cb + li] = sacc[db][cb][i];
        }
  }
}

}  // namespace

bool chunk_supported(int dk, int dv) { return dk == D && dv == D; }

hipError_t launch_chunk(const ScanArgs& a, int dk, int dv, hipStream_t st) {
  if (!chunk_supported(dk, dv)) return hipErrorInvalidValue;
  dim3 grid(a.num_seqs * a.num_v_heads * (D / NS));
  hipLaunchKernelGGL(chunk_scan_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace gdn
