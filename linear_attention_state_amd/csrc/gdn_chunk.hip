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
// Work split: one 256-thread workgroup (4 waves, one per SIMD) per (sequence,
// value head); it walks the sequence's chunks in order.  Wave w owns the d_v
// columns [32w, 32w+32) of the 128 x 128 fp32 state, held in its registers.
// The columns of S evolve independently, so the state pass of a chunk
// (U = U~ - W S, O, S update) is local to each wave: S, U and O stay in
// registers and only the shared operands W, Q, P, K^T come from LDS.  The
// chunk preparation (Gram products, T, W, P) is shared by all waves through
// LDS.  All products are v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32
// accumulate).  T comes from fp32 forward substitution on its four 16x16
// diagonal blocks (column-oriented, so each step's updates are independent)
// and two levels of block products.  The next chunk's K, V, Q, g, beta are
// loaded into registers while the current chunk computes and staged in LDS at
// the top of the next iteration; global pointers are address space 1 and the
// workgroup barriers wait for LDS traffic only, so those loads and the output
// stores stay in flight across them.  Sequences are launched longest first.
//
// MFMA 16x16x32 bf16 operand layout (lane l, r = l & 15, grp = l >> 4):
//   A: row r, 8 values of k;  B: column r, the same 8 values of k;
//   D: column r, rows 4*grp + {0,1,2,3}.
// The MFMA sums over k, so any k order shared by both operands gives the same
// product; "permuted" operands below take k = {4grp..4grp+3, 16+4grp..16+4grp+3}
// of each 32-wide step, which is what a D tile pair holds.
#include "gdn_device.h"

namespace gdn {
namespace {

constexpr int BT = 64;     // chunk length
constexpr int D = 128;     // d_k = d_v
constexpr int PQ = D + 8;  // LDS pitch (elements) of [*][128] bf16 tiles
constexpr int PT = BT + 8; // LDS pitch of [*][64] bf16 tiles
constexpr int PY = 40;     // LDS pitch of the [*][32] temporaries
constexpr int PA = 20;     // fp32 pitch of the transposed diagonal blocks of A
constexpr int PS = D + 4;  // fp32 pitch of the staged state

struct alignas(16) Smem {
  uint16_t q[BT * PQ];        // Q rows [t][d]
  union {
    uint16_t k[BT * PQ];      // K rows [t][d] (Gram products)
    uint16_t w[BT * PQ];      // -W rows [t][d] (state pass)
  } kw;
  union {
    struct {
      uint16_t kt[D * PT];    // K^T [d][t ^ swz(d)]
      uint16_t vt[D * PT];    // (diag(b) V)^T [n][t ^ swz(n)]
      uint16_t p[BT * PT];    // P = M o Q K^T [t][j]; blocks above the diagonal stay zero
      uint16_t t1[BT * PT];   // T diag(b Gamma) [t][j]; blocks above the diagonal stay zero
      uint16_t tr[BT * PT];   // T [t][j]
      uint16_t tt[BT * PT];   // T^T [j][t]
    };
    float sst[D * PS];        // the fp32 state [d][n], staged at the start and the end
  };
  uint16_t ab[BT * PT];       // A, off-diagonal blocks [t][j]
  uint16_t yt[BT * PY];       // transposed temporaries of the block products
  float at[4 * 16 * PA];      // diagonal blocks of A, fp32, transposed: [block][j][t]
  float gam[BT];              // running sum of g inside the chunk
  float beta[BT];
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// permuted k: 4 values at p, 4 values at p + 16
__device__ __forceinline__ bf16x8 ldsp(const uint16_t* p) {
  bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// permuted k from two separate 4-value halves
__device__ __forceinline__ bf16x8 ldsp2(const uint16_t* lo_p, const uint16_t* hi_p) {
  bf16x4 lo = *reinterpret_cast<const bf16x4*>(lo_p);
  bf16x4 hi = *reinterpret_cast<const bf16x4*>(hi_p);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// k values 8*grp..8*grp+7 of a 16-deep product padded to 32 (groups 2, 3 give zero)
__device__ __forceinline__ bf16x8 lds8_k16(const uint16_t* p, int grp) {
  bf16x8 z = {};
  return grp < 2 ? lds8(p) : z;
}

__device__ __forceinline__ uint16_t bfb(float f) { return f32_to_bf16_bits(f); }

__device__ __forceinline__ void st4bf(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

// two accumulator tiles (rows 4grp+i of 16-row blocks 2kk and 2kk+1) as one
// permuted operand over those 32 rows
__device__ __forceinline__ bf16x8 pair_operand(f32x4 lo, f32x4 hi) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = (__bf16)lo[i];
    v[4 + i] = (__bf16)hi[i];
  }
  return v;
}

// K^T and V^T rows are stored with their token index XOR-swizzled by a
// multiple of 8 that depends on the row (d >> 3): the transposed stores of
// 16 lanes holding different 8-row groups then hit different banks, and
// every aligned group of 4 or 8 tokens stays contiguous for the operand reads.
__device__ __forceinline__ int swz(int d) { return 8 * ((d >> 3) & 7); }

constexpr int NW = 4;            // waves per workgroup
constexpr int NT = 64 * NW;      // threads per workgroup
constexpr int NB = D / 16 / NW;  // 16-column state tiles per wave

struct Prefetch {
  u32x4 k[4], v[4], q[4];  // row (tid + NT it) >> 4, columns [8c8, 8c8+8), c8 = tid & 15
  float b[4];              // beta of those rows
  float g0, b0;            // g and beta of row (tid & 63), read by wave 0
};

// Loads the nv rows of a chunk starting at packed row rbase; buffer ranges end
// at row nv, so rows past the end read as zero.  A wave's 16-byte loads cover
// 4 whole 256-byte row segments.
__device__ __forceinline__ void prefetch(Prefetch& p, const ScanArgs& a, int64_t rbase, int nv, int m,
                                         int qoff, int koff, int voff, int tid, int wv) {
  const int C = a.channels, Hv = a.num_v_heads;
  const __amdgpu_buffer_rsrc_t ry =
      make_rsrc(reinterpret_cast<const uint16_t*>(a.y) + rbase * C, (uint32_t)nv * C * 2);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.g + rbase * Hv, (uint32_t)nv * Hv * 4);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.beta + rbase * Hv, (uint32_t)nv * Hv * 4);
  if (wv == 0) {
    const int t = tid & 63;
    p.g0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, 4 * (t * Hv + m), 0, 0));
    p.b0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, 4 * (t * Hv + m), 0, 0));
  }
  const int c8 = tid & 15;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = (tid + NT * it) >> 4;
    const int row = r * C + 8 * c8;
    p.k[it] = __builtin_amdgcn_raw_buffer_load_b128(ry, 2 * (row + koff), 0, 0);
    p.v[it] = __builtin_amdgcn_raw_buffer_load_b128(ry, 2 * (row + voff), 0, 0);
    p.q[it] = __builtin_amdgcn_raw_buffer_load_b128(ry, 2 * (row + qoff), 0, 0);
    p.b[it] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, 4 * (r * Hv + m), 0, 0));
  }
}

// Output rows [row0, row0 + nv) of the wave's state columns: lane holds rows
// 16tb + 4lg + i of columns n0 + 16nb + li as packed bf16 pairs.  The buffer
// range ends at row nv, so the stores of rows past the end are dropped.
__device__ __forceinline__ void store_out(const ScanArgs& a, const uint32_t (&opk)[4][NB][2], int64_t row0, int nv,
                                          int m, int n0, int li, int lg) {
  const int Hv = a.num_v_heads;
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(reinterpret_cast<uint16_t*>(a.out) + row0 * Hv * D, (uint32_t)nv * Hv * D * 2);
  const int obase = m * D + n0 + li + 4 * lg * Hv * D;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = opk[tb][nb][i >> 1];
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)((i & 1) ? (w >> 16) : (w & 0xffff)), ro,
                                              2 * (obase + 16 * nb + (16 * tb + i) * Hv * D), 0, 0);
      }
}

// lower 16x16 block pair number e (0..9) in row order: (0,0) (1,0) (1,1) (2,0) ...
__device__ __forceinline__ void lower_pair(int e, int& bi, int& bj) {
  bi = e >= 6 ? 3 : e >= 3 ? 2 : e >= 1 ? 1 : 0;
  bj = e - (bi * (bi + 1)) / 2;
}

__global__ __launch_bounds__(NT) void chunk_scan_kernel(ScanArgs a, SeqOrder ord) {
  __shared__ Smem sm;
  const int Hv = a.num_v_heads;
  const int rank = blockIdx.x / Hv;
  const int m = blockIdx.x % Hv;
  const int s = ord.n > 0 ? (rank < ord.n ? (int)ord.seq[rank] : a.num_seqs) : rank;
  if (s >= a.num_seqs) return;
  const int r0 = a.cu[s];
  const int L = a.cu[s + 1] - r0;
  if (L < a.min_len || L > a.max_len) return;
  if (!seq_active(a.read_idx, a.write_idx, s, a.num_blocks)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
  const int li = lane & 15, lg = lane >> 4;
  const int h = m / (Hv / a.num_k_heads);
  const int qoff = h * D, koff = a.num_k_heads * D + h * D;
  const int voff = 2 * a.num_k_heads * D + m * D;
  const int64_t head_off = (int64_t)m * D * D;
  const int n0 = 16 * NB * wv;  // this wave's state / output columns [n0, n0 + 16 NB)

  // S[:, n0 + 16nb + li]: sacc[db][nb] holds rows d = 16 db + 4 lg + i.
  // Read with coalesced 16-byte loads, staged through LDS.
  f32x4 sacc[8][NB];
  {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(
        reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.ssm_pool) +
                                       (int64_t)a.read_idx[s] * a.ssm_stride) + head_off, D * D * 4);
#pragma unroll
    for (int it = 0; it < D * D / 4 / NT; ++it) {
      const int f = tid + NT * it, row = f >> 5, c4 = f & 31;
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * f, 0, 0);
      *reinterpret_cast<u32x4*>(&sm.sst[row * PS + 4 * c4]) = v;
    }
    lds_barrier();
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[db][nb][i] = sm.sst[(16 * db + 4 * lg + i) * PS + n0 + 16 * nb + li];
    lds_barrier();
  }
  for (int i = tid; i < BT * PT; i += NT) {
    sm.t1[i] = 0;
    sm.p[i] = 0;
  }

  Prefetch pf;
  prefetch(pf, a, r0, min(BT, L), m, qoff, koff, voff, tid, wv);
  // the previous chunk's output, packed bf16 pairs; stored during the next chunk
  // so the stores are long complete when the loop top waits for the prefetch
  uint32_t opk[4][NB][2];
  int64_t obase_row = 0;
  int onv = 0;

  for (int c0 = 0; c0 < L; c0 += BT) {
    const int nv = min(BT, L - c0);
    const int64_t rbase = r0 + c0;

    // ---- stage this chunk from the prefetch registers, then prefetch the next one
    {
      const int c8 = tid & 15, tsw = 8 * (c8 & 7);  // swz(8 c8 + e) for every e
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int t = (tid + NT * it) >> 4;
        *reinterpret_cast<u32x4*>(&sm.kw.k[t * PQ + 8 * c8]) = pf.k[it];
        *reinterpret_cast<u32x4*>(&sm.q[t * PQ + 8 * c8]) = pf.q[it];
        const uint32_t kw[4] = {pf.k[it][0], pf.k[it][1], pf.k[it][2], pf.k[it][3]};
        const uint32_t vw[4] = {pf.v[it][0], pf.v[it][1], pf.v[it][2], pf.v[it][3]};
        const int ts = t ^ tsw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.kt[(8 * c8 + 2 * e) * PT + ts] = (uint16_t)(kw[e] & 0xffff);
          sm.kt[(8 * c8 + 2 * e + 1) * PT + ts] = (uint16_t)(kw[e] >> 16);
          const uint32_t vv = pack_bf16x2(pf.b[it] * __uint_as_float(vw[e] << 16),
                                          pf.b[it] * __uint_as_float(vw[e] & 0xffff0000u));
          sm.vt[(8 * c8 + 2 * e) * PT + ts] = (uint16_t)(vv & 0xffff);
          sm.vt[(8 * c8 + 2 * e + 1) * PT + ts] = (uint16_t)(vv >> 16);
        }
      }
      if (wv == 0) {
        float gv = pf.g0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float o = __shfl_up(gv, off);
          if (lane >= off) gv += o;
        }
        sm.gam[lane] = gv;
        sm.beta[lane] = pf.b0;
      }
    }
    lds_barrier();

    // ---- Gram products: 10 lower 16x16 blocks of K K^T (-> A) and 10 of Q K^T
    //      (-> P), five per wave
#pragma unroll
    for (int r = 0; r < 5; ++r) {
      const int e = wv + NW * r;
      int bi, bj;
      lower_pair(e % 10, bi, bj);
      const bool isq = e >= 10;
      // K K^T block (bi, bj): lane holds A[t = 16bi + 4lg + i][j = 16bj + li];
      // (Q K^T)^T block: lane holds P[t = 16bi + li][j = 16bj + 4lg + i]
      const uint16_t* xrow = isq ? &sm.kw.k[(16 * bj + li) * PQ] : &sm.kw.k[(16 * bi + li) * PQ];
      const uint16_t* yrow = isq ? &sm.q[(16 * bi + li) * PQ] : &sm.kw.k[(16 * bj + li) * PQ];
      bf16x8 xa[4], yb[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        xa[kk] = ldsp(xrow + 32 * kk + 4 * lg);
        yb[kk] = ldsp(yrow + 32 * kk + 4 * lg);
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mfma(xa[kk], yb[kk], acc);
      float v[4];
      if (!isq) {
        const int j = 16 * bj + li;
        const float gj = sm.gam[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * bi + 4 * lg + i;
          const float f = sm.beta[t] * __expf(sm.gam[t] - gj) * acc[i];
          v[i] = (j < t) ? f : 0.f;
        }
        if (bi == bj) {
          *reinterpret_cast<float4*>(&sm.at[(16 * bi + li) * PA + 4 * lg]) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) sm.ab[(16 * bi + 4 * lg + i) * PT + j] = bfb(v[i]);
        }
      } else {
        const int t = 16 * bi + li;
        const float gt = sm.gam[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 16 * bj + 4 * lg + i;
          const float f = __expf(gt - sm.gam[j]) * acc[i];
          v[i] = (j <= t) ? f : 0.f;
        }
        st4bf(&sm.p[t * PT + 16 * bj + 4 * lg], v[0], v[1], v[2], v[3]);
      }
    }
    lds_barrier();

    // ---- T = (I + A)^-1, diagonal block w by column-oriented fp32 forward
    //      substitution: lane (li = column c, lg) holds rows t = 4lg..4lg+3 of
    //      column c; step j broadcasts the finished x_j from its owner (lane
    //      li + 16 (j >> 2)) and every lane applies x_t -= A[t][j] x_j (A is zero
    //      on and above the diagonal).  Then the blocks above the diagonal that
    //      later products read are cleared: T(0,1), T(2,3), T^T(1,0).
    {
      const int rg = wv, c = li;
      const float* ab = &sm.at[(16 * rg) * PA + 4 * lg];
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (4 * lg + i == c) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < 15; ++j) {
        const float xj = __shfl(x[j & 3], li + 16 * (j >> 2));
        const f32x4 col = *reinterpret_cast<const f32x4*>(&ab[j * PA]);
        x -= col * xj;
      }
      const int cg = 16 * rg + c;
      const float bgc = sm.beta[cg] * __expf(sm.gam[cg]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tg = 16 * rg + 4 * lg + i;
        sm.tr[tg * PT + cg] = bfb(x[i]);
        sm.t1[tg * PT + cg] = bfb(x[i] * bgc);
      }
      st4bf(&sm.tt[cg * PT + 16 * rg + 4 * lg], x[0], x[1], x[2], x[3]);
      if (rg == 0 || rg == 2)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.tr[(16 * rg + 4 * lg + i) * PT + 16 * rg + 16 + c] = 0;
      if (rg == 1) st4bf(&sm.tt[(16 + c) * PT + 4 * lg], 0.f, 0.f, 0.f, 0.f);
    }
    lds_barrier();

    // ---- first-level blocks in the wave that solved the row block:
    //      wave 1: T10 = -T11 (A10 T00);  wave 3: T32 = -T33 (A32 T22)
    if (wv == 1 || wv == 3) {
      const int rb = 16 * wv, cb0 = 16 * (wv - 1);
      uint16_t* y = &sm.yt[(16 * (wv >> 1)) * PY];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma(lds8_k16(&sm.ab[(rb + li) * PT + cb0 + 8 * lg], lg),
                 lds8_k16(&sm.tt[(cb0 + li) * PT + cb0 + 8 * lg], lg), acc);
      st4bf(&y[li * PY + 4 * lg], acc[0], acc[1], acc[2], acc[3]);
      f32x4 tacc = {0.f, 0.f, 0.f, 0.f};
      tacc = mfma(lds8_k16(&sm.tr[(rb + li) * PT + rb + 8 * lg], lg), lds8_k16(&y[li * PY + 8 * lg], lg), tacc);
      const int cg = cb0 + li;
      const float bgc = sm.beta[cg] * __expf(sm.gam[cg]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tg = rb + 4 * lg + i;
        sm.tr[tg * PT + cg] = bfb(-tacc[i]);
        sm.t1[tg * PT + cg] = bfb(-tacc[i] * bgc);
      }
      st4bf(&sm.tt[cg * PT + rb + 4 * lg], -tacc[0], -tacc[1], -tacc[2], -tacc[3]);
    }
    lds_barrier();

    // ---- second level: T[32:64, 16c:16c+16] = -T_BB (A_BA T_AA)[:, 16c:16c+16],
    //      one 16-column block c per wave 0..1, both row blocks
    if (wv < 2) {
      const int cb0 = 16 * wv;
      uint16_t* y = &sm.yt[(32 + 16 * wv) * PY];
      const bf16x8 tb = lds8(&sm.tt[(cb0 + li) * PT + 8 * lg]);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma(lds8(&sm.ab[(32 + 16 * hb + li) * PT + 8 * lg]), tb, acc);
        st4bf(&y[li * PY + 16 * hb + 4 * lg], acc[0], acc[1], acc[2], acc[3]);
      }
      const int cg = cb0 + li;
      const float bgc = sm.beta[cg] * __expf(sm.gam[cg]);
      const bf16x8 yb = lds8(&y[li * PY + 8 * lg]);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        f32x4 tacc = {0.f, 0.f, 0.f, 0.f};
        tacc = mfma(lds8(&sm.tr[(32 + 16 * hb + li) * PT + 32 + 8 * lg]), yb, tacc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tg = 32 + 16 * hb + 4 * lg + i;
          sm.tr[tg * PT + cg] = bfb(-tacc[i]);
          sm.t1[tg * PT + cg] = bfb(-tacc[i] * bgc);
        }
      }
    }
    lds_barrier();

    // the global traffic of this chunk is issued here, after the small solve
    // phases, so that their waits never wait for it
    if (c0 + BT < L) prefetch(pf, a, rbase + BT, min(BT, L - c0 - BT), m, qoff, koff, voff, tid, wv);
    if (c0 > 0) store_out(a, opk, obase_row, onv, m, n0, li, lg);

    // ---- -W = -(T diag(b Gamma)) K into LDS (wave w: d blocks 2w, 2w+1, all
    //      chunk rows), and U~ = T (diag(b) V) for the wave's columns in the U
    //      accumulators
    f32x4 uacc[4][NB];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int nk = tb < 2 ? 1 : 2;
      f32x4 acc[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) uacc[tb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < nk; ++kk) {
        const bf16x8 bt = lds8(&sm.t1[(16 * tb + li) * PT + 32 * kk + 8 * lg]);
        const bf16x8 at = lds8(&sm.tr[(16 * tb + li) * PT + 32 * kk + 8 * lg]);
        bf16x8 ka[2], vb[NB];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int d = 16 * (2 * wv + e) + li;
          ka[e] = lds8(&sm.kt[d * PT + ((32 * kk + 8 * lg) ^ swz(d))]);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int n = n0 + 16 * nb + li;
          vb[nb] = lds8(&sm.vt[n * PT + ((32 * kk + 8 * lg) ^ swz(n))]);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) acc[e] = mfma(ka[e], bt, acc[e]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) uacc[tb][nb] = mfma(at, vb[nb], uacc[tb][nb]);
      }
      // lane holds W[t = 16tb + li][d = 16(2w+e) + 4lg + i]
#pragma unroll
      for (int e = 0; e < 2; ++e)
        st4bf(&sm.kw.w[(16 * tb + li) * PQ + 16 * (2 * wv + e) + 4 * lg], -acc[e][0], -acc[e][1], -acc[e][2],
              -acc[e][3]);
    }
    lds_barrier();

    // ---- state pass for the wave's columns, in registers
    {
      f32x4 oacc[4][NB];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[tb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8 sb[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sb[nb] = pair_operand(sacc[2 * kk][nb], sacc[2 * kk + 1][nb]);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const bf16x8 wa = ldsp(&sm.kw.w[(16 * tb + li) * PQ + 32 * kk + 4 * lg]);
          const bf16x8 qa = ldsp(&sm.q[(16 * tb + li) * PQ + 32 * kk + 4 * lg]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            uacc[tb][nb] = mfma(wa, sb[nb], uacc[tb][nb]);  // U = U~ - W S
            oacc[tb][nb] = mfma(qa, sb[nb], oacc[tb][nb]);  // Q S
          }
        }
      }
      const float glast = sm.gam[BT - 1];
      bf16x8 ub[2][NB], upb[2][NB];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float g0[4], g1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          g0[i] = sm.gam[32 * kk + 4 * lg + i];
          g1[i] = sm.gam[32 * kk + 16 + 4 * lg + i];
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          ub[kk][nb] = pair_operand(uacc[2 * kk][nb], uacc[2 * kk + 1][nb]);
          f32x4 lo, hi;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            lo[i] = uacc[2 * kk][nb][i] * __expf(glast - g0[i]);
            hi[i] = uacc[2 * kk + 1][nb][i] * __expf(glast - g1[i]);
            oacc[2 * kk][nb][i] *= __expf(g0[i]);
            oacc[2 * kk + 1][nb][i] *= __expf(g1[i]);
          }
          upb[kk][nb] = pair_operand(lo, hi);
        }
      }
      // O += P U
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int nk = tb < 2 ? 1 : 2;
#pragma unroll
        for (int kk = 0; kk < nk; ++kk) {
          const bf16x8 pa = ldsp(&sm.p[(16 * tb + li) * PT + 32 * kk + 4 * lg]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) oacc[tb][nb] = mfma(pa, ub[kk][nb], oacc[tb][nb]);
        }
      }
      // S <- Gamma_c S + K^T U'
      const float gc = __expf(glast);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const uint16_t* row = &sm.kt[(16 * db + li) * PT];
        const int sw = swz(16 * db + li);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 ka = ldsp2(row + ((32 * kk + 4 * lg) ^ sw), row + ((32 * kk + 16 + 4 * lg) ^ sw));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            if (kk == 0) sacc[db][nb] *= gc;
            sacc[db][nb] = mfma(ka, upb[kk][nb], sacc[db][nb]);
          }
        }
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          opk[tb][nb][0] = pack_bf16x2(oacc[tb][nb][0], oacc[tb][nb][1]);
          opk[tb][nb][1] = pack_bf16x2(oacc[tb][nb][2], oacc[tb][nb][3]);
        }
      obase_row = rbase;
      onv = nv;
    }
    lds_barrier();
  }

  store_out(a, opk, obase_row, onv, m, n0, li, lg);
  {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.sst[(16 * db + 4 * lg + i) * PS + n0 + 16 * nb + li] = sacc[db][nb][i];
    lds_barrier();
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(
        reinterpret_cast<float*>(reinterpret_cast<char*>(a.ssm_pool) + (int64_t)a.write_idx[s] * a.ssm_stride) +
            head_off, D * D * 4);
#pragma unroll
    for (int it = 0; it < D * D / 4 / NT; ++it) {
      const int f = tid + NT * it, row = f >> 5, c4 = f & 31;
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(&sm.sst[row * PS + 4 * c4]), rs,
                                             16 * f, 0, 0);
    }
  }
}

}  // namespace

bool chunk_supported(int dk, int dv) { return dk == D && dv == D; }

hipError_t launch_chunk(const ScanArgs& a, const SeqOrder& order, int dk, int dv, hipStream_t st) {
  if (!chunk_supported(dk, dv)) return hipErrorInvalidValue;
  const int rows = order.n > 0 ? order.n : a.num_seqs;
  dim3 grid(rows * a.num_v_heads);
  hipLaunchKernelGGL(chunk_scan_kernel, grid, dim3(NT), 0, st, a, order);
  return hipGetLastError();
}

}  // namespace gdn
