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

constexpr int BT = 64;            // chunk length
constexpr int D = 128;            // d_k = d_v
constexpr int NW = 4;             // waves per workgroup
constexpr int NT = 64 * NW;       // threads per workgroup
constexpr int NB = D / 16 / NW;   // 16-column state tiles per wave
constexpr int PV = D + 16;        // pitch (elements) of the V rows
constexpr int PW = D + 8;         // pitch of the -W rows
constexpr int PP = BT + 8;        // pitch of the P rows
constexpr int PX = BT + 16;       // pitch of the transposed 64 x 64 tiles
constexpr int PA = 20;            // fp32 pitch of the transposed diagonal blocks of A
constexpr int PS = D + 4;         // fp32 pitch of the staged state
constexpr int PO = BT + 8;        // pitch of a wave's staged output tile [n][t]

// LDS.  "k-permuted" rows store element d of each 32-wide group at
// 8*((d>>2)&3) + 4*((d>>4)&1) + (d&3): the 8 values an operand lane needs
// (k = 4g..4g+3 and 16+4g..16+4g+3 of the group) are then one 16-byte read.
struct alignas(16) Smem {
  union {
    struct {
      uint16_t q[BT * D];     // Q rows [t][perm d], 16-byte chunks XOR-swizzled by row
      uint16_t k[BT * D];     // K rows, same layout
      uint16_t v[BT * PV];    // V rows [j][n]; after the W phase, each wave's output tile
      uint16_t w[BT * PW];    // -W rows [t][perm d]
    };
    float sst[D * PS];        // the fp32 state [d][n], staged at the start and the end
  };
  uint16_t p[BT * PP];        // P = M o Q K^T, [t][perm j]; blocks above the diagonal stay zero
  uint16_t tt[BT * PX];       // T^T [j][t]; blocks above the diagonal of T stay zero
  uint16_t t1t[BT * PX];      // (T diag(b Gamma))^T
  uint16_t t2t[BT * PX];      // (T diag(b))^T
  uint16_t abt[BT * PX];      // A^T, blocks below the diagonal
  float at[4 * 16 * PA];      // diagonal blocks of A, fp32, [block][j][t]
  float gam[BT];              // running sum of g inside the chunk
  float eg[BT];               // e^gamma
  float ed[BT];               // e^(gamma_last - gamma)
  float beta[BT];
  float bg[BT];               // beta e^gamma
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// A 16-deep product (lane holds k = 4g..4g+3 of each operand) on the same
// 16x16x32 instruction, zero-padded: every accumulation chain in the kernel
// then uses one MFMA shape (the two shapes take the same issue time).
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  const bf16x4 z = {};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7),
                                                 __builtin_shufflevector(b, z, 0, 1, 2, 3, 4, 5, 6, 7), c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 lds4(const uint16_t* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ds_read_b64_tr_b16.  Within each 16-lane group g, every lane reads 4
// consecutive 16-bit values at its own address; lane 16g + 4a + b then
// receives value b of lanes 16g + a, 16g + a + 4, 16g + a + 8, 16g + a + 12.
// When lane 16g + a + 4i points at row (base + i), columns c0 + 4a .. c0 + 4a + 3
// of a row-major tile, lane 16g + n receives column c0 + n of rows base..base+3:
// a transposed operand read straight from row-major storage.
__device__ __forceinline__ bf16x4 ldtr(const uint16_t* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<uint16_t*>(p))));
}

// DPP lane move within each row of 16 lanes (or across rows for the row
// broadcasts); lanes without a source lane get zero.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8 inside
// each row of 16 lanes, then lane 15 of row 0 and lane 31 carried into the
// later rows.
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp_move<0x111, 0xf>(v);  // row_shr:1
  v += dpp_move<0x112, 0xf>(v);  // row_shr:2
  v += dpp_move<0x114, 0xf>(v);  // row_shr:4
  v += dpp_move<0x118, 0xf>(v);  // row_shr:8
  v += dpp_move<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Scheduling fence: the compiler keeps every instruction on its side, so
// operand reads placed before it are issued ahead of the products after it.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ uint16_t bfb(float f) { return f32_to_bf16_bits(f); }
__device__ __forceinline__ void st4bf(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (__bf16)v[i];
  return r;
}

// two accumulator tiles (rows 4g+i of 16-row blocks 2kk and 2kk+1) as one
// k-permuted operand over those 32 rows
__device__ __forceinline__ bf16x8 pair_operand(f32x4 lo, f32x4 hi) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = (__bf16)lo[i];
    v[4 + i] = (__bf16)hi[i];
  }
  return v;
}

// stored position of natural index d in a k-permuted row
__device__ __forceinline__ constexpr int perm(int d) {
  return (d & ~31) | ((d & 12) << 1) | ((d & 16) >> 2) | (d & 3);
}

// element offset of (row t, stored position pos) in a swizzled [64][128] tile:
// 16-byte chunk c of row t sits at chunk c ^ (2 (t & 7) + ((t >> 3) & 1)).  The
// 16 rows of a row-operand read and the 8 rows x 32 bytes of each half of a
// transposed read then fall on distinct banks.
__device__ __forceinline__ int swz_off(int t, int pos) {
  const int f = 2 * (t & 7) + ((t >> 3) & 1);
  return t * D + (((pos >> 3) ^ f) << 3) + (pos & 7);
}

// Operand lanes: r = l & 15, g = l >> 4; as a transposed-read source, lane l
// supplies row i = (l >> 2) & 3 and column group a = l & 3.
struct Lane {
  int r, g, a, i;
};

// rows t0 + r of a swizzled Q / K tile, k = d of 32-group kk (permuted)
__device__ __forceinline__ bf16x8 ld_row_qk(const uint16_t* base, int t0, int kk, const Lane& L) {
  return lds8(base + swz_off(t0 + L.r, 32 * kk + 8 * L.g));
}

// K^T operand from the swizzled K tile: lane gets K[t][16 db + r] for the
// permuted token set t = 32 kk + {4g..4g+3, 16+4g..16+4g+3}
__device__ __forceinline__ bf16x8 ld_tr_qk(const uint16_t* base, int db, int kk, const Lane& L) {
  const int pos = perm(16 * db + 4 * L.a);
  const int t = 32 * kk + 4 * L.g + L.i;
  return cat(ldtr(base + swz_off(t, pos)), ldtr(base + swz_off(t + 16, pos)));
}

// transposed operand from a row-major [j][c] tile of pitch P: lane gets
// X[j][c0 + r] for the permuted set j = 32 kk + {4g..4g+3, 16+4g..16+4g+3}
template <int P>
__device__ __forceinline__ bf16x8 ld_tr(const uint16_t* base, int c0, int kk, const Lane& L) {
  const uint16_t* p = base + (32 * kk + 4 * L.g + L.i) * P + c0 + 4 * L.a;
  return cat(ldtr(p), ldtr(p + 16 * P));
}

struct Prefetch {
  u32x4 k[4], v[4], q[4];  // row (tid + NT it) >> 4, columns [8c8, 8c8+8), c8 = tid & 15
  float g0, b0;            // g and beta of row (tid & 63), read by wave 0
};

// Loads the nv rows of a chunk starting at packed row rbase; buffer ranges end
// at row nv, so rows past the end read as zero.  A wave's 16-byte loads cover
// 4 whole 256-byte row segments.
__device__ __forceinline__ void prefetch(Prefetch& p, const ScanArgs& a, int64_t rbase, int nv, int m,
                                         int qoff, int koff, int voff, int tid, int wv) {
  const int C = a.channels, Hv = a.num_v_heads;
  if (wv == 0) {
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.g + rbase * Hv, (uint32_t)nv * Hv * 4);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.beta + rbase * Hv, (uint32_t)nv * Hv * 4);
    const int t = tid & 63;
    p.g0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, 4 * (t * Hv + m), 0, 0));
    p.b0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, 4 * (t * Hv + m), 0, 0));
  }
  const __amdgpu_buffer_rsrc_t ry =
      make_rsrc(reinterpret_cast<const uint16_t*>(a.y) + rbase * C, (uint32_t)nv * C * 2);
  const int c8 = tid & 15;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = ((tid + NT * it) >> 4) * C + 8 * c8;
    p.k[it] = __builtin_amdgcn_raw_buffer_load_b128(ry, 2 * (row + koff), 0, 0);
    p.v[it] = __builtin_amdgcn_raw_buffer_load_b128(ry, 2 * (row + voff), 0, 0);
    p.q[it] = __builtin_amdgcn_raw_buffer_load_b128(ry, 2 * (row + qoff), 0, 0);
  }
}

// The 16 rows 16b..16b+15 of a swizzled Q / K tile as four row operands (all 128 d).
struct Blk {
  bf16x8 v[4];
};
__device__ __forceinline__ Blk ld_blk(const uint16_t* base, int b, const Lane& L) {
  Blk x;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) x.v[kk] = ld_row_qk(base, 16 * b, kk, L);
  return x;
}
// D[row][col] = sum_d X[row][d] Y[col][d] over two 16-row blocks
__device__ __forceinline__ f32x4 dot_blk(const Blk& x, const Blk& y) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) acc = mfma(x.v[kk], y.v[kk], acc);
  return acc;
}

// Block (bi, bj), bj <= bi, of A = strictly-lower(b_t e^{gamma_t - gamma_j} K K^T)
// from acc = K_bi K_bj^T: lane holds A[t = 16bi + 4g + i][j = 16bj + r].
// Diagonal blocks go to `at` in fp32, the others to `abt` in bf16, both transposed.
__device__ __forceinline__ void put_a(Smem& sm, int bi, int bj, f32x4 acc, const Lane& L) {
  const int j = 16 * bj + L.r;
  const float gj = sm.gam[j];
  const f32x4 gt = *reinterpret_cast<const f32x4*>(&sm.gam[16 * bi + 4 * L.g]);
  const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[16 * bi + 4 * L.g]);
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float f = bt[i] * __expf(gt[i] - gj) * acc[i];
    v[i] = (j < 16 * bi + 4 * L.g + i) ? f : 0.f;
  }
  if (bi == bj)
    *reinterpret_cast<float4*>(&sm.at[(16 * bi + L.r) * PA + 4 * L.g]) = make_float4(v[0], v[1], v[2], v[3]);
  else
    st4bf(&sm.abt[j * PX + 16 * bi + 4 * L.g], v[0], v[1], v[2], v[3]);
}

// Block (bi, bj), bj <= bi, of P = M o Q K^T from acc = K_bj Q_bi^T (transposed):
// lane holds P[t = 16bi + r][j = 16bj + 4g + i].
__device__ __forceinline__ void put_p(Smem& sm, int bi, int bj, f32x4 acc, const Lane& L) {
  const int t = 16 * bi + L.r;
  const float gt = sm.gam[t];
  const f32x4 gj = *reinterpret_cast<const f32x4*>(&sm.gam[16 * bj + 4 * L.g]);
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float f = __expf(gt - gj[i]) * acc[i];
    v[i] = (16 * bj + 4 * L.g + i <= t) ? f : 0.f;
  }
  st4bf(&sm.p[t * PP + perm(16 * bj + 4 * L.g)], v[0], v[1], v[2], v[3]);
}

// Column c of T's block (R, C) in a lane's D tile (rows 4g + i) -> T^T and its
// two column-scaled copies.
__device__ __forceinline__ void put_t(Smem& sm, int R, int C, f32x4 tv, const Lane& L) {
  const int jc = 16 * C + L.r;
  const int o = jc * PX + 16 * R + 4 * L.g;
  const float s1 = sm.bg[jc], s2 = sm.beta[jc];
  st4bf(&sm.tt[o], tv[0], tv[1], tv[2], tv[3]);
  st4bf(&sm.t1t[o], s1 * tv[0], s1 * tv[1], s1 * tv[2], s1 * tv[3]);
  st4bf(&sm.t2t[o], s2 * tv[0], s2 * tv[1], s2 * tv[2], s2 * tv[3]);
}

// 16x16x16 operands of the block products, from the transposed tiles:
// A rows 16R + r, k = 16C + 4g + i (lane gets X[16R + r][16C + 4g..+3])
__device__ __forceinline__ bf16x4 blk_a(const uint16_t* xt, int R, int C, const Lane& L) {
  return ldtr(xt + (16 * C + 4 * L.g + L.i) * PX + 16 * R + 4 * L.a);
}
// B k = 16R + 4g + i, column 16C + r (lane gets X[16R + 4g..+3][16C + r])
__device__ __forceinline__ bf16x4 blk_b(const uint16_t* xt, int R, int C, const Lane& L) {
  return lds4(xt + (16 * C + L.r) * PX + 16 * R + 4 * L.g);
}

// T = (I + A)^-1 in one wave.  The four diagonal blocks by fp32 forward
// substitution, one column per lane (lane 16 rg + c solves block rg, column
// c, all 16 rows in registers, so no lane exchange is needed), then the blocks
// below the diagonal by MFMA block products:
//   T10 = -T11 A10 T00,  T32 = -T33 A32 T22,
//   [T20 T21; T30 T31] = -[T22 0; T32 T33] [A20 A21; A30 A31] [T00 0; T10 T11].
__device__ __forceinline__ void solve_t(Smem& sm, const Lane& L, int lane) {
  {
    const int c = lane & 15, rg = lane >> 4;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) x[t] = (t == c) ? 1.f : 0.f;
    const float* col = &sm.at[16 * rg * PA];
#pragma unroll
    for (int j = 0; j < 15; ++j) {
      const float xj = x[j];
      float aj[16];
#pragma unroll
      for (int q4 = (j + 1) >> 2; q4 < 4; ++q4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&col[j * PA + 4 * q4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) aj[4 * q4 + e] = v[e];
      }
#pragma unroll
      for (int t = j + 1; t < 16; ++t) x[t] -= aj[t] * xj;
    }
    const int jc = 16 * rg + c;
    const float s1 = sm.bg[jc], s2 = sm.beta[jc];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int o = jc * PX + 16 * rg + 8 * h;
      u32x4 w0, w1, w2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = x[8 * h + 2 * e], x1 = x[8 * h + 2 * e + 1];
        w0[e] = pack_bf16x2(x0, x1);
        w1[e] = pack_bf16x2(s1 * x0, s1 * x1);
        w2[e] = pack_bf16x2(s2 * x0, s2 * x1);
      }
      *reinterpret_cast<u32x4*>(&sm.tt[o]) = w0;
      *reinterpret_cast<u32x4*>(&sm.t1t[o]) = w1;
      *reinterpret_cast<u32x4*>(&sm.t2t[o]) = w2;
    }
  }
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  // first level: T10, T32 (the wave's own LDS writes are visible to its later reads)
  f32x4 t10, t32;
  {
    const f32x4 y10 = mfma16(blk_a(sm.abt, 1, 0, L), blk_b(sm.tt, 0, 0, L), z);
    const f32x4 y32 = mfma16(blk_a(sm.abt, 3, 2, L), blk_b(sm.tt, 2, 2, L), z);
    t10 = -mfma16(blk_a(sm.tt, 1, 1, L), to_bf16x4(y10), z);
    t32 = -mfma16(blk_a(sm.tt, 3, 3, L), to_bf16x4(y32), z);
    put_t(sm, 1, 0, t10, L);
    put_t(sm, 3, 2, t32, L);
  }
  // second level
  {
    const bf16x4 b00 = blk_b(sm.tt, 0, 0, L), b11 = blk_b(sm.tt, 1, 1, L), b10 = to_bf16x4(t10);
    const bf16x4 a20 = blk_a(sm.abt, 2, 0, L), a21 = blk_a(sm.abt, 2, 1, L);
    const bf16x4 a30 = blk_a(sm.abt, 3, 0, L), a31 = blk_a(sm.abt, 3, 1, L);
    const f32x4 y20 = mfma16(a21, b10, mfma16(a20, b00, z));
    const f32x4 y21 = mfma16(a21, b11, z);
    const f32x4 y30 = mfma16(a31, b10, mfma16(a30, b00, z));
    const f32x4 y31 = mfma16(a31, b11, z);
    const bf16x4 t22 = blk_a(sm.tt, 2, 2, L), t33 = blk_a(sm.tt, 3, 3, L), t32a = blk_a(sm.tt, 3, 2, L);
    const bf16x4 c20 = to_bf16x4(y20), c21 = to_bf16x4(y21);
    put_t(sm, 2, 0, -mfma16(t22, c20, z), L);
    put_t(sm, 2, 1, -mfma16(t22, c21, z), L);
    put_t(sm, 3, 0, -mfma16(t33, to_bf16x4(y30), mfma16(t32a, c20, z)), L);
    put_t(sm, 3, 1, -mfma16(t33, to_bf16x4(y31), mfma16(t32a, c21, z)), L);
  }
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
  const Lane ln{lane & 15, lane >> 4, lane & 3, (lane >> 2) & 3};
  const int li = ln.r, lg = ln.g;
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
  // blocks above the diagonal are read by the full-width products and never written
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int i = tid; i < BT * PP / 8; i += NT) reinterpret_cast<u32x4*>(sm.p)[i] = zero;
    for (int i = tid; i < BT * PX / 8; i += NT) {
      reinterpret_cast<u32x4*>(sm.tt)[i] = zero;
      reinterpret_cast<u32x4*>(sm.t1t)[i] = zero;
      reinterpret_cast<u32x4*>(sm.t2t)[i] = zero;
    }
  }

  Prefetch pf;
  prefetch(pf, a, r0, min(BT, L), m, qoff, koff, voff, tid, wv);

  for (int c0 = 0; c0 < L; c0 += BT) {
    const int nv = min(BT, L - c0);
    const int64_t rbase = r0 + c0;

    // ---- stage this chunk from the prefetch registers
    {
      const int c8 = tid & 15;
      const int p1 = perm(8 * c8), p2 = perm(8 * c8 + 4);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int t = (tid + NT * it) >> 4;
        *reinterpret_cast<uint2*>(&sm.q[swz_off(t, p1)]) = make_uint2(pf.q[it][0], pf.q[it][1]);
        *reinterpret_cast<uint2*>(&sm.q[swz_off(t, p2)]) = make_uint2(pf.q[it][2], pf.q[it][3]);
        *reinterpret_cast<uint2*>(&sm.k[swz_off(t, p1)]) = make_uint2(pf.k[it][0], pf.k[it][1]);
        *reinterpret_cast<uint2*>(&sm.k[swz_off(t, p2)]) = make_uint2(pf.k[it][2], pf.k[it][3]);
        *reinterpret_cast<u32x4*>(&sm.v[t * PV + 8 * c8]) = pf.v[it];
      }
      if (wv == 0) {
        const float gv = wave_prefix_sum(pf.g0);
        const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gv), 63));
        const float e = __expf(gv);
        sm.gam[lane] = gv;
        sm.eg[lane] = e;
        sm.ed[lane] = __expf(glast - gv);
        sm.beta[lane] = pf.b0;
        sm.bg[lane] = pf.b0 * e;
      }
    }
    lds_barrier();

    // ---- A = strictly-lower(b e^{gamma_t - gamma_j} K K^T): ten 16x16 blocks,
    //      operand blocks read before the products
    if (wv == 0) {
      const Blk k0 = ld_blk(sm.k, 0, ln), k3 = ld_blk(sm.k, 3, ln);
      fence();
      const f32x4 a00 = dot_blk(k0, k0), a30 = dot_blk(k3, k0), a33 = dot_blk(k3, k3);
      put_a(sm, 0, 0, a00, ln); put_a(sm, 3, 0, a30, ln); put_a(sm, 3, 3, a33, ln);
    } else if (wv == 1) {
      const Blk k0 = ld_blk(sm.k, 0, ln), k1 = ld_blk(sm.k, 1, ln), k3 = ld_blk(sm.k, 3, ln);
      fence();
      const f32x4 a10 = dot_blk(k1, k0), a11 = dot_blk(k1, k1), a31 = dot_blk(k3, k1);
      put_a(sm, 1, 0, a10, ln); put_a(sm, 1, 1, a11, ln); put_a(sm, 3, 1, a31, ln);
    } else if (wv == 2) {
      const Blk k0 = ld_blk(sm.k, 0, ln), k2 = ld_blk(sm.k, 2, ln);
      fence();
      const f32x4 a20 = dot_blk(k2, k0), a22 = dot_blk(k2, k2);
      put_a(sm, 2, 0, a20, ln); put_a(sm, 2, 2, a22, ln);
    } else {
      const Blk k1 = ld_blk(sm.k, 1, ln), k2 = ld_blk(sm.k, 2, ln), k3 = ld_blk(sm.k, 3, ln);
      fence();
      const f32x4 a21 = dot_blk(k2, k1), a32 = dot_blk(k3, k2);
      put_a(sm, 2, 1, a21, ln); put_a(sm, 3, 2, a32, ln);
    }
    lds_barrier();

    // ---- T = (I + A)^-1 in wave 0; P = M o Q K^T in the others
    if (wv == 0) {
      solve_t(sm, ln, lane);
    } else if (wv == 1) {
      const Blk q3 = ld_blk(sm.q, 3, ln), k0 = ld_blk(sm.k, 0, ln), k1 = ld_blk(sm.k, 1, ln);
      const Blk k2 = ld_blk(sm.k, 2, ln), k3 = ld_blk(sm.k, 3, ln);
      fence();
      const f32x4 p30 = dot_blk(k0, q3), p31 = dot_blk(k1, q3), p32 = dot_blk(k2, q3), p33 = dot_blk(k3, q3);
      put_p(sm, 3, 0, p30, ln); put_p(sm, 3, 1, p31, ln); put_p(sm, 3, 2, p32, ln); put_p(sm, 3, 3, p33, ln);
    } else if (wv == 2) {
      const Blk q2 = ld_blk(sm.q, 2, ln), k0 = ld_blk(sm.k, 0, ln), k1 = ld_blk(sm.k, 1, ln);
      const Blk k2 = ld_blk(sm.k, 2, ln);
      fence();
      const f32x4 p20 = dot_blk(k0, q2), p21 = dot_blk(k1, q2), p22 = dot_blk(k2, q2);
      put_p(sm, 2, 0, p20, ln); put_p(sm, 2, 1, p21, ln); put_p(sm, 2, 2, p22, ln);
    } else {
      const Blk q0 = ld_blk(sm.q, 0, ln), q1 = ld_blk(sm.q, 1, ln), k0 = ld_blk(sm.k, 0, ln);
      const Blk k1 = ld_blk(sm.k, 1, ln);
      fence();
      const f32x4 p10 = dot_blk(k0, q1), p11 = dot_blk(k1, q1), p00 = dot_blk(k0, q0);
      put_p(sm, 1, 0, p10, ln); put_p(sm, 1, 1, p11, ln); put_p(sm, 0, 0, p00, ln);
    }
    lds_barrier();

    // the next chunk's loads are issued here, after the short phases, and
    // have the W phase and the state pass to arrive
    if (c0 + BT < L) prefetch(pf, a, rbase + BT, min(BT, L - c0 - BT), m, qoff, koff, voff, tid, wv);

    // ---- -W = -(T diag(b Gamma) K) rows into LDS (wave w: d blocks 2w, 2w+1),
    //      U~ = T diag(b) V for the wave's columns in registers
    f32x4 uacc[4][NB];
    {
      f32x4 wacc[4][2];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
        for (int e = 0; e < 2; ++e) wacc[tb][e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) uacc[tb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      bf16x8 ka[2][2], vb[2][NB], b1[2][4], a2[2][4];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int e = 0; e < 2; ++e) ka[kk][e] = ld_tr_qk(sm.k, 2 * wv + e, kk, ln);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) vb[kk][nb] = ld_tr<PV>(sm.v, n0 + 16 * nb, kk, ln);
#pragma unroll
        for (int tb = 2 * kk; tb < 4; ++tb) {
          b1[kk][tb] = ld_tr<PX>(sm.t1t, 16 * tb, kk, ln);  // T1[t][j] as the B operand
          a2[kk][tb] = ld_tr<PX>(sm.t2t, 16 * tb, kk, ln);  // T2[t][j] as the A operand
        }
        fence();
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int tb = 2 * kk; tb < 4; ++tb) {
#pragma unroll
          for (int e = 0; e < 2; ++e) wacc[tb][e] = mfma(ka[kk][e], b1[kk][tb], wacc[tb][e]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) uacc[tb][nb] = mfma(a2[kk][tb], vb[kk][nb], uacc[tb][nb]);
        }
      // lane holds W[t = 16tb + li][d = 16(2w+e) + 4lg + i]
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          st4bf(&sm.w[(16 * tb + li) * PW + perm(16 * (2 * wv + e) + 4 * lg)], -wacc[tb][e][0], -wacc[tb][e][1],
                -wacc[tb][e][2], -wacc[tb][e][3]);
    }
    lds_barrier();

    // ---- state pass for the wave's columns, in registers.  Operand reads run
    //      one step ahead of the products that use them (the scheduling
    //      barriers keep them there).
    {
      f32x4 oacc[4][NB];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[tb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 wa[2][4], qa[2][4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        wa[0][tb] = lds8(&sm.w[(16 * tb + li) * PW + 8 * lg]);
        qa[0][tb] = ld_row_qk(sm.q, 16 * tb, 0, ln);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int cur = kk & 1;
        fence();
        if (kk < 3) {
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) {
            wa[cur ^ 1][tb] = lds8(&sm.w[(16 * tb + li) * PW + 32 * (kk + 1) + 8 * lg]);
            qa[cur ^ 1][tb] = ld_row_qk(sm.q, 16 * tb, kk + 1, ln);
          }
        }
        fence();
        bf16x8 sb[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sb[nb] = pair_operand(sacc[2 * kk][nb], sacc[2 * kk + 1][nb]);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            uacc[tb][nb] = mfma(wa[cur][tb], sb[nb], uacc[tb][nb]);  // U = U~ - W S
            oacc[tb][nb] = mfma(qa[cur][tb], sb[nb], oacc[tb][nb]);  // Q S
          }
      }
      fence();
      // P rows, read while U is scaled
      bf16x8 pa[6];
#pragma unroll
      for (int tb = 0, e = 0; tb < 4; ++tb)
#pragma unroll
        for (int kk = 0; kk <= (tb >> 1); ++kk, ++e) pa[e] = lds8(&sm.p[(16 * tb + li) * PP + 32 * kk + 8 * lg]);
      fence();
      bf16x8 ub[2][NB], upb[2][NB];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const f32x4 e0 = *reinterpret_cast<const f32x4*>(&sm.eg[32 * kk + 4 * lg]);
        const f32x4 e1 = *reinterpret_cast<const f32x4*>(&sm.eg[32 * kk + 16 + 4 * lg]);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&sm.ed[32 * kk + 4 * lg]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&sm.ed[32 * kk + 16 + 4 * lg]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          ub[kk][nb] = pair_operand(uacc[2 * kk][nb], uacc[2 * kk + 1][nb]);
          upb[kk][nb] = pair_operand(uacc[2 * kk][nb] * d0, uacc[2 * kk + 1][nb] * d1);
          oacc[2 * kk][nb] *= e0;
          oacc[2 * kk + 1][nb] *= e1;
        }
      }
      fence();
      // O += P U, while the K^T operands of the first half of the state update arrive
      bf16x8 kt[8];
#pragma unroll
      for (int db = 0; db < 8; ++db) kt[db] = ld_tr_qk(sm.k, db, 0, ln);
      fence();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int tb = 2 * kk; tb < 4; ++tb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            oacc[tb][nb] = mfma(pa[kk == 0 ? (tb < 2 ? tb : 2 * tb - 2) : 2 * tb - 1], ub[kk][nb], oacc[tb][nb]);
      // S <- Gamma_c S + K^T U', tokens 0..31 then 32..63; the second half's
      // operands are read during the first half's products
      const float gc = sm.eg[BT - 1];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 kn[8];
        fence();
        if (kk == 0) {
#pragma unroll
          for (int db = 0; db < 8; ++db) kn[db] = ld_tr_qk(sm.k, db, 1, ln);
        }
        fence();
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            if (kk == 0) sacc[db][nb] *= gc;
            sacc[db][nb] = mfma(kt[db], upb[kk][nb], sacc[db][nb]);
          }
        if (kk == 0) {
#pragma unroll
          for (int db = 0; db < 8; ++db) kt[db] = kn[db];
        }
      }
      fence();
      // O: through the wave's LDS tile [n][t] to 16-byte row stores
      uint16_t* ot = &sm.v[wv * 32 * PO];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          st4bf(&ot[(16 * nb + li) * PO + 16 * tb + 4 * lg], oacc[tb][nb][0], oacc[tb][nb][1], oacc[tb][nb][2],
                oacc[tb][nb][3]);
      const __amdgpu_buffer_rsrc_t ro =
          make_rsrc(reinterpret_cast<uint16_t*>(a.out) + rbase * Hv * D, (uint32_t)nv * Hv * D * 2);
      const int ao = (lane & 15) >> 2, bo = lane & 3;  // this lane's output: columns 8 ao.., row 16 rho + 4 lg + bo
#pragma unroll
      for (int rho = 0; rho < 4; ++rho) {
        const uint16_t* src = &ot[(8 * ln.a + ln.i) * PO + 16 * rho + 4 * lg];
        const bf16x8 o8 = cat(ldtr(src), ldtr(src + 4 * PO));
        const int t = 16 * rho + 4 * lg + bo;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o8), ro,
                                               2 * (t * Hv * D + m * D + n0 + 8 * ao), 0, 0);
      }
    }
    lds_barrier();
  }

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
