// gdn_mfma.h -- building blocks of the chunked (WY / UT form) kernels on gfx950:
// MFMA wrappers, the LDS tile layout and its operand reads, the blocked
// triangular solve T = (I + A)^-1 of a 64-row chunk, and LDS flags.  Shared by
// the gated-delta-rule chunk kernel and the Kimi-delta-attention chunk kernel
// (not part of the C ABI).
//
// MFMA 16x16x32 bf16 operand layout (lane l, r = l & 15, grp = l >> 4):
//   A: row r, 8 values of k;  B: column r, the same 8 values of k;
//   D: column r, rows 4*grp + {0,1,2,3}.
// The MFMA sums over k, so any k order shared by both operands gives the same
// product.  A D tile X can be used as the B operand X or as the A operand X^T
// of a later product; a pair of D tiles (row blocks 2kk and 2kk+1) is then an
// operand over the 32 k values {4grp..4grp+3, 16+4grp..16+4grp+3} of step kk
// ("pair order").  State rows are kept in registers relabelled (sigma below) so
// that pair order over d is natural order over the columns of K and Q.
#pragma once

#include "gdn_device.h"

namespace gdn {
namespace {

constexpr int BT = 64;            // chunk length
constexpr int D = 128;            // d_k = d_v
constexpr int PP = BT + 8;        // pitch of the P rows
constexpr int PB = 16;            // pitch of a 16 x 16 block
constexpr int PA = 20;            // fp32 pitch of the transposed diagonal blocks of A

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
// operand over those 32 rows in pair order
__device__ __forceinline__ bf16x8 pair_operand(f32x4 lo, f32x4 hi) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = (__bf16)lo[i];
    v[4 + i] = (__bf16)hi[i];
  }
  return v;
}

// position of index j of P's rows in pair order: j = 32kk + 4g + i -> 32kk + 8g + i and
// j = 32kk + 16 + 4g + i -> 32kk + 8g + 4 + i, so the 8 values a lane needs are one
// 16-byte read
__device__ __forceinline__ constexpr int perm(int d) {
  return (d & ~31) | ((d & 12) << 1) | ((d & 16) >> 2) | (d & 3);
}

// element offset of (row t, column c) in a swizzled [64][128] tile: 16-byte
// chunk c >> 3 of row t sits at chunk (c >> 3) ^ f(t), f(t) = (t & 15) ^ (8 (bit 1 of t)).
// On gfx950 the LDS serves 256 bytes a pass.  A 16-byte read takes four passes of
// 16 lanes, lane l in pass (bit 5 of l, parity of bits 2-4 of l), not 16 consecutive
// lanes; an 8-byte read takes two passes of 32 consecutive lanes (both measured with
// the bank-conflict counter).  With this f a row-operand read (lane l: row l & 15,
// chunk 4 kk + (l >> 4)) meets 16 distinct chunks in every pass.  A transposed
// read (32 lanes on rows 4 g + i, four chunks each, one 8-byte half) covers each of
// the 16 chunks twice: two-way, the least any layout of 256-byte rows allows.
__device__ __forceinline__ constexpr int swz_f(int t) { return (t & 15) ^ ((t & 2) << 2); }
__device__ __forceinline__ int swz_off(int t, int c) { return t * D + (((c >> 3) ^ swz_f(t)) << 3) + (c & 7); }

// Operand lanes: r = l & 15, g = l >> 4; as a transposed-read source, lane l
// supplies row i = (l >> 2) & 3 and column group a = l & 3.
struct Lane {
  int r, g, a, i;
};

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 16 rows 16b..16b+15 of a [rows][C] bf16 matrix, columns col..col+127, as four
// row operands in natural k order: lane (r, g) gets row 16b + r, columns
// col + 32kk + 8g .. +7.  Rows past the buffer end read as zero.
struct Blk {
  bf16x8 v[4];
};
__device__ __forceinline__ Blk ld_blk_g(__amdgpu_buffer_rsrc_t rs, int C, int col, int b, const Lane& L) {
  Blk x;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    x.v[kk] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, 2 * ((16 * b + L.r) * C + col + 32 * kk + 8 * L.g), 0, 0));
  return x;
}

// Blocks below the diagonal, stored as 16 x 16 tiles: slot of block (R, C), R > C
__device__ __forceinline__ constexpr int low_slot(int R, int C) { return R * (R - 1) / 2 + C; }
// Blocks of T2 (R >= C), and the zero block (slot 10) that stands for R < C
__device__ __forceinline__ constexpr int t2_slot(int R, int C) { return C <= R ? R * (R + 1) / 2 + C : 10; }

// Block (bi, bj), bj <= bi, of A = strictly-lower(b_t e^{gamma_t - gamma_j} K K^T)
// from acc = K_bi K_bj^T: lane holds A[t = 16bi + 4g + i][j = 16bj + r].
// Diagonal blocks go to `at` in fp32, the others to `ab` in bf16, both transposed.
__device__ __forceinline__ void put_a(float* at, uint16_t (*ab)[16 * PB], const float* gam, const float* beta, int bi,
                                      int bj, f32x4 acc, const Lane& L) {
  const int j = 16 * bj + L.r;
  const float gj = gam[j];
  const f32x4 gt = *reinterpret_cast<const f32x4*>(&gam[16 * bi + 4 * L.g]);
  const f32x4 bt = *reinterpret_cast<const f32x4*>(&beta[16 * bi + 4 * L.g]);
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float f = bt[i] * __expf(gt[i] - gj) * acc[i];
    v[i] = (j < 16 * bi + 4 * L.g + i) ? f : 0.f;
  }
  if (bi == bj)
    *reinterpret_cast<float4*>(&at[(16 * bi + L.r) * PA + 4 * L.g]) = make_float4(v[0], v[1], v[2], v[3]);
  else
    st4bf(&ab[low_slot(bi, bj)][L.r * PB + 4 * L.g], v[0], v[1], v[2], v[3]);
}

// Block (bi, bj), bj <= bi, of P = M o Q K^T from acc = K_bj Q_bi^T (transposed):
// lane holds P[t = 16bi + r][j = 16bj + 4g + i].
__device__ __forceinline__ void put_p(uint16_t* p, const float* gam, int bi, int bj, f32x4 acc, const Lane& L) {
  const int t = 16 * bi + L.r;
  const float gt = gam[t];
  const f32x4 gj = *reinterpret_cast<const f32x4*>(&gam[16 * bj + 4 * L.g]);
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float f = __expf(gt - gj[i]) * acc[i];
    v[i] = (16 * bj + 4 * L.g + i <= t) ? f : 0.f;
  }
  st4bf(&p[t * PP + perm(16 * bj + 4 * L.g)], v[0], v[1], v[2], v[3]);
}

// 16x16x16 operands of the block products from transposed 16 x 16 tiles xt = X^T:
// A: lane gets X[r][4g..4g+3];  B: lane gets X[4g..4g+3][r]
__device__ __forceinline__ bf16x4 blk_a(const uint16_t* xt, const Lane& L) {
  return ldtr(xt + (4 * L.g + L.i) * PB + 4 * L.a);
}
__device__ __forceinline__ bf16x4 blk_b(const uint16_t* xt, const Lane& L) { return lds4(xt + L.r * PB + 4 * L.g); }

// Column c of T's block (R, C) in a lane's D tile (rows 4g + i) -> T2^T (column
// scaled by beta) and, when a later product reads it, the T^T tile `keep`.
__device__ __forceinline__ void put_t(uint16_t* keep, uint16_t* t2, const float* beta, int R, int C, f32x4 tv,
                                      const Lane& L) {
  const int jc = 16 * C + L.r;
  const float s = beta[jc];
  if (keep) st4bf(&keep[L.r * PB + 4 * L.g], tv[0], tv[1], tv[2], tv[3]);
  st4bf(&t2[t2_slot(R, C) * 16 * PB + L.r * PB + 4 * L.g], s * tv[0], s * tv[1], s * tv[2], s * tv[3]);
}

// The four 16x16 diagonal blocks of T = (I + A)^-1 by fp32 forward
// substitution, one column per lane: lane 16 rg + c solves block rg, column c,
// with all 16 rows in registers, so no lane exchange is needed.
__device__ __forceinline__ void solve_diag(const float* at, uint16_t (*tb)[16 * PB], uint16_t* t2, const float* beta,
                                           int lane) {
  const int c = lane & 15, rg = lane >> 4;
  float x[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) x[t] = (t == c) ? 1.f : 0.f;
  const float* col = &at[16 * rg * PA];
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
  const float s = beta[16 * rg + c];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4 w0, w2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = x[8 * h + 2 * e], x1 = x[8 * h + 2 * e + 1];
      w0[e] = pack_bf16x2(x0, x1);
      w2[e] = pack_bf16x2(s * x0, s * x1);
    }
    *reinterpret_cast<u32x4*>(&tb[rg][c * PB + 8 * h]) = w0;
    *reinterpret_cast<u32x4*>(&t2[t2_slot(rg, rg) * 16 * PB + c * PB + 8 * h]) = w2;
  }
}

// The blocks of T below the diagonal by MFMA block products:
//   T10 = -T11 A10 T00,  T32 = -T33 A32 T22,
//   [T20 T21; T30 T31] = -[T22 0; T32 T33] [A20 A21; A30 A31] [T00 0; T10 T11].
// (The wave's own LDS writes are visible to its later reads.)
__device__ __forceinline__ void solve_blocks(uint16_t (*ab)[16 * PB], uint16_t (*tb)[16 * PB], uint16_t* t2,
                                             const float* beta, const Lane& L) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 t10;
  {
    const f32x4 y10 = mfma16(blk_a(ab[low_slot(1, 0)], L), blk_b(tb[0], L), z);
    const f32x4 y32 = mfma16(blk_a(ab[low_slot(3, 2)], L), blk_b(tb[2], L), z);
    t10 = -mfma16(blk_a(tb[1], L), to_bf16x4(y10), z);
    const f32x4 t32 = -mfma16(blk_a(tb[3], L), to_bf16x4(y32), z);
    put_t(nullptr, t2, beta, 1, 0, t10, L);
    put_t(tb[4], t2, beta, 3, 2, t32, L);
  }
  {
    const bf16x4 b00 = blk_b(tb[0], L), b11 = blk_b(tb[1], L), b10 = to_bf16x4(t10);
    const bf16x4 a20 = blk_a(ab[low_slot(2, 0)], L), a21 = blk_a(ab[low_slot(2, 1)], L);
    const bf16x4 a30 = blk_a(ab[low_slot(3, 0)], L), a31 = blk_a(ab[low_slot(3, 1)], L);
    const f32x4 y20 = mfma16(a21, b10, mfma16(a20, b00, z));
    const f32x4 y21 = mfma16(a21, b11, z);
    const f32x4 y30 = mfma16(a31, b10, mfma16(a30, b00, z));
    const f32x4 y31 = mfma16(a31, b11, z);
    const bf16x4 t22 = blk_a(tb[2], L), t33 = blk_a(tb[3], L), t32a = blk_a(tb[4], L);
    const bf16x4 c20 = to_bf16x4(y20), c21 = to_bf16x4(y21);
    put_t(nullptr, t2, beta, 2, 0, -mfma16(t22, c20, z), L);
    put_t(nullptr, t2, beta, 2, 1, -mfma16(t22, c21, z), L);
    put_t(nullptr, t2, beta, 3, 0, -mfma16(t33, to_bf16x4(y30), mfma16(t32a, c20, z)), L);
    put_t(nullptr, t2, beta, 3, 1, -mfma16(t33, to_bf16x4(y31), mfma16(t32a, c21, z)), L);
  }
}

// LDS flag accesses (ds_read / ds_write, never flat, so a poll waits for LDS only)
typedef __attribute__((address_space(3))) int lds_int;
__device__ __forceinline__ void set_flag(int* flag, int v) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the data it publishes is written first
  *(volatile lds_int*)(flag) = v;
}
// Waits until the flag reaches `target`.  The wait is bounded (about 2^20
// polls), so a kernel can never hang on it; a wait that gives up raises
// kStatusWaitExpired (the call's results are then not valid).
__device__ __forceinline__ void wait_flag(const int* flag, int target) {
  bool done = false;
  for (int n = 0; n < (1 << 20) && !done; ++n) {
    const int v = __builtin_amdgcn_readfirstlane(*(const volatile lds_int*)(flag));
    done = v >= target;
    if (!done) __builtin_amdgcn_s_sleep(1);
  }
  if (!done && (threadIdx.x & 63) == 0) raise_status(kStatusWaitExpired);
  asm volatile("" ::: "memory");
}

// state row held in register row d (see the header)
__device__ __forceinline__ constexpr int sigma(int d) {
  return (d & ~31) | (((d >> 2) & 3) << 3) | (((d >> 4) & 1) << 2) | (d & 3);
}

}  // namespace
}  // namespace gdn
