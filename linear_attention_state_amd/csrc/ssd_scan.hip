// ssd_scan.hip -- packed-batch Mamba2 scan with per-sequence paged states, gfx950.
//
// The recurrence (Mamba2's selective SSM with A a scalar per head: Dao and
// Gu, "Transformers are SSMs", ICML 2024), per sequence and head m:
//   d_t = softplus(dt_t + dt_bias_m),  a_t = exp(d_t A_m)
//   h_t = a_t h_{t-1} + d_t x_t B_t^T          h: [P][N] fp32
//   y_t = h_t C_t + D_m x_t
// run chunk by chunk in its dual (quadratic) form.  With gamma_t the running
// sum of d A inside a chunk of 64 rows and Gamma = e^gamma:
//   Y = diag(Gamma) C S + (L o C B^T) X + D X,  L_tj = e^{gamma_t - gamma_j} d_j (j <= t)
//   S <- Gamma_last S + B^T diag(e^{gamma_last - gamma} d) X
// where S = h^T ([N][P]) enters the chunk and X, B, C are its rows.  Unlike
// the delta rule, nothing inside a chunk depends on S except the C S term.
//
// One 256-thread workgroup per (sequence, head), P = 64, N = 128.  Wave w owns
// state columns [16w, 16w + 16) (8 accumulator tiles over N, fp32) and output
// columns [16w, 16w + 16); rows 16w..16w+15 of the masked C B^T.  The chunk's
// C, B and X rows are staged in LDS in their natural row-major order; the
// transposed operands (B^T and X as the k side) are read with
// ds_read_b64_tr_b16.  All products are v_mfma_f32_16x16x32_bf16.
#include "gdn_device.h"

namespace gdn {
namespace {

constexpr int SBT = 64;   // chunk rows
constexpr int SN = 128;   // state size
constexpr int SP = 64;    // head size
constexpr int SNT = 256;  // threads

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// HP heads of one group per workgroup: C and B rows (and C B^T) are shared,
// the rest is per head.
template <int HP>
struct alignas(16) SsdSmem {
  uint16_t c[SBT * SN];        // C rows [t][n]; 16-byte chunks XOR-swizzled by row
  uint16_t b[SBT * SN];        // B rows [t][n]
  uint16_t x[HP][SBT * SP];    // X rows [t][p]
  uint16_t p[HP][SBT * SBT];   // L o C B^T [t][j], bf16
  uint16_t y[HP][SBT * SP];    // output rows [t][p], bf16
  float gam[HP][SBT];          // running sum of d A within the chunk
  float dd[HP][SBT];           // d_t (0 past the sequence end)
  float wv[HP][SBT];           // e^{gamma_last - gamma_j} d_j
};
static_assert(sizeof(SsdSmem<1>) <= 80 * 1024, "two workgroups per CU");
static_assert(sizeof(SsdSmem<2>) <= 160 * 1024, "LDS");

// Element offsets in the swizzled tiles: 256-byte rows (16 chunks) and 128-byte rows (8 chunks).
// On gfx950 the LDS serves 256 bytes a pass: a 16-byte read in four passes of 16 lanes, lane l
// in the pass keyed by (bit 5 of l, parity of bits 2-4 of l); an 8-byte read, plain or
// transposed, in two passes of 32 consecutive lanes.  Chunk c of a 256-byte row r sits at
// c ^ f(r), f(r) = (2 (r & 7) + b) ^ 8 b with b = bit 3 of r, so that every access below meets
// distinct banks in each pass: the 16-byte row-operand reads of B and C (rows i16 of a block,
// chunk 4 kk + g), the 8-byte reads of C rows, and the transposed reads of B (8 rows, two
// chunks, both halves).  The 128-byte-row function already does so for X, P and Y.
__device__ __forceinline__ int sw256(int row, int col) {
  const int b = (row >> 3) & 1;
  const int f = (2 * (row & 7) + b) ^ (8 * b);
  return row * 128 + ((((col >> 3) ^ f) << 3) | (col & 7));
}
__device__ __forceinline__ int sw128(int row, int col) {
  const int f = (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
  return row * 64 + ((((col >> 3) ^ f) << 3) | (col & 7));
}
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
  return u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 ld4(const uint16_t* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ bf16x8 join(bf16x4 lo, bf16x4 hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }
// ds_read_b64_tr_b16: within each 16-lane group, lane 16g + a + 4i reads 4
// consecutive bf16 of row (base + i) at columns c0 + 4a..c0 + 4a + 3, and lane
// 16g + n receives column c0 + n of rows base..base + 3.  Never under a partial exec mask.
__device__ __forceinline__ bf16x4 ldtr(const uint16_t* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<uint16_t*>(p))));
}

// k order of an operand: "natural" puts k = 8g + e at element e of lane group
// g; "pair" puts k = 4g + e (e < 4) and 16 + 4g + e - 4 (e >= 4), the order in
// which two accumulator tiles (rows 4g..4g+3 each) form one operand.  Both
// operands of a product use the same order.

__device__ __forceinline__ float softplus_f(float v) { return v > 20.f ? v : log1pf(__expf(v)); }

// HP = 1: 256 threads per (sequence, head), two workgroups per CU.  HP = 2:
// 512 threads per (sequence, pair of heads of one group): waves 4h..4h+3 own
// head h; the C and B rows are staged once and each C B^T tile is formed once
// and masked for both heads.
// Workgroups go by rank in `ord` (longest sequence first) when it is given:
// a pair's workgroup fills a CU, so the grid runs in rounds, and the longest
// chains must start in the first.
template <int HP>
__global__ __launch_bounds__(SNT * HP, 2 / HP) void ssd_chunk_kernel(SsdArgs a, SeqOrder ord) {
  constexpr int NTH = SNT * HP;
  __shared__ SsdSmem<HP> sm;
  const int H = a.num_heads, HB = H / HP;  // workgroups per sequence
  const int rank = blockIdx.x / HB;
  const int s = ord.n > 0 ? (rank < ord.n ? (int)ord.seq[rank] : a.num_seqs) : rank;
  int k = blockIdx.x % HB;
  if (HB % 8 == 0) k = (k % 8) * (HB / 8) + k / 8;  // heads of a group on one XCD (workgroups go round-robin over 8)
  if (s >= a.num_seqs || !seq_active(a.read_idx, a.write_idx, s, a.num_blocks)) return;
  const int r0 = a.cu[s], L = a.cu[s + 1] - r0;
  if (r0 < 0 || L < 2 || r0 + L > a.total_tokens) return;  // token kernel: L <= 1; offsets outside the rows
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, i16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = w >> 2, wl = w & 3, lt = tid & (SNT - 1);  // this wave's head, its wave and thread within the head
  const int m = HP * k + hh;
  const int grp = (HP * k) / (H / a.num_groups);
  const float Am = a.A[m], Dm = a.D ? a.D[m] : 0.f, bias = a.dt_bias ? a.dt_bias[m] : 0.f;

  // state: accumulator tile nb holds S[16nb + 4g + r][16wl + i16] = h[p][n]
  f32x4 S[8];
  {
    const gptr<const f32x4> src = as_global(reinterpret_cast<const f32x4*>(
        a.pool + (int64_t)a.read_idx[s] * a.pool_stride + (int64_t)m * SP * SN + (16 * wl + i16) * SN));
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) S[nb] = src[4 * nb + g];
  }
  gptr<f32x4> dst = as_global(reinterpret_cast<f32x4*>(
      a.pool + (int64_t)a.write_idx[s] * a.pool_stride + (int64_t)m * SP * SN + (16 * wl + i16) * SN));

  const int nch = (L + SBT - 1) / SBT;
  // chunk loads: C and B tiles 4/HP x 16 bytes per thread (16 threads per
  // row), each head's X 2 x 16 bytes (8 threads per row), d A of row `lane`
  // of each head in its first wave
  constexpr int NCB = 4 / HP;
  u32x4 rc[NCB], rb[NCB], rx[2];
  float rdt = 0.f;
  auto load = [&](int c) {
    const int row0 = r0 + c * SBT, nv = min(SBT, L - c * SBT);
    const __amdgpu_buffer_rsrc_t cs = make_rsrc(a.c + (int64_t)row0 * a.bc_stride + grp * SN,
                                                (uint32_t)(((int64_t)(nv - 1) * a.bc_stride + SN) * 2));
    const __amdgpu_buffer_rsrc_t bs = make_rsrc(a.b + (int64_t)row0 * a.bc_stride + grp * SN,
                                                (uint32_t)(((int64_t)(nv - 1) * a.bc_stride + SN) * 2));
    const __amdgpu_buffer_rsrc_t xs = make_rsrc(a.x + (int64_t)row0 * a.x_stride + m * SP,
                                                (uint32_t)(((int64_t)(nv - 1) * a.x_stride + SP) * 2));
    // d A first, by every wave (wave 0 of each head uses it), rows past the end
    // reading 0: no memory access of the step sits under a branch and the rows
    // follow this load, so the waits for them and for it never cover the
    // previous chunk's y stores
    const __amdgpu_buffer_rsrc_t ds = make_rsrc(a.dt + (int64_t)row0 * H + m, (uint32_t)(((nv - 1) * H + 1) * 4));
    rdt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ds, lane < nv ? lane * H * 4 : -1, 0, 0));
#pragma unroll
    for (int i = 0; i < NCB; ++i) {
      const int q = tid + NTH * i, t = q >> 4, cc = q & 15;
      const int off = t < nv ? (int)((t * a.bc_stride + 8 * cc) * 2) : -1;  // rows past the end read 0
      rc[i] = __builtin_amdgcn_raw_buffer_load_b128(cs, (uint32_t)off, 0, 0);
      rb[i] = __builtin_amdgcn_raw_buffer_load_b128(bs, (uint32_t)off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = lt + SNT * i, t = q >> 3, cc = q & 7;
      const int off = t < nv ? (int)((t * a.x_stride + 8 * cc) * 2) : -1;
      rx[i] = __builtin_amdgcn_raw_buffer_load_b128(xs, (uint32_t)off, 0, 0);
    }
  };
  if (nch > 0) load(0);
  // a chunk's output rows go out at the start of the next step, before the
  // waits for that step's rows, so that on every path into the loop the same
  // accesses follow those loads and the waits never cover the stores (the
  // first step's stores have no rows: the range check drops them)
  u32x4 yst[2] = {};
  int yoff[2] = {-1, -1};
  __amdgpu_buffer_rsrc_t ysr = make_rsrc(a.y, 0u);
  for (int c = 0; c < nch; ++c) {
    const int nv = min(SBT, L - c * SBT);
#pragma unroll
    for (int i = 0; i < 2; ++i) __builtin_amdgcn_raw_buffer_store_b128(yst[i], ysr, yoff[i], 0, 0);
    // no barrier before the staging: every read of C, B, X and the gamma rows
    // of the previous chunk came before its last barrier, and the only reads
    // since (its output rows) touch none of what is staged here
#pragma unroll
    for (int i = 0; i < NCB; ++i) {
      const int q = tid + NTH * i, t = q >> 4, cc = q & 15;
      *reinterpret_cast<u32x4*>(&sm.c[sw256(t, 8 * cc)]) = rc[i];
      *reinterpret_cast<u32x4*>(&sm.b[sw256(t, 8 * cc)]) = rb[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = lt + SNT * i, t = q >> 3, cc = q & 7;
      *reinterpret_cast<u32x4*>(&sm.x[hh][sw128(t, 8 * cc)]) = rx[i];
    }
    if (wl == 0) {
      float d = 0.f;
      if (lane < nv) d = a.softplus ? softplus_f(rdt + bias) : rdt + bias;
      // running sum of d A over the chunk's rows (lanes): in lane registers
      // (row shifts and broadcasts), not through LDS permutes, since every
      // other wave waits for it at the next barrier
      const float v = wave_prefix_sum(d * Am);
      const float last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
      sm.gam[hh][lane] = v;
      sm.dd[hh][lane] = d;
      sm.wv[hh][lane] = __expf(last - v) * d;
    }
    if (c + 1 < nch) load(c + 1);  // the next chunk's rows stay in flight through this one
    lds_barrier();

    // rows 16wl..16wl+15 of L o C B^T (blocks right of the diagonal are
    // zero), computed transposed (B C^T): a lane holds 4 consecutive j of row
    // t.  With two heads, the waves of head h form the j blocks of parity h
    // and mask each tile for both heads.
    {
      const int t = 16 * wl + i16;
#pragma unroll
      for (int jj = 0; jj < 4 / HP; ++jj) {
        const int jb = HP == 1 ? jj : 2 * jj + hh;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (jb <= wl) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            acc = mma(ld8(&sm.b[sw256(16 * jb + i16, 32 * kk + 8 * g)]), ld8(&sm.c[sw256(t, 32 * kk + 8 * g)]), acc);
        }
        const int j0 = 16 * jb + 4 * g;
#pragma unroll
        for (int e = 0; e < HP; ++e) {
          const float gt = sm.gam[e][t];
          const f32x4 gj = *reinterpret_cast<const f32x4*>(&sm.gam[e][j0]);
          const f32x4 dj = *reinterpret_cast<const f32x4*>(&sm.dd[e][j0]);
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = j0 + r <= t ? acc[r] * __expf(gt - gj[r]) * dj[r] : 0.f;
          *reinterpret_cast<u32x2*>(&sm.p[e][sw128(t, j0)]) = pack4(v[0], v[1], v[2], v[3]);
        }
      }
    }
    // S as the k side of C S, pair order: tiles 2kk and 2kk + 1
    bf16x8 sop[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sop[kk][e] = (__bf16)S[2 * kk][e];
        sop[kk][4 + e] = (__bf16)S[2 * kk + 1][e];
      }
    // X as the k side (rows j, column 16wl + i16), pair order
    const uint16_t* X = sm.x[hh];
    bf16x8 xop[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int a4 = lane & 3, i4 = (lane >> 2) & 3;
      xop[kk] = join(ldtr(&X[sw128(32 * kk + 4 * g + i4, 16 * wl + 4 * a4)]),
                     ldtr(&X[sw128(32 * kk + 16 + 4 * g + i4, 16 * wl + 4 * a4)]));
    }
    lds_barrier();  // every row of L o C B^T is written

    // Y[:, 16wl..16wl+15] = Gamma (C S) + (L o C B^T) X + D X, computed
    // transposed (S^T C^T + X^T P^T): a lane holds 4 consecutive p of one row t
    const uint16_t* P = sm.p[hh];
    uint16_t* Y = sm.y[hh];
    const float* gam = sm.gam[hh];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      f32x4 ys = {0.f, 0.f, 0.f, 0.f}, yp = {0.f, 0.f, 0.f, 0.f};
      const int tr = 16 * tb + i16;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        ys = mma(sop[kk], join(ld4(&sm.c[sw256(tr, 32 * kk + 4 * g)]), ld4(&sm.c[sw256(tr, 32 * kk + 16 + 4 * g)])), ys);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        if (kk <= tb / 2)
          yp = mma(xop[kk], join(ld4(&P[sw128(tr, 32 * kk + 4 * g)]), ld4(&P[sw128(tr, 32 * kk + 16 + 4 * g)])), yp);
      const u32x2 xr = *reinterpret_cast<const u32x2*>(&X[sw128(tr, 16 * wl + 4 * g)]);
      const float egt = __expf(gam[tr]);
      float yv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t xw2 = xr[r / 2];
        const float xv = __uint_as_float((r & 1) ? (xw2 & 0xffff0000u) : (xw2 << 16));
        yv[r] = egt * ys[r] + yp[r] + Dm * xv;
      }
      *reinterpret_cast<u32x2*>(&Y[sw128(tr, 16 * wl + 4 * g)]) = pack4(yv[0], yv[1], yv[2], yv[3]);
    }
    // S <- Gamma_last S + B^T diag(w) X
    {
      const float glast = __expf(gam[SBT - 1]);
      bf16x8 xw[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 32 * kk + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
          xw[kk][e] = (__bf16)((float)xop[kk][e] * sm.wv[hh][j]);
        }
      const int a4 = lane & 3, i4 = (lane >> 2) & 3;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        f32x4 acc = S[nb] * glast;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          acc = mma(join(ldtr(&sm.b[sw256(32 * kk + 4 * g + i4, 16 * nb + 4 * a4)]),
                         ldtr(&sm.b[sw256(32 * kk + 16 + 4 * g + i4, 16 * nb + 4 * a4)])),
                    xw[kk], acc);
        S[nb] = acc;
      }
    }
    lds_barrier();  // every output row is staged
    // this chunk's output rows, stored at the start of the next step (rows
    // past the end are dropped by the buffer's range check)
    ysr = make_rsrc(a.y + ((int64_t)(r0 + c * SBT) * H + m) * SP, (uint32_t)(((nv - 1) * H + 1) * SP * 2));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = lt + SNT * i, t = q >> 3, cc = q & 7;
      yst[i] = *reinterpret_cast<const u32x4*>(&Y[sw128(t, 8 * cc)]);
      yoff[i] = t < nv ? (t * H * SP + 8 * cc) * 2 : -1;
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) __builtin_amdgcn_raw_buffer_store_b128(yst[i], ysr, yoff[i], 0, 0);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) dst[4 * nb + g] = S[nb];
}

// One token (or none) per sequence: the recurrence step itself, in fp32, as a
// streaming read-modify-write of the head's state.  256 threads per (sequence,
// head); pass i moves 4 KiB of h: thread t holds h[p][n..n+3] with
// p = 8i + t / 32 and n = 4 (t % 32), so every load and store of a wave covers
// 1 KiB contiguously.  y_p sums over the 32 lanes that hold row p.  A sequence
// of length 0 copies its state.
__global__ __launch_bounds__(SNT) void ssd_token_kernel(SsdArgs a) {
  const int H = a.num_heads;
  const int s = blockIdx.x / H;
  int m = blockIdx.x % H;
  if (H % 8 == 0) m = (m % 8) * (H / 8) + m / 8;
  if (s >= a.num_seqs || !seq_active(a.read_idx, a.write_idx, s, a.num_blocks)) return;
  const int r0 = a.cu[s], L = a.cu[s + 1] - r0;
  if (r0 < 0 || L < 0 || L > 1 || r0 + L > a.total_tokens) return;
  const int tid = threadIdx.x, lane = tid & 63, n0 = 4 * (tid & 31), prow = tid >> 5;
  const int64_t head = (int64_t)m * SP * SN;
  const f32x4* src = reinterpret_cast<const f32x4*>(a.pool + (int64_t)a.read_idx[s] * a.pool_stride + head) + tid;
  f32x4* dst = reinterpret_cast<f32x4*>(a.pool + (int64_t)a.write_idx[s] * a.pool_stride + head) + tid;
  f32x4 h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = __builtin_nontemporal_load(src + SNT * i);
  if (L == 1) {
    const int grp = m / (H / a.num_groups);
    const float bias = a.dt_bias ? a.dt_bias[m] : 0.f;
    float d = a.dt[(int64_t)r0 * H + m] + bias;
    if (a.softplus) d = softplus_f(d);
    const float decay = __expf(d * a.A[m]);
    const float Dm = a.D ? a.D[m] : 0.f;
    const uint16_t* xr = a.x + (int64_t)r0 * a.x_stride + m * SP;
    const u32x2 bw = *reinterpret_cast<const u32x2*>(a.b + (int64_t)r0 * a.bc_stride + grp * SN + n0);
    const u32x2 cw = *reinterpret_cast<const u32x2*>(a.c + (int64_t)r0 * a.bc_stride + grp * SN + n0);
    float bn[4], cn[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t bb = bw[e / 2], cc = cw[e / 2];
      bn[e] = __uint_as_float((e & 1) ? (bb & 0xffff0000u) : (bb << 16));
      cn[e] = __uint_as_float((e & 1) ? (cc & 0xffff0000u) : (cc << 16));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = 8 * i + prow;
      const float xp = bf16_bits_to_f32(xr[p]);
      const float dx = d * xp;
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[i][e] = decay * h[i][e] + dx * bn[e];
        acc += h[i][e] * cn[e];
      }
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
      if ((lane & 31) == 0) a.y[((int64_t)r0 * H + m) * SP + p] = f32_to_bf16_bits(acc + Dm * xp);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) __builtin_nontemporal_store(h[i], dst + SNT * i);
}

}  // namespace

bool ssd_supported(int head_dim, int state_dim) { return head_dim == SP && state_dim == SN; }

hipError_t launch_ssd_token(const SsdArgs& a, hipStream_t st) {
  if (a.num_seqs <= 0 || a.num_heads <= 0) return hipSuccess;
  const int64_t blocks = (int64_t)a.num_seqs * a.num_heads;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ssd_token_kernel, dim3((unsigned)blocks), dim3(SNT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_ssd(const SsdArgs& a, const SeqOrder& ord, hipStream_t st) {
  if (a.num_seqs <= 0 || a.num_heads <= 0) return hipSuccess;
  if (ord.n < 0 || ord.n > kMaxOrder || ord.n > a.num_seqs) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)(ord.n > 0 ? ord.n : a.num_seqs) * a.num_heads;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if ((a.num_heads / a.num_groups) % 2 == 0)  // pairs of heads of one group share B, C and C B^T
    hipLaunchKernelGGL(ssd_chunk_kernel<2>, dim3((unsigned)(blocks / 2)), dim3(2 * SNT), 0, st, a, ord);
  else
    hipLaunchKernelGGL(ssd_chunk_kernel<1>, dim3((unsigned)blocks), dim3(SNT), 0, st, a, ord);
  return hipGetLastError();
}

GDN_STATUS_ACCESSOR(status_ssd)

}  // namespace gdn
