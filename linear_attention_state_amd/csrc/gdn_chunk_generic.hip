// gdn_chunk_generic.hip -- chunked prefill of the gated delta rule for every
// head size of the layer (d_k, d_v in {16, 32, 64, 128}) and both activation
// dtypes, computed in fp32 on the fp32 MFMA (v_mfma_f32_16x16x4_f32).  The bf16
// layer with d_k = d_v = 128 takes the faster bf16 kernel of gdn_chunk.hip; this
// one serves every other shape, and the all-fp32 layer, whose outputs must match
// an fp64 evaluation far more closely than bf16 operands allow.
//
// Recurrence (Gated Delta Networks, Yang et al., ICLR 2025), state [d_k][d_v]
// carried per request in its cache block (page "Continuous batching for linear
// attention layers", PR description):
//     S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t,
// evaluated 64 rows at a time in the WY / UT form (chunkwise DeltaNet, Yang et
// al., NeurIPS 2024), with gamma the running sum of g inside the chunk:
//     A  = strictly-lower( b_t e^{gamma_t-gamma_j} k_t.k_j ),   T = (I + A)^-1
//     U  = T diag(b) (V - diag(e^gamma) K S)
//     O  = diag(e^gamma) Q S + (M o Q K^T) U,   M_tj = e^{gamma_t-gamma_j} (j <= t)
//     S <- e^{gamma_last} S + K^T diag(e^{gamma_last-gamma}) U
// Only differences of running sums are exponentiated (every factor <= 1).
//
// One 256-thread workgroup (4 waves) per (sequence, value head), chunk by chunk
// in phases separated by workgroup barriers: the chunk's q, k, v rows (the conv
// output, already normalised) into LDS as fp32; the ten 16 x 16 blocks of A and
// of P = M o Q K^T; T by fp32 forward substitution on the diagonal blocks and
// block products below them (one wave); then the state pass, in which wave w
// owns the 16-column tiles nt = w, w + 4, ... of S in registers.
//
// fp32 MFMA 16x16x4 layout (lane l, r = l & 15, kq = l >> 4): A: row r, k = kq;
// B: column r, k = kq; D: column r, rows 4 kq + {0,1,2,3}.  A D tile (the state,
// X, U) serves directly as the B operand of a later product when that product's
// k steps run in the order k = 4 kq + s (step s takes element s of the tile),
// with the A operand read from LDS in the same order.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int GT = 256;          // threads per workgroup
constexpr int GC = 64;           // chunk length
constexpr int GPA = GC + 4;      // pitch of the 64 x 64 fp32 matrices

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int DK, int DV>
struct alignas(16) GSmem {
  float k[GC][DK + 4];
  float q[GC][DK + 4];
  float v[GC][DV + 4];
  float a[GC][GPA];  // A (blocks above the diagonal stay zero)
  float t[GC][GPA];  // T (b enters through the rows of X)
  float p[GC][GPA];  // P = M o Q K^T
  float gam[GC], eg[GC], ed[GC], bet[GC];
};

// 4 consecutive activations as fp32
template <bool BF16>
__device__ __forceinline__ float4 load4(const void* y, int64_t idx) {
  if constexpr (BF16) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(y) + idx);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(y) + idx);
  }
}

// 4 consecutive activations as raw bits (8 bytes in bf16, 16 in fp32), and as fp32
template <bool BF16>
struct Raw4 {
  typedef typename std::conditional<BF16, uint2, float4>::type type;
};
template <bool BF16>
__device__ __forceinline__ typename Raw4<BF16>::type load_raw4(const void* y, int64_t idx) {
  if constexpr (BF16) return *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(y) + idx);
  else return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(y) + idx);
}
template <bool BF16>
__device__ __forceinline__ float4 raw4_f32(typename Raw4<BF16>::type w) {
  if constexpr (BF16)
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xffff0000u));
  else return w;
}

// pair index 0..9 -> block (R, C), C <= R, in the order (0,0) (1,0) (1,1) (2,0) ...
__device__ __forceinline__ void pair_rc(int pr, int& R, int& C) {
  R = pr >= 6 ? 3 : pr >= 3 ? 2 : pr >= 1 ? 1 : 0;
  C = pr - R * (R + 1) / 2;
}

template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(GT) void chunk_generic_kernel(ScanArgs a, SeqOrder ord) {
  __shared__ GSmem<DK, DV> sm;
  constexpr int NKT = DK / 16, NVT = DV / 16, NVW = (NVT + 3) / 4;
  const int Hv = a.num_v_heads, Hk = a.num_k_heads, C = a.channels;
  const int rank = blockIdx.x / Hv;
  const int m = blockIdx.x % Hv;
  const int s = ord.n > 0 ? (rank < ord.n ? (int)ord.seq[rank] : a.num_seqs) : rank;
  if (s >= a.num_seqs) return;
  const int r0 = a.cu[s], L = a.cu[s + 1] - r0;
  if (L < a.min_len || L > a.max_len) return;
  if (!seq_active(a.read_idx, a.write_idx, s, a.num_blocks)) return;
  const int h = m / (Hv / Hk);
  const int N = (L + GC - 1) / GC;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;

  for (int i = tid; i < GC * GPA; i += GT) {
    (&sm.a[0][0])[i] = 0.f;
    (&sm.t[0][0])[i] = 0.f;
    (&sm.p[0][0])[i] = 0.f;
  }
  // the state: wave wv owns column tiles nt = wv + 4 j; lane holds rows 16 dt + 4 lq + i, column 16 nt + lr
  const int64_t head_off = (int64_t)m * DK * DV;
  const float* s_in = reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.ssm_pool) +
                                                     (int64_t)__builtin_amdgcn_readfirstlane(a.read_idx[s]) *
                                                         a.ssm_stride) + head_off;
  f32x4 S[NVW][NKT];
#pragma unroll
  for (int j = 0; j < NVW; ++j) {
    const int nt = wv + 4 * j;
#pragma unroll
    for (int dt = 0; dt < NKT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[j][dt][i] = nt < NVT ? s_in[(16 * dt + 4 * lq + i) * DV + 16 * nt + lr] : 0.f;
  }

  // The chunk's q, k, v rows: groups of 4 activations, group i = tid + GT j of
  // the [GC][2 DK + DV] rows (a thread's NL groups).  Where their raw bits fit
  // the registers beside the state pass (PF), chunk c + 1's rows load while
  // chunk c is computed; else each chunk loads its own at the start.
  constexpr int W4 = (2 * DK + DV) / 4;
  constexpr int NL = GC * W4 / GT;
  static_assert(GC * W4 % GT == 0, "whole groups per thread");
  constexpr bool PF = NL * (BF16 ? 2 : 4) <= 48 && DK * DV < D * D;  // the 128 x 128 state leaves no room
  typename Raw4<BF16>::type raw[PF ? NL : 1];
  float gpre = 0.f, bpre = 0.f;
  auto group = [&](int i, int& t, int& gcol, float*& dst) {
    t = i / W4;
    const int col = 4 * (i % W4);
    if (col < DK) {
      gcol = h * DK + col;
      dst = &sm.q[t][col];
    } else if (col < 2 * DK) {
      gcol = (Hk + h) * DK + col - DK;
      dst = &sm.k[t][col - DK];
    } else {
      gcol = 2 * Hk * DK + m * DV + col - 2 * DK;
      dst = &sm.v[t][col - 2 * DK];
    }
  };
  // rows past the end of the sequence load as zero
  auto prefetch = [&](int c) {
    const int nv = min(GC, L - c * GC);
    const int64_t row0 = (int64_t)r0 + c * GC;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      int t, gcol;
      float* dst;
      group(tid + GT * j, t, gcol, dst);
      raw[PF ? j : 0] = t < nv ? load_raw4<BF16>(a.y, (row0 + t) * C + gcol) : typename Raw4<BF16>::type{};
    }
    if (wv == 0) {
      gpre = lane < nv ? a.g[(row0 + lane) * Hv + m] : 0.f;
      bpre = lane < nv ? a.beta[(row0 + lane) * Hv + m] : 0.f;
    }
  };
  // Split prefetch (SP, fp32 where PF does not fit): chunk c + 1's q and k rows
  // into registers while chunk c is computed, and chunk c's v rows issued at
  // its start, in flight through the A and P products (v is first read by the
  // state pass).
  constexpr bool SP = !PF && !BF16;
  constexpr int WQK = DK / 2, WV = DV / 4;  // groups per row of q and k, of v
  constexpr int NQK = GC * WQK / GT, NV = GC * WV / GT;
  static_assert(GC * WQK % GT == 0 && GC * WV % GT == 0, "whole groups per thread");
  float4 qkraw[SP ? NQK : 1], vraw[SP ? NV : 1];
  auto prefetch_qk = [&](int c) {
    const int nv = min(GC, L - c * GC);
    const int64_t row0 = (int64_t)r0 + c * GC;
#pragma unroll
    for (int j = 0; j < NQK; ++j) {
      const int i = tid + GT * j, t = i / WQK, col = 4 * (i % WQK);
      const int gcol = col < DK ? h * DK + col : (Hk + h) * DK + col - DK;
      qkraw[SP ? j : 0] = t < nv ? load4<false>(a.y, (row0 + t) * C + gcol) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (wv == 0) {
      gpre = lane < nv ? a.g[(row0 + lane) * Hv + m] : 0.f;
      bpre = lane < nv ? a.beta[(row0 + lane) * Hv + m] : 0.f;
    }
  };
  if constexpr (PF) prefetch(0);
  if constexpr (SP) prefetch_qk(0);

  for (int c = 0; c < N; ++c) {
    const int nv = min(GC, L - c * GC);
    const int64_t row0 = (int64_t)r0 + c * GC;
    __syncthreads();  // the previous chunk's tiles are read
    // ---- q, k, v rows (zero past the end), g and b
    if constexpr (PF) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        int t, gcol;
        float* dst;
        group(tid + GT * j, t, gcol, dst);
        *reinterpret_cast<float4*>(dst) = raw4_f32<BF16>(raw[j]);
      }
    } else if constexpr (SP) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int i = tid + GT * j, t = i / WV, col = 4 * (i % WV);
        vraw[j] = t < nv ? load4<false>(a.y, (row0 + t) * C + 2 * Hk * DK + m * DV + col) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < NQK; ++j) {
        const int i = tid + GT * j, t = i / WQK, col = 4 * (i % WQK);
        float* dst = col < DK ? &sm.q[t][col] : &sm.k[t][col - DK];
        *reinterpret_cast<float4*>(dst) = qkraw[j];
      }
    } else {
      for (int i = tid; i < GC * W4; i += GT) {
        int t, gcol;
        float* dst;
        group(i, t, gcol, dst);
        const float4 val = t < nv ? load4<BF16>(a.y, (row0 + t) * C + gcol) : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(dst) = val;
      }
      if (wv == 0) {
        gpre = lane < nv ? a.g[(row0 + lane) * Hv + m] : 0.f;
        bpre = lane < nv ? a.beta[(row0 + lane) * Hv + m] : 0.f;
      }
    }
    if (wv == 0) {
      const int t = lane;
      const float g = gpre;
      const float b = bpre;
      const float gm = wave_prefix_sum(g);  // rows past the end add nothing
      const float glast = __shfl(gm, GC - 1);
      sm.gam[t] = gm;
      sm.eg[t] = __expf(gm);
      sm.ed[t] = __expf(glast - gm);
      sm.bet[t] = b;
    }
    __syncthreads();
    if constexpr (PF) {
      if (c + 1 < N) prefetch(c + 1);  // in flight through this chunk's products
    }
    if constexpr (SP) {
      if (c + 1 < N) prefetch_qk(c + 1);
    }
    // ---- blocks of A (even w) and P (odd w): lane holds D[t = 16R + 4 lq + i][j = 16Cb + lr].
    // The channel sum runs in the order 16 g + 4 lq + s, so that a lane's four
    // channels of group g are one 16-byte read of each operand row.
    for (int w = wv; w < 20; w += 4) {
      int R, Cb;
      pair_rc(w >> 1, R, Cb);
      const bool isp = w & 1;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < DK / 16; ++g) {
        const f32x4 xv = *reinterpret_cast<const f32x4*>(isp ? &sm.q[16 * R + lr][16 * g + 4 * lq] : &sm.k[16 * R + lr][16 * g + 4 * lq]);
        const f32x4 yv = *reinterpret_cast<const f32x4*>(&sm.k[16 * Cb + lr][16 * g + 4 * lq]);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma4(xv[s], yv[s], acc);
      }
      const int j = 16 * Cb + lr;
      const float gj = sm.gam[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * R + 4 * lq + i;
        const float e = __expf(fminf(sm.gam[t] - gj, 0.f));  // <= 1 where it is used (j <= t)
        if (isp)
          sm.p[t][j] = j <= t ? e * acc[i] : 0.f;
        else
          sm.a[t][j] = j < t ? sm.bet[t] * e * acc[i] : 0.f;
      }
    }
    if constexpr (SP) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int i = tid + GT * j, t = i / WV, col = 4 * (i % WV);
        *reinterpret_cast<float4*>(&sm.v[t][col]) = vraw[j];
      }
    }
    __syncthreads();
    // ---- T = (I + A)^-1 (one wave): diagonal blocks by forward substitution
    // (lane: block lq, column lr), then T_RC = -T_RR sum_{k=C}^{R-1} A_Rk T_kC
    if (wv == 0) {
      {
        const int bo = 16 * lq;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) x[t] = t == lr ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 15; ++j) {
          const float xj = x[j];
#pragma unroll
          for (int t = j + 1; t < 16; ++t) x[t] -= sm.a[bo + t][bo + j] * xj;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) sm.t[bo + t][bo + lr] = x[t];
      }
#pragma unroll
      for (int R = 1; R < 4; ++R)
#pragma unroll
        for (int Cb = 0; Cb < R; ++Cb) {
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = Cb; kb < R; ++kb)
#pragma unroll
            for (int st = 0; st < 4; ++st)
              y = mfma4(sm.a[16 * R + lr][16 * kb + 4 * st + lq], sm.t[16 * kb + 4 * st + lq][16 * Cb + lr], y);
          f32x4 tv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int st = 0; st < 4; ++st) tv = mfma4(sm.t[16 * R + lr][16 * R + 4 * lq + st], y[st], tv);
#pragma unroll
          for (int i = 0; i < 4; ++i) sm.t[16 * R + 4 * lq + i][16 * Cb + lr] = -tv[i];
        }
    }
    __syncthreads();
    // ---- state pass over the wave's column tiles
    const float glast = sm.eg[GC - 1];
#pragma unroll
    for (int j = 0; j < NVW; ++j) {
      const int nt = wv + 4 * j;
      if (nt >= NVT) break;  // uniform
      const int col = 16 * nt + lr;
      f32x4 ks[4], qs[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) ks[tb] = qs[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < NKT; ++dt)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const float sb = S[j][dt][st];
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) {
            ks[tb] = mfma4(sm.k[16 * tb + lr][16 * dt + 4 * lq + st], sb, ks[tb]);
            qs[tb] = mfma4(sm.q[16 * tb + lr][16 * dt + 4 * lq + st], sb, qs[tb]);
          }
        }
      // diag(b) X with X = V - e^gamma K S (in place of K S), then U = T diag(b) X
      f32x4 u[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * tb + 4 * lq + i;
          ks[tb][i] = sm.bet[t] * (sm.v[t][col] - sm.eg[t] * ks[tb][i]);
        }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        u[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jb = 0; jb <= tb; ++jb)
#pragma unroll
          for (int st = 0; st < 4; ++st) u[tb] = mfma4(sm.t[16 * tb + lr][16 * jb + 4 * lq + st], ks[jb][st], u[tb]);
      }
      // O = e^gamma Q S + P U, rows past the end dropped
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jb = 0; jb <= tb; ++jb)
#pragma unroll
          for (int st = 0; st < 4; ++st) o = mfma4(sm.p[16 * tb + lr][16 * jb + 4 * lq + st], u[jb][st], o);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * tb + 4 * lq + i;
          const float ov = sm.eg[t] * qs[tb][i] + o[i];
          if (t < nv) {
            const int64_t oi = (row0 + t) * Hv * DV + (int64_t)m * DV + col;
            if constexpr (BF16)
              reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_bits(ov);
            else
              reinterpret_cast<float*>(a.out)[oi] = ov;
          }
        }
      }
      // S <- e^{gamma_last} S + (e^{gamma_last - gamma} o K)^T U
#pragma unroll
      for (int dt = 0; dt < NKT; ++dt) {
        S[j][dt] *= glast;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const int t = 16 * tb + 4 * lq + st;
            S[j][dt] = mfma4(sm.ed[t] * sm.k[t][16 * dt + lr], u[tb][st], S[j][dt]);
          }
      }
    }
  }
  float* s_out = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ssm_pool) +
                                          (int64_t)__builtin_amdgcn_readfirstlane(a.write_idx[s]) * a.ssm_stride) +
                 head_off;
#pragma unroll
  for (int j = 0; j < NVW; ++j) {
    const int nt = wv + 4 * j;
    if (nt >= NVT) break;
#pragma unroll
    for (int dt = 0; dt < NKT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_out[(16 * dt + 4 * lq + i) * DV + 16 * nt + lr] = S[j][dt][i];
  }
}

template <int DK, int DV>
hipError_t gen_launch(const ScanArgs& a, const SeqOrder& order, bool bf16, hipStream_t st) {
  const int rows = order.n > 0 ? order.n : a.num_seqs;
  if (bf16)
    hipLaunchKernelGGL((chunk_generic_kernel<DK, DV, true>), dim3(rows * a.num_v_heads), dim3(GT), 0, st, a, order);
  else
    hipLaunchKernelGGL((chunk_generic_kernel<DK, DV, false>), dim3(rows * a.num_v_heads), dim3(GT), 0, st, a, order);
  return hipGetLastError();
}

template <int DK>
hipError_t gen_dv(const ScanArgs& a, const SeqOrder& order, int dv, bool bf16, hipStream_t st) {
  switch (dv) {
    case 16: return gen_launch<DK, 16>(a, order, bf16, st);
    case 32: return gen_launch<DK, 32>(a, order, bf16, st);
    case 64: return gen_launch<DK, 64>(a, order, bf16, st);
    case 128: return gen_launch<DK, 128>(a, order, bf16, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool chunk_generic_supported(int dk, int dv) {
  auto ok = [](int d) { return d == 16 || d == 32 || d == 64 || d == 128; };
  return ok(dk) && ok(dv);
}

hipError_t launch_chunk_generic(const ScanArgs& a, const SeqOrder& order, int dk, int dv, bool bf16,
                                hipStream_t st) {
  if (!chunk_generic_supported(dk, dv) || !a.y) return hipErrorInvalidValue;
  switch (dk) {
    case 16: return gen_dv<16>(a, order, dv, bf16, st);
    case 32: return gen_dv<32>(a, order, dv, bf16, st);
    case 64: return gen_dv<64>(a, order, dv, bf16, st);
    default: return gen_dv<128>(a, order, dv, bf16, st);
  }
}

}  // namespace gdn
