// gdn_recurrent.hip -- token-by-token gated delta rule for gfx950: the decode
// path (one token per sequence) and the all-fp32 path.
//
// Recurrence (Gated Delta Networks, Yang et al., ICLR 2025), state of a value
// head stored [d_k][d_v] with d_v fastest, carried per request in its block
// (page "Continuous batching for linear attention layers", PR description):
//     S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t.
// Evaluated in delta form: kS = S^T k, u = b (v - a kS), S <- a S + k u^T, and
// o = a S_{t-1}^T q + (k.q) u, so one reduction pass over d_k serves both kS and
// the output.
//
// One workgroup of 256 threads owns one (sequence, value head).  A thread holds
// 4 adjacent d_v columns of d_k/(256/(d_v/4)) rows in registers; a wave's load
// instruction therefore covers 64/(d_v/4) whole state rows (1 KB for d_v=128),
// fully coalesced.  For a one-token sequence the kernel is a pure streaming
// read-modify-write of the 64 KB head state: reductions over d_k use lane
// shuffles inside the wave and one LDS exchange across the four waves; no MFMA.
#include "gdn_device.h"

namespace gdn {
namespace {

template <bool BF16>
__device__ __forceinline__ float ld1(const void* base, int64_t i) {
  if constexpr (BF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
  else return reinterpret_cast<const float*>(base)[i];
}

template <bool BF16>
__device__ __forceinline__ float4 ld4(const void* base, int64_t i) {
  if constexpr (BF16) {
    uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + i);
  }
}

template <bool BF16>
__device__ __forceinline__ void st4(void* base, int64_t i, float4 v) {
  if constexpr (BF16) {
    uint2 u;
    u.x = (uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
    u.y = (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + i) = u;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + i) = v;
  }
}

__device__ __forceinline__ float4 f4_fma(float a, float4 x, float4 y) {
  return make_float4(fmaf(a, x.x, y.x), fmaf(a, x.y, y.y), fmaf(a, x.z, y.z), fmaf(a, x.w, y.w));
}

template <bool BF16, int DK, int DV>
__global__ __launch_bounds__(256) void recurrent_kernel(ScanArgs a) {
  constexpr int NT = 256;
  constexpr int C4 = DV / 4;          // threads across one state row
  constexpr int RG = NT / C4;         // row groups
  constexpr int RPT = (DK + RG - 1) / RG;
  constexpr int NW = NT / 64;
  static_assert(C4 <= 64 && (64 % C4) == 0, "row group must fit a wave");

  const int s = blockIdx.x, m = blockIdx.y;
  if (s >= a.num_seqs) return;
  const int r0 = a.cu[s];
  const int L = a.cu[s + 1] - r0;
  if (L < a.min_len || L > a.max_len) return;
  if (!seq_active(a.read_idx, a.write_idx, s, a.num_blocks)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c4 = tid % C4, rg = tid / C4;
  const int h = m / (a.num_v_heads / a.num_k_heads);
  const int64_t head_off = (int64_t)m * DK * DV;
  const float* S0 = reinterpret_cast<const float*>(
      reinterpret_cast<const char*>(a.ssm_pool) + (int64_t)a.read_idx[s] * a.ssm_stride) + head_off;
  float* S1 = reinterpret_cast<float*>(
      reinterpret_cast<char*>(a.ssm_pool) + (int64_t)a.write_idx[s] * a.ssm_stride) + head_off;

  float4 S[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    S[i] = row < DK ? *reinterpret_cast<const float4*>(S0 + row * DV + c4 * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  __shared__ float sq[DK], sk[DK];
  __shared__ float red[NW][2 * DV + 4];
  const int64_t C = a.channels;
  const int64_t qoff = (int64_t)h * DK, koff = (int64_t)a.num_k_heads * DK + h * DK;
  const int64_t voff = 2 * (int64_t)a.num_k_heads * DK + (int64_t)m * DV + c4 * 4;

  for (int t = 0; t < L; ++t) {
    const int64_t r = r0 + t;
    if (tid < DK) sq[tid] = ld1<BF16>(a.y, r * C + qoff + tid);
    else if (tid < 2 * DK) sk[tid - DK] = ld1<BF16>(a.y, r * C + koff + tid - DK);
    const float4 v = ld4<BF16>(a.y, r * C + voff);
    const float gv = a.g[r * a.num_v_heads + m];
    const float bv = a.beta[r * a.num_v_heads + m];
    __syncthreads();

    float4 kS = make_float4(0.f, 0.f, 0.f, 0.f), Sq = kS;
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg + RG * i;
      if (row < DK) {
        const float kr = sk[row], qr = sq[row];
        kS = f4_fma(kr, S[i], kS);
        Sq = f4_fma(qr, S[i], Sq);
        kq = fmaf(kr, qr, kq);
      }
    }
#pragma unroll
    for (int off = C4; off < 64; off <<= 1) {
      kS.x += __shfl_xor(kS.x, off); kS.y += __shfl_xor(kS.y, off);
      kS.z += __shfl_xor(kS.z, off); kS.w += __shfl_xor(kS.w, off);
      Sq.x += __shfl_xor(Sq.x, off); Sq.y += __shfl_xor(Sq.y, off);
      Sq.z += __shfl_xor(Sq.z, off); Sq.w += __shfl_xor(Sq.w, off);
      kq += __shfl_xor(kq, off);
    }
    if (lane < C4) {
      *reinterpret_cast<float4*>(&red[wave][c4 * 4]) = kS;
      *reinterpret_cast<float4*>(&red[wave][DV + c4 * 4]) = Sq;
      if (c4 == 0) red[wave][2 * DV] = kq;
    }
    __syncthreads();
    kS = make_float4(0.f, 0.f, 0.f, 0.f);
    Sq = kS;
    kq = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float4 x = *reinterpret_cast<const float4*>(&red[w][c4 * 4]);
      const float4 y = *reinterpret_cast<const float4*>(&red[w][DV + c4 * 4]);
      kS.x += x.x; kS.y += x.y; kS.z += x.z; kS.w += x.w;
      Sq.x += y.x; Sq.y += y.y; Sq.z += y.z; Sq.w += y.w;
      kq += red[w][2 * DV];
    }
    const float av = __expf(gv);
    float4 u;
    u.x = bv * (v.x - av * kS.x); u.y = bv * (v.y - av * kS.y);
    u.z = bv * (v.z - av * kS.z); u.w = bv * (v.w - av * kS.w);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg + RG * i;
      if (row < DK) {
        const float kr = sk[row];
        S[i].x = fmaf(av, S[i].x, kr * u.x); S[i].y = fmaf(av, S[i].y, kr * u.y);
        S[i].z = fmaf(av, S[i].z, kr * u.z); S[i].w = fmaf(av, S[i].w, kr * u.w);
      }
    }
    if (rg == 0) {
      float4 o;
      o.x = fmaf(av, Sq.x, kq * u.x); o.y = fmaf(av, Sq.y, kq * u.y);
      o.z = fmaf(av, Sq.z, kq * u.z); o.w = fmaf(av, Sq.w, kq * u.w);
      st4<BF16>(a.out, (r * a.num_v_heads + m) * DV + c4 * 4, o);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    if (row < DK) *reinterpret_cast<float4*>(S1 + row * DV + c4 * 4) = S[i];
  }
}

template <bool BF16, int DK, int DV>
hipError_t rec_dispatch(const ScanArgs& a, hipStream_t st) {
  dim3 grid(a.num_seqs, a.num_v_heads);
  hipLaunchKernelGGL((recurrent_kernel<BF16, DK, DV>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <bool BF16, int DK>
hipError_t rec_dv(const ScanArgs& a, int dv, hipStream_t st) {
  switch (dv) {
    case 16: return rec_dispatch<BF16, DK, 16>(a, st);
    case 32: return rec_dispatch<BF16, DK, 32>(a, st);
    case 64: return rec_dispatch<BF16, DK, 64>(a, st);
    case 128: return rec_dispatch<BF16, DK, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

template <bool BF16>
hipError_t rec_dk(const ScanArgs& a, int dk, int dv, hipStream_t st) {
  switch (dk) {
    case 16: return rec_dv<BF16, 16>(a, dv, st);
    case 32: return rec_dv<BF16, 32>(a, dv, st);
    case 64: return rec_dv<BF16, 64>(a, dv, st);
    case 128: return rec_dv<BF16, 128>(a, dv, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_recurrent(const ScanArgs& a, int dk, int dv, bool bf16, hipStream_t st) {
  return bf16 ? rec_dk<true>(a, dk, dv, st) : rec_dk<false>(a, dk, dv, st);
}

}  // namespace gdn
