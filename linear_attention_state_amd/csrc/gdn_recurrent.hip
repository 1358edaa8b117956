// gdn_recurrent.hip -- token-by-token gated delta rule for gfx950: the decode
// path (one token per sequence) and the all-fp32 path.
//
// Recurrence (Gated Delta Networks, Yang et al., ICLR 2025), state of a value
// head stored [d_k][d_v] with d_v fastest, carried per request in its block
// (page "Continuous batching for linear attention layers", PR description):
//     S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t.
// Kimi delta attention (KDA; Kimi Linear technical report, 2025) replaces the
// scalar a_t by a decay per key channel: S_t = (I - b_t k_t k_t^T) diag(a_t) S_{t-1}
// + b_t k_t v_t^T; the same pass runs it with each state row's decay folded into
// k and q (template flag KDA, g then [T][H_v][d_k]).
// Evaluated in delta form: kS = S^T k, u = b (v - a kS), S <- a S + k u^T, and
// o = a S_{t-1}^T q + (k.q) u, so one reduction pass over d_k serves both kS and
// the output.  The kernel also runs the token's causal conv + SiLU for the
// 2 d_k + d_v channels its head reads (window of W-1 inputs in registers,
// started from the conv state) and folds the q/k L2 normalisation into that same
// reduction pass (|k|^2 and |q|^2 are reduced with the dot products and applied
// afterwards), so q, k and v stay in fp32 from x to the output.
//
// One workgroup of 256 threads owns one (sequence, value head).  A thread holds
// 4 adjacent d_v columns of d_k/(256/(d_v/4)) consecutive rows in registers; a
// wave's load instruction therefore covers 64/(d_v/4) whole state rows (1 KB for
// d_v=128), fully coalesced, and a thread's rows sit at small fixed offsets from
// one address (4% faster than rows interleaved across the row groups).  For a one-token sequence the kernel is a pure streaming
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

// element i as raw bits (bf16 in the low half), and those bits as fp32
template <bool BF16>
__device__ __forceinline__ uint32_t ldraw(const void* base, int64_t i) {
  if constexpr (BF16) return reinterpret_cast<const uint16_t*>(base)[i];
  else return reinterpret_cast<const uint32_t*>(base)[i];
}
template <bool BF16>
__device__ __forceinline__ float rawf(uint32_t b) {
  if constexpr (BF16) return __uint_as_float(b << 16);
  else return __uint_as_float(b);
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

// The state is read once and written once per call: non-temporal accesses
// (cache policy NT) keep it from displacing cached data.  Offsets: a per-lane
// byte offset plus a constant one (folded into the instruction's immediate or
// its scalar offset).
constexpr int kNonTemporal = 2;
__device__ __forceinline__ float4 ld_state(__amdgpu_buffer_rsrc_t rs, int voff, int coff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + coff, 0, kNonTemporal);
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}
__device__ __forceinline__ void st_state(__amdgpu_buffer_rsrc_t rs, int voff, int coff, float4 v) {
  const u32x4 w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(w, rs, voff + coff, 0, kNonTemporal);
}

__device__ __forceinline__ float4 f4_fma(float a, float4 x, float4 y) {
  return make_float4(fmaf(a, x.x, y.x), fmaf(a, x.y, y.y), fmaf(a, x.z, y.z), fmaf(a, x.w, y.w));
}

template <bool BF16, int DK, int DV, int DVS, bool KDA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KDA ? 3 : 1))) void recurrent_kernel(ScanArgs a) {
  constexpr int NT = 256;
  constexpr int C4 = DVS / 4;         // threads across the workgroup's part of a state row
  constexpr int RG = NT / C4;         // row groups
  constexpr int RPT = (DK + RG - 1) / RG;
  constexpr int NW = NT / 64;
  constexpr int NCH = 2 * DK + DVS;   // conv channels read: q, k of the key head, this part of v
  static_assert(C4 <= 64 && (64 % C4) == 0, "row group must fit a wave");
  static_assert(NCH <= 2 * NT, "two channels per thread at most");

  const int s = blockIdx.x, m = blockIdx.y;
  const int n0 = DVS * blockIdx.z;  // this workgroup's d_v columns [n0, n0 + DVS)
  if (s >= a.num_seqs) return;
  const int r0 = a.cu[s];
  const int L = a.cu[s + 1] - r0;
  if (L < a.min_len || L > a.max_len) return;
  if (!seq_active(a.read_idx, a.write_idx, s, a.num_blocks)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c4 = tid % C4, rg = tid / C4;
  // whether state row `row` of this thread exists (always, when the row groups
  // tile d_k exactly: a compile-time fact the loads below must not branch on)
  auto row_ok = [](int row) { return RG * RPT == DK || row < DK; };
  const int h = m / (a.num_v_heads / a.num_k_heads);
  const int64_t head_off = (int64_t)m * DK * DV + n0;
  const float* S0 = reinterpret_cast<const float*>(
      reinterpret_cast<const char*>(a.ssm_pool) + (int64_t)a.read_idx[s] * a.ssm_stride) + head_off;
  float* S1 = reinterpret_cast<float*>(
      reinterpret_cast<char*>(a.ssm_pool) + (int64_t)a.write_idx[s] * a.ssm_stride) + head_off;

  // conv channels owned by this thread (index i into [q | k | v] of this head)
  const int64_t C = a.channels;
  const int W = a.width;
  int64_t gch[2];
  bool has[2];
  float wt[2][4], win[2][3], wlast[2];
  const char* tail = a.conv_pool && W > 1 ? a.conv_pool + (int64_t)a.read_idx[s] * a.conv_stride : nullptr;
  // The conv inputs of the first token (taps, the W-1 previous inputs, x) are
  // loaded first, all at once, as raw bits: every load is unconditional at a
  // clamped index (a thread past the channel count reads channel 0), and no
  // value is used before the state loads below have been issued, so neither
  // group waits for the other.  Where a source does not exist (an empty
  // sequence, whose x and taps may be NULL; no conv state) the load reads
  // element 0 of the state pool instead, and the value is masked.
  uint32_t wraw[2][4], traw[2][3], xraw[2];
  const bool have_in = L > 0;
  const void* wsrc = have_in ? a.w : (const void*)a.ssm_pool;
  const void* xsrc = have_in ? a.x : (const void*)a.ssm_pool;
  const void* tsrc = have_in && tail ? (const void*)tail : (const void*)a.ssm_pool;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = tid + NT * e;
    has[e] = i < NCH && have_in;
    const int ic = i < NCH ? i : 0;
    gch[e] = ic < DK ? (int64_t)h * DK + ic
           : ic < 2 * DK ? (int64_t)a.num_k_heads * DK + h * DK + (ic - DK)
                         : 2 * (int64_t)a.num_k_heads * DK + (int64_t)m * DV + n0 + (ic - 2 * DK);
#pragma unroll
    for (int j = 0; j < 4; ++j) wraw[e][j] = ldraw<BF16>(wsrc, have_in ? gch[e] * W + (j < W ? j : 0) : 0);
#pragma unroll
    for (int j = 0; j < 3; ++j)
      traw[e][j] = ldraw<BF16>(tsrc, have_in && tail ? (int64_t)(j < W - 1 ? j : 0) * C + gch[e] : 0);
    xraw[e] = ldraw<BF16>(xsrc, have_in ? (int64_t)r0 * C + gch[e] : 0);
  }
  // scheduling barriers: the state loads issue right after the conv-input
  // loads, before anything waits for those
  __builtin_amdgcn_sched_barrier(0);
  // the thread's rows through one buffer resource per head (scalar base): one
  // offset register for all RPT loads, each at a fixed offset from it
  const __amdgpu_buffer_rsrc_t rs0 = make_rsrc(S0, (uint32_t)(DK * DV * 4));
  const int soff = (rg * RPT * DV + c4 * 4) * 4;
  float4 S[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg * RPT + i;
    S[i] = row_ok(row) ? ld_state(rs0, soff, i * DV * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __builtin_amdgcn_sched_barrier(0);
  // the taps, window and first input, converted and masked only now (taps
  // past W, window rows past W-1, threads past the channel count, no inputs)
  float xin0[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    wlast[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wt[e][j] = has[e] && j < W ? rawf<BF16>(wraw[e][j]) : 0.f;
      if (j == W - 1) wlast[e] = wt[e][j];
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) win[e][j] = has[e] && tail && j < W - 1 ? rawf<BF16>(traw[e][j]) : 0.f;
    xin0[e] = has[e] ? rawf<BF16>(xraw[e]) : 0.f;
  }

  __shared__ __align__(16) float sy[NCH];
  __shared__ float sdec[KDA ? DK : 1];  // KDA: exp(g) of the token, per key channel
  __shared__ __align__(16) float red[NW][2 * DVS + 4];

  for (int t = 0; t < L; ++t) {
    const int64_t r = r0 + t;
    // ---- causal conv + SiLU of this token for the head's channels (the first
    // token's x was loaded with the taps; later ones at a clamped index)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float xin = t == 0 ? xin0[e] : ld1<BF16>(a.x, r * C + gch[e]);
      if (!has[e]) continue;
      float acc = wlast[e] * xin;
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < W - 1) acc = fmaf(wt[e][j], win[e][j], acc);
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (j + 1 < W - 1) win[e][j] = win[e][j + 1];
        else if (j == W - 2) win[e][j] = xin;
      }
      sy[tid + NT * e] = silu(acc);
    }
    // decay: one per value head (gated delta rule), or one per key channel
    // (KDA: read once per row into LDS, beside the conv outputs)
    const float gv = KDA ? 0.f : a.g[r * a.num_v_heads + m];
    if (KDA && tid < DK) sdec[tid] = __expf(a.g[(r * a.num_v_heads + m) * DK + tid]);
    const float bv = a.beta[r * a.num_v_heads + m];
    __syncthreads();

    // ---- one pass over the state rows: S^T k, S^T q, k.q, |k|^2, |q|^2 (unnormalised q, k)
    float4 kS = make_float4(0.f, 0.f, 0.f, 0.f), Sq = kS;
    float kq = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg * RPT + i;
      if (row_ok(row)) {
        const float kr = sy[DK + row], qr = sy[row];
        // KDA reads the decayed state diag(a) S: the row's decay folded into k and q
        const float dr = KDA ? sdec[row] : 1.f;  // read at each use: no registers held for it
        kS = f4_fma(KDA ? kr * dr : kr, S[i], kS);
        Sq = f4_fma(KDA ? qr * dr : qr, S[i], Sq);
        kq = fmaf(kr, qr, kq);
        kk = fmaf(kr, kr, kk);
        qq = fmaf(qr, qr, qq);
      }
    }
#pragma unroll
    for (int off = C4; off < 64; off <<= 1) {
      kS.x += __shfl_xor(kS.x, off); kS.y += __shfl_xor(kS.y, off);
      kS.z += __shfl_xor(kS.z, off); kS.w += __shfl_xor(kS.w, off);
      Sq.x += __shfl_xor(Sq.x, off); Sq.y += __shfl_xor(Sq.y, off);
      Sq.z += __shfl_xor(Sq.z, off); Sq.w += __shfl_xor(Sq.w, off);
      kq += __shfl_xor(kq, off);
      kk += __shfl_xor(kk, off);
      qq += __shfl_xor(qq, off);
    }
    if (lane < C4) {
      *reinterpret_cast<float4*>(&red[wave][c4 * 4]) = kS;
      *reinterpret_cast<float4*>(&red[wave][DVS + c4 * 4]) = Sq;
      if (c4 == 0) {
        red[wave][2 * DVS] = kq;
        red[wave][2 * DVS + 1] = kk;
        red[wave][2 * DVS + 2] = qq;
      }
    }
    __syncthreads();
    kS = make_float4(0.f, 0.f, 0.f, 0.f);
    Sq = kS;
    kq = kk = qq = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float4 x = *reinterpret_cast<const float4*>(&red[w][c4 * 4]);
      const float4 y = *reinterpret_cast<const float4*>(&red[w][DVS + c4 * 4]);
      kS.x += x.x; kS.y += x.y; kS.z += x.z; kS.w += x.w;
      Sq.x += y.x; Sq.y += y.y; Sq.z += y.z; Sq.w += y.w;
      kq += red[w][2 * DVS];
      kk += red[w][2 * DVS + 1];
      qq += red[w][2 * DVS + 2];
    }
    // normalisation folded in: k_hat = k / sqrt(|k|^2 + eps), q_hat = q_scale q / sqrt(|q|^2 + eps)
    const float ik = rsqrt_fast(kk + a.eps);
    const float iq = a.q_scale * rsqrt_fast(qq + a.eps);
    const float av = KDA ? 1.f : __expf(gv);  // KDA: already in kS and Sq
    const float4 v = *reinterpret_cast<const float4*>(&sy[2 * DK + c4 * 4]);
    float4 u;
    u.x = bv * (v.x - av * kS.x * ik); u.y = bv * (v.y - av * kS.y * ik);
    u.z = bv * (v.z - av * kS.z * ik); u.w = bv * (v.w - av * kS.w * ik);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg * RPT + i;
      if (row_ok(row)) {
        const float kr = sy[DK + row] * ik;
        const float dec = KDA ? sdec[row] : av;
        S[i].x = fmaf(dec, S[i].x, kr * u.x); S[i].y = fmaf(dec, S[i].y, kr * u.y);
        S[i].z = fmaf(dec, S[i].z, kr * u.z); S[i].w = fmaf(dec, S[i].w, kr * u.w);
      }
    }
    if (rg == 0) {
      const float kqn = kq * ik * iq, aq = av * iq;
      float4 o;
      o.x = fmaf(aq, Sq.x, kqn * u.x); o.y = fmaf(aq, Sq.y, kqn * u.y);
      o.z = fmaf(aq, Sq.z, kqn * u.z); o.w = fmaf(aq, Sq.w, kqn * u.w);
      st4<BF16>(a.out, (r * a.num_v_heads + m) * DV + n0 + c4 * 4, o);
    }
    __syncthreads();
  }

  const __amdgpu_buffer_rsrc_t rs1 = make_rsrc(S1, (uint32_t)(DK * DV * 4));
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg * RPT + i;
    if (row_ok(row)) st_state(rs1, soff, i * DV * 4, S[i]);
  }
}

// d_v is split over DV / DVS workgroups per (sequence, head): the columns of S
// evolve independently, so each part needs only q, k and its own columns of v;
// smaller parts leave more workgroups resident to cover the state's memory latency.
template <bool BF16, int DK, int DV>
hipError_t rec_dispatch(const ScanArgs& a, hipStream_t st) {
  constexpr int DVS = DV;
  dim3 grid(a.num_seqs, a.num_v_heads, DV / DVS);
  if (a.kda)
    hipLaunchKernelGGL((recurrent_kernel<BF16, DK, DV, DVS, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((recurrent_kernel<BF16, DK, DV, DVS, false>), grid, dim3(256), 0, st, a);
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

GDN_STATUS_ACCESSOR(status_recurrent)

}  // namespace gdn
