// gdn_conv.hip -- varlen depthwise causal conv1d + SiLU + q/k L2 normalisation,
// and the conv-state commit, for gfx950.
//
// Page "Continuous batching for linear attention layers" (PR description): the
// varlen causal convolution continues every sequence of the packed row from its
// own conv state, which holds the sequence's last W-1 inputs.  Taps: w[c][W-1]
// multiplies the current token; the conv state is stored [W-1][C], oldest row
// first; SiLU follows on every channel; q and k are then normalised per key
// head as x / sqrt(sum x^2 + eps), q also multiplied by q_scale.
//
// Layout: x and the output y are [T][C] rows; one thread owns 8 consecutive
// channels (one 16-byte bf16 load per row, two for fp32), a one-wave block
// covers 512 channels of `rows_per_block` consecutive rows, so every row read
// is a coalesced 1 KB (bf16) segment.  The host sizes the blocks so that there
// are about 16 per CU: long row ranges keep the W-1 re-read rows at a block's
// start a small fraction of the traffic.  The W-1 previous inputs of each channel
// slide along in registers; the first rows of a sequence take them from the
// sequence's conv state.  The Σx² of a head is reduced across the d_k/8 lanes
// that hold it with lane shuffles, so the normalisation costs no extra pass.
#include "gdn_device.h"

namespace gdn {
namespace {

template <bool BF16>
struct Act8 {
  // NT: non-temporal access (the activations stream through once)
  template <bool NT = false>
  static __device__ __forceinline__ void load(const void* base, int64_t idx, float v[8]) {
    if constexpr (BF16) {
      const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + idx);
      const u32x4 u = NT ? __builtin_nontemporal_load(p) : *p;
      uint32_t w[4] = {u[0], u[1], u[2], u[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
      float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  }
  template <bool NT = false>
  static __device__ __forceinline__ void store(void* base, int64_t idx, const float v[8]) {
    if constexpr (BF16) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
      u32x4* p = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(base) + idx);
      if (NT) __builtin_nontemporal_store(w, p);
      else *p = w;
    } else {
      float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx);
      p[0] = make_float4(v[0], v[1], v[2], v[3]);
      p[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
};

// 8 raw elements (bit-exact copies of the conv state, and the rows in flight
// of the conv kernel).
template <bool BF16>
struct Raw8 {
  uint4 u[BF16 ? 1 : 2];
  __device__ __forceinline__ void load(const char* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < (BF16 ? 1 : 2); ++i) u[i] = q[i];
  }
  __device__ __forceinline__ void store(char* p) const {
    uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
    for (int i = 0; i < (BF16 ? 1 : 2); ++i) q[i] = u[i];
  }
  // non-temporal load of activation row elements [idx, idx + 8)
  __device__ __forceinline__ void load_stream(const void* base, int64_t idx) {
    const u32x4* q = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + idx * (BF16 ? 2 : 4));
#pragma unroll
    for (int i = 0; i < (BF16 ? 1 : 2); ++i) {
      const u32x4 v = __builtin_nontemporal_load(q + i);
      u[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
  __device__ __forceinline__ void to_f32(float v[8]) const {
    if constexpr (BF16) {
      const uint32_t w[4] = {u[0].x, u[0].y, u[0].z, u[0].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        v[4 * i] = __uint_as_float(u[i].x); v[4 * i + 1] = __uint_as_float(u[i].y);
        v[4 * i + 2] = __uint_as_float(u[i].z); v[4 * i + 3] = __uint_as_float(u[i].w);
      }
    }
  }
};

template <bool BF16, int W, bool SILU>
__global__ __launch_bounds__(256) void conv_silu_norm_kernel(ConvArgs a) {
  constexpr int ESZ = BF16 ? 2 : 4;
  if (a.skip && *a.skip) return;  // device plan: the chunk kernel runs the conv (uniform)
  const int c0 = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
  const bool cok = c0 < a.channels;
  const int r_begin = blockIdx.x * a.rows_per_block;
  const int r_end = min(r_begin + a.rows_per_block, a.total_tokens);
  if (r_begin >= r_end) return;  // uniform over the block

  float wt[8][W];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int j = 0; j < W; ++j) wt[e][j] = 0.f;
  if (cok) {
    if constexpr (BF16) {
      const uint16_t* w = reinterpret_cast<const uint16_t*>(a.w);
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < W; ++j) wt[e][j] = bf16_bits_to_f32(w[(int64_t)(c0 + e) * W + j]);
    } else {
      const float* w = reinterpret_cast<const float*>(a.w);
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < W; ++j) wt[e][j] = w[(int64_t)(c0 + e) * W + j];
    }
  }
  const bool do_norm = c0 < 2 * a.qk_channels;
  const float scale = c0 < a.qk_channels ? a.q_scale : 1.0f;
  const int group = a.head_k_dim >> 3;  // lanes holding one head (power of two)

  int s = find_seq(a.cu, a.num_seqs, r_begin);
  int seq_begin = a.cu[s], seq_end = a.cu[s + 1];
  bool fresh = true;
  bool on = seq_active(a.read_idx, a.write_idx, s, a.num_blocks);  // rows of a padding sequence are not written
  // LA rows of x in flight per thread (row r is loaded LA rows ahead of its
  // use), and the inputs of rows r-LA+1..r in a circular buffer indexed by
  // r mod LA; r_begin is a multiple of LA, so every index is static.
  constexpr int LA = 4;
  static_assert(W <= LA, "window must fit the buffer");
  Raw8<BF16> ring[LA];
  float xr[LA][8];
#pragma unroll
  for (int k = 0; k < LA; ++k) {
#pragma unroll
    for (int e = 0; e < 8; ++e) xr[k][e] = 0.f;
    if (cok && r_begin + k < r_end) ring[k].load_stream(a.x, (int64_t)(r_begin + k) * a.channels + c0);
  }
  for (int rb = r_begin; rb < r_end; rb += LA) {
#pragma unroll
    for (int k = 0; k < LA; ++k) {
      const int r = rb + k;
      if (r >= r_end) break;
      while (r >= seq_end && s < a.num_seqs - 1) {
        ++s;
        seq_begin = seq_end;
        seq_end = a.cu[s + 1];
        fresh = true;
        on = seq_active(a.read_idx, a.write_idx, s, a.num_blocks);
      }
      if constexpr (W > 1) {
        if (fresh) {  // the W-1 inputs before row r: earlier rows of the sequence, else its conv state
          const bool act = seq_active(a.read_idx, a.write_idx, s, a.num_blocks);
          const char* tail = a.conv_pool + (act ? (int64_t)a.read_idx[s] * a.conv_stride : 0);
          const int pos = r - seq_begin;
#pragma unroll
          for (int j = 1; j < W; ++j) {
            float* dst = xr[(k - j + LA) % LA];
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[e] = 0.f;
            if (!cok) continue;
            const int p = pos - j;
            if (p >= 0)
              Act8<BF16>::load(a.x, (int64_t)(seq_begin + p) * a.channels + c0, dst);
            else if (act)
              Act8<BF16>::load(tail, ((int64_t)(W - 1 + p) * a.channels + c0), dst);
          }
        }
      }
      fresh = false;
      if (cok) ring[k].to_f32(xr[k]);
      if (cok && r + LA < r_end) ring[k].load_stream(a.x, (int64_t)(r + LA) * a.channels + c0);
      float yv[8];
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float acc = wt[e][W - 1] * xr[k][e];
#pragma unroll
        for (int j = 1; j < W; ++j) acc += wt[e][W - 1 - j] * xr[(k - j + LA) % LA][e];
        yv[e] = SILU ? silu(acc) : acc;
        ss += yv[e] * yv[e];
      }
      ss = group_sum(ss, group);
      if (do_norm) {
        const float inv = scale * rsqrt_fast(ss + a.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) yv[e] *= inv;
      }
      if (cok && on) Act8<BF16>::template store<true>(a.y, (int64_t)r * a.channels + c0, yv);
    }
  }
  (void)ESZ;
}

// New conv state of every sequence: the last W-1 rows of [old state; x].
// One thread per 8 channels reads all W-1 source rows before it writes, so the
// ordinary in-place case (read block == write block) is safe; this kernel runs
// after the conv kernel on the same stream, which has consumed the old states.
template <bool BF16, int W>
__global__ __launch_bounds__(256) void conv_tail_commit_kernel(TailArgs a) {
  constexpr int ESZ = BF16 ? 2 : 4;
  const int s = blockIdx.x;
  const int c0 = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
  if (c0 >= a.channels || s >= a.num_seqs) return;
  if (!seq_active(a.read_idx, a.write_idx, s, a.num_blocks)) return;
  const int r0 = a.cu[s];
  const int L = a.cu[s + 1] - r0;
  if (L > ((a.fused && *a.fused) ? 1 : a.max_len)) return;
  const char* src_tail = a.conv_pool + (int64_t)a.read_idx[s] * a.conv_stride;
  char* dst_tail = a.conv_pool + (int64_t)a.write_idx[s] * a.conv_stride;
  const char* xb = reinterpret_cast<const char*>(a.x);
  // global (not flat) accesses: with flat ones this kernel ran three times slower
  constexpr int NV = BF16 ? 1 : 2;  // 16-byte pieces per thread and row
  u32x4 rows[W - 1][NV];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int i = L + j;  // row of [old state; x]
    const char* src = (i < W - 1) ? src_tail + ((int64_t)i * a.channels + c0) * ESZ
                                  : xb + ((int64_t)(r0 + i - (W - 1)) * a.channels + c0) * ESZ;
    const gptr<const u32x4> g = as_global(reinterpret_cast<const u32x4*>(src));
#pragma unroll
    for (int h = 0; h < NV; ++h) rows[j][h] = g[h];
  }
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const gptr<u32x4> g = as_global(reinterpret_cast<u32x4*>(dst_tail + ((int64_t)j * a.channels + c0) * ESZ));
#pragma unroll
    for (int h = 0; h < NV; ++h) g[h] = rows[j][h];
  }
}

template <bool BF16, int W, bool SILU>
hipError_t conv_dispatch(const ConvArgs& a, hipStream_t st) {
  const int threads = 64;  // one wave: 512 channels
  const int per_block = threads * 8;
  dim3 grid((a.total_tokens + a.rows_per_block - 1) / a.rows_per_block,
            (a.channels + per_block - 1) / per_block);
  hipLaunchKernelGGL((conv_silu_norm_kernel<BF16, W, SILU>), grid, dim3(threads), 0, st, a);
  return hipGetLastError();
}

template <bool BF16, int W>
hipError_t tail_dispatch(const TailArgs& a, hipStream_t st) {
  const int threads = 256;
  const int per_block = threads * 8;
  dim3 grid(a.num_seqs, (a.channels + per_block - 1) / per_block);
  hipLaunchKernelGGL((conv_tail_commit_kernel<BF16, W>), grid, dim3(threads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv(const ConvArgs& a, int width, bool bf16, bool silu, hipStream_t st) {
  switch (width * 4 + (bf16 ? 2 : 0) + (silu ? 1 : 0)) {
    case 4: return conv_dispatch<false, 1, false>(a, st);
    case 5: return conv_dispatch<false, 1, true>(a, st);
    case 6: return conv_dispatch<true, 1, false>(a, st);
    case 7: return conv_dispatch<true, 1, true>(a, st);
    case 8: return conv_dispatch<false, 2, false>(a, st);
    case 9: return conv_dispatch<false, 2, true>(a, st);
    case 10: return conv_dispatch<true, 2, false>(a, st);
    case 11: return conv_dispatch<true, 2, true>(a, st);
    case 12: return conv_dispatch<false, 3, false>(a, st);
    case 13: return conv_dispatch<false, 3, true>(a, st);
    case 14: return conv_dispatch<true, 3, false>(a, st);
    case 15: return conv_dispatch<true, 3, true>(a, st);
    case 16: return conv_dispatch<false, 4, false>(a, st);
    case 17: return conv_dispatch<false, 4, true>(a, st);
    case 18: return conv_dispatch<true, 4, false>(a, st);
    case 19: return conv_dispatch<true, 4, true>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_tail_commit(const TailArgs& a, int width, bool bf16, hipStream_t st) {
  switch (width * 2 + (bf16 ? 1 : 0)) {
    case 4: return tail_dispatch<false, 2>(a, st);
    case 5: return tail_dispatch<true, 2>(a, st);
    case 6: return tail_dispatch<false, 3>(a, st);
    case 7: return tail_dispatch<true, 3>(a, st);
    case 8: return tail_dispatch<false, 4>(a, st);
    case 9: return tail_dispatch<true, 4>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

namespace gdn {
namespace {

// Copies block src[i] of both pools to block dst[i].  Block x = pair i, block y
// = 32 KiB piece of the concatenation [recurrent state; conv state]; 256
// threads move 16 bytes per access, in two rounds of four loads followed by
// their four stores, non-temporal (the blocks are touched once; 4% faster than
// cached accesses).  Measured on 256 pairs of 2 MiB + 48 KiB: 0.207 ms, against
// 0.214 ms for 64 KiB pieces with all sixteen loads issued before any store;
// eight loads before the first store ran at 0.475 ms.
constexpr int kCopyPiece = 32768;
__global__ __launch_bounds__(256) void state_copy_kernel(StateCopyArgs a) {
  const int i = blockIdx.x;
  const int sb = a.src[i], db = a.dst[i];
  if (sb < 0 || sb >= a.num_blocks || db < 0 || db >= a.num_blocks || sb == db) return;
  const int64_t piece = (int64_t)blockIdx.y * kCopyPiece;
  const int64_t ssm_bytes = a.ssm_bytes, total = a.ssm_bytes + a.conv_bytes;
  if (piece >= total) return;
  constexpr int K = kCopyPiece / (256 * 16), G = 4;
#pragma unroll
  for (int g0 = 0; g0 < K; g0 += G) {
    u32x4 v[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int64_t o = piece + ((int64_t)(g0 + k) * 256 + threadIdx.x) * 16;
      if (o < total) {
        const char* src = o < ssm_bytes ? a.ssm_pool + (int64_t)sb * a.ssm_stride + o
                                        : a.conv_pool + (int64_t)sb * a.conv_stride + (o - ssm_bytes);
        v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
      }
    }
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int64_t o = piece + ((int64_t)(g0 + k) * 256 + threadIdx.x) * 16;
      if (o < total) {
        char* dst = o < ssm_bytes ? a.ssm_pool + (int64_t)db * a.ssm_stride + o
                                  : a.conv_pool + (int64_t)db * a.conv_stride + (o - ssm_bytes);
        __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4*>(dst));
      }
    }
  }
}

}  // namespace

hipError_t launch_state_copy(const StateCopyArgs& a, int n, hipStream_t st) {
  const int64_t total = a.ssm_bytes + a.conv_bytes;
  const int64_t pieces = (total + kCopyPiece - 1) / kCopyPiece;
  if (n <= 0 || pieces <= 0) return hipSuccess;
  if (pieces > 65535 || n > 2147483647) return hipErrorInvalidValue;
  hipLaunchKernelGGL(state_copy_kernel, dim3(n, (unsigned)pieces), dim3(256), 0, st, a);
  return hipGetLastError();
}

GDN_STATUS_ACCESSOR(status_conv)

}  // namespace gdn
