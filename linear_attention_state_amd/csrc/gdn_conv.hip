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
// channels (one 16-byte bf16 load per row, two for fp32), a 256-thread block
// covers 2048 channels of `rows_per_block` consecutive rows, so every row read
// is a coalesced 4 KB (bf16) segment.  The W-1 previous inputs of each channel
// slide along in registers; the first rows of a sequence take them from the
// sequence's conv state.  The Σx² of a head is reduced across the d_k/8 lanes
// that hold it with lane shuffles, so the normalisation costs no extra pass.
#include "gdn_device.h"

namespace gdn {
namespace {

template <bool BF16>
struct Act8 {
  static __device__ __forceinline__ void load(const void* base, int64_t idx, float v[8]) {
    if constexpr (BF16) {
      uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
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
  static __device__ __forceinline__ void store(void* base, int64_t idx, const float v[8]) {
    if constexpr (BF16) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)f32_to_bf16_bits(v[2 * i]) | ((uint32_t)f32_to_bf16_bits(v[2 * i + 1]) << 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(base) + idx) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx);
      p[0] = make_float4(v[0], v[1], v[2], v[3]);
      p[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
};

// 8 raw elements (bit-exact copies of the conv state).
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
};

template <bool BF16, int W>
__global__ __launch_bounds__(256) void conv_silu_norm_kernel(ConvArgs a) {
  constexpr int ESZ = BF16 ? 2 : 4;
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
  float win[W > 1 ? W - 1 : 1][8];
  bool fresh = true;
  for (int r = r_begin; r < r_end; ++r) {
    while (r >= seq_end && s < a.num_seqs - 1) {
      ++s;
      seq_begin = seq_end;
      seq_end = a.cu[s + 1];
      fresh = true;
    }
    if constexpr (W > 1) {
      if (fresh) {
        const bool act = seq_active(a.read_idx, a.write_idx, s, a.num_blocks);
        const char* tail = a.conv_pool + (act ? (int64_t)a.read_idx[s] * a.conv_stride : 0);
        const int pos = r - seq_begin;
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
          const int p = pos - (W - 1) + j;
#pragma unroll
          for (int e = 0; e < 8; ++e) win[j][e] = 0.f;
          if (!cok) continue;
          if (p >= 0)
            Act8<BF16>::load(a.x, (int64_t)(seq_begin + p) * a.channels + c0, win[j]);
          else if (act)
            Act8<BF16>::load(tail, ((int64_t)(W - 1 + p) * a.channels + c0), win[j]);
        }
      }
    }
    fresh = false;
    float xin[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (cok) Act8<BF16>::load(a.x, (int64_t)r * a.channels + c0, xin);
    float yv[8];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = wt[e][W - 1] * xin[e];
#pragma unroll
      for (int j = 0; j < W - 1; ++j) acc += wt[e][j] * win[j][e];
      yv[e] = silu(acc);
      ss += yv[e] * yv[e];
    }
    if constexpr (W > 1) {
#pragma unroll
      for (int j = 0; j < W - 2; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) win[j][e] = win[j + 1][e];
#pragma unroll
      for (int e = 0; e < 8; ++e) win[W - 2][e] = xin[e];
    }
    for (int off = 1; off < group; off <<= 1) ss += __shfl_xor(ss, off);
    if (do_norm) {
      const float inv = scale / sqrtf(ss + a.eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[e] *= inv;
    }
    if (cok) Act8<BF16>::store(a.y, (int64_t)r * a.channels + c0, yv);
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
  const char* src_tail = a.conv_pool + (int64_t)a.read_idx[s] * a.conv_stride;
  char* dst_tail = a.conv_pool + (int64_t)a.write_idx[s] * a.conv_stride;
  const char* xb = reinterpret_cast<const char*>(a.x);
  Raw8<BF16> rows[W - 1];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int i = L + j;  // row of [old state; x]
    const char* src = (i < W - 1) ? src_tail + ((int64_t)i * a.channels + c0) * ESZ
                                  : xb + ((int64_t)(r0 + i - (W - 1)) * a.channels + c0) * ESZ;
    rows[j].load(src);
  }
#pragma unroll
  for (int j = 0; j < W - 1; ++j) rows[j].store(dst_tail + ((int64_t)j * a.channels + c0) * ESZ);
}

template <bool BF16, int W>
hipError_t conv_dispatch(const ConvArgs& a, hipStream_t st) {
  const int threads = 256;
  const int per_block = threads * 8;
  dim3 grid((a.total_tokens + a.rows_per_block - 1) / a.rows_per_block,
            (a.channels + per_block - 1) / per_block);
  hipLaunchKernelGGL((conv_silu_norm_kernel<BF16, W>), grid, dim3(threads), 0, st, a);
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

hipError_t launch_conv(const ConvArgs& a, int width, bool bf16, hipStream_t st) {
  switch (width * 2 + (bf16 ? 1 : 0)) {
    case 2: return conv_dispatch<false, 1>(a, st);
    case 3: return conv_dispatch<true, 1>(a, st);
    case 4: return conv_dispatch<false, 2>(a, st);
    case 5: return conv_dispatch<true, 2>(a, st);
    case 6: return conv_dispatch<false, 3>(a, st);
    case 7: return conv_dispatch<true, 3>(a, st);
    case 8: return conv_dispatch<false, 4>(a, st);
    case 9: return conv_dispatch<true, 4>(a, st);
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
