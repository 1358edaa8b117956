// gdn_device.h -- device helpers and kernel launchers shared by the HIP
// sources of the gfx950 gated-delta-net library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

// A sequence takes part in a call when it has a write block inside the pool and
// a read block inside the pool; anything else is skipped without memory access.
__device__ __forceinline__ bool seq_active(const int32_t* read_idx, const int32_t* write_idx,
                                           int s, int num_blocks) {
  int rb = read_idx[s], wb = write_idx[s];
  return wb >= 0 && wb < num_blocks && rb >= 0 && rb < num_blocks;
}

// Index s with cu[s] <= row < cu[s+1] (the last such s when empty sequences repeat offsets).
__device__ __forceinline__ int find_seq(const int32_t* cu, int n, int row) {
  int lo = 0, hi = n;  // invariant: cu[lo] <= row < cu[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

struct ConvArgs {
  const void* x;
  const void* w;
  const int32_t* cu;
  const int32_t* read_idx;
  const int32_t* write_idx;
  const char* conv_pool;
  int64_t conv_stride;
  void* y;
  int num_seqs, total_tokens, num_blocks, channels, qk_channels, head_k_dim, rows_per_block;
  float eps, q_scale;
};

struct TailArgs {
  const void* x;
  const int32_t* cu;
  const int32_t* read_idx;
  const int32_t* write_idx;
  char* conv_pool;
  int64_t conv_stride;
  int num_seqs, num_blocks, channels;
};

struct ScanArgs {
  const void* y;  // conv output after SiLU/normalisation, [T][C] (chunked path)
  const void* x;  // conv input [T][C] and weights [C][W] (token path, which runs the conv itself)
  const void* w;
  const char* conv_pool;
  int64_t conv_stride;
  int width;
  float eps, q_scale;
  const float* g;
  const float* beta;
  const int32_t* cu;
  const int32_t* read_idx;
  const int32_t* write_idx;
  float* ssm_pool;
  int64_t ssm_stride;  // bytes
  void* out;
  int num_seqs, num_blocks, num_k_heads, num_v_heads, channels;
  int min_len, max_len;  // only sequences with min_len <= L <= max_len
};

hipError_t launch_conv(const ConvArgs& a, int width, bool bf16, hipStream_t st);
hipError_t launch_tail_commit(const TailArgs& a, int width, bool bf16, hipStream_t st);
hipError_t launch_recurrent(const ScanArgs& a, int dk, int dv, bool bf16, hipStream_t st);
hipError_t launch_chunk(const ScanArgs& a, int dk, int dv, hipStream_t st);
bool chunk_supported(int dk, int dv);

}  // namespace gdn
