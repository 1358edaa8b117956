// gdn_probe.hip -- measurement support, so that kernel rates can be reported as
// a fraction of a measured peak beside the published one:
//  - the MFMA rate this device reaches on back-to-back independent products
//    (eight accumulator chains per wave, four waves per SIMD); it touches no
//    memory but one store that never happens (it keeps the products alive);
//  - the HBM rate of a plain streaming copy: 16-byte non-temporal loads and
//    stores, four in flight per thread, one block per 32 KiB span.
#include "gdn_device.h"

namespace gdn {
namespace {

__device__ float g_probe_sink[256];

template <bool BF16>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float seed) {
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float base = seed * (1.0f + 1e-3f * (float)(threadIdx.x & 63));
  asm volatile("" : "+v"(base));  // a run-time value: nothing below folds
  if constexpr (BF16) {
    bf16x8 a[8], b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (__bf16)(base / (float)(e + 1));
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) a[j][e] = (__bf16)(base * (float)(e + 1 + j));
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b, acc[j], 0, 0, 0);
      // every round's products are kept, each chain on its own
      asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
                   "+v"(acc[6]), "+v"(acc[7]));
    }
  } else {
    float a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = base + (float)j;
    const float b = 1.0f / (base + 1.0f);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b, acc[j], 0, 0, 0);
      asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
                   "+v"(acc[6]), "+v"(acc[7]));
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) sum += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (sum == -1.0f) g_probe_sink[threadIdx.x] = sum;  // the operands are positive: never taken
}

// n 16-byte elements from src to dst.  Each block copies its own span of
// kCopySpan consecutive elements (32 KiB), four loads in flight per thread:
// short-lived blocks over contiguous spans stream about a fifth faster on this
// chip than a persistent grid-stride loop over the whole buffer.
constexpr int kCopySpan = 2048;

__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n) {
  const int64_t b0 = (int64_t)blockIdx.x * kCopySpan;
  const int64_t b1 = b0 + kCopySpan < n ? b0 + kCopySpan : n;
  int64_t i = b0 + threadIdx.x;
  for (; i + 3 * 256 < b1; i += 4 * 256) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + 256);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 512);
    const u32x4 v3 = __builtin_nontemporal_load(src + i + 768);
    __builtin_nontemporal_store(v0, dst + i);
    __builtin_nontemporal_store(v1, dst + i + 256);
    __builtin_nontemporal_store(v2, dst + i + 512);
    __builtin_nontemporal_store(v3, dst + i + 768);
  }
  for (; i < b1; i += 256) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

// n16 16-byte elements, one 256-thread block per 32 KiB span
hipError_t launch_copy_probe(const void* src, void* dst, int64_t n16, hipStream_t st) {
  const int64_t blocks = (n16 + kCopySpan - 1) / kCopySpan;
  if (blocks < 1 || blocks > (1 << 22)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_probe_kernel, dim3(blocks), dim3(256), 0, st, reinterpret_cast<const u32x4*>(src),
                     reinterpret_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

// blocks x 256 threads, `iters` iterations of 8 products per wave
hipError_t launch_mfma_probe(bool bf16, int blocks, int iters, hipStream_t st) {
  if (bf16)
    hipLaunchKernelGGL(mfma_probe_kernel<true>, dim3(blocks), dim3(256), 0, st, iters, 0.5f);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<false>, dim3(blocks), dim3(256), 0, st, iters, 0.5f);
  return hipGetLastError();
}

}  // namespace gdn
