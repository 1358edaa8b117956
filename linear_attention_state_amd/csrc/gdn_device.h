// gdn_device.h -- device helpers and kernel launchers shared by the HIP
// sources of the gfx950 gated-delta-net library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Global-memory pointers in address space 1: loads and stores through them
// are global (not flat) instructions, so they are counted by vmcnt only and an
// LDS wait never waits for them.
template <class T>
using gptr = __attribute__((address_space(1))) T*;
template <class T>
__device__ __forceinline__ gptr<T> as_global(T* p) {
  return (gptr<T>)(p);
}

// Buffer resource (V#) over `bytes` bytes from `base`: raw buffer loads past
// the end return zero and raw buffer stores past the end are dropped, which
// bounds every access by hardware.  Offsets are 32-bit byte offsets.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// DPP lane move within each row of 16 lanes (or across rows for the row
// broadcasts); lanes without a source lane get zero.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false));
}

// Sum over the `group` lanes of a head (2, 4, 8 or 16, aligned within a row
// of 16, the same for the whole wave), in lane registers: the pairings of a
// butterfly over lane xor 1, 2, 4 and 8.  After each step both lanes of a pair
// hold the same bits, so pairing by mirror (lane 7 - i within 8, 15 - i within
// 16) adds the same two partial sums as xor 4 and xor 8 would.
__device__ __forceinline__ float group_sum(float v, int group) {
  if (group >= 2) v += dpp_move<0xB1, 0xf>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  if (group >= 4) v += dpp_move<0x4E, 0xf>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  if (group >= 8) v += dpp_move<0x141, 0xf>(v);  // row_half_mirror
  if (group >= 16) v += dpp_move<0x140, 0xf>(v); // row_mirror
  return v;
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

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 -> two bf16 packed in one dword (first in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Workgroup barrier that only waits for this wave's LDS traffic: outstanding
// global loads (prefetches) and stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// SiLU with the hardware reciprocal (about 1 ulp) instead of an IEEE division.
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// 1 / sqrt(x) with the hardware reciprocal square root (about 1 ulp), x > 0.
__device__ __forceinline__ float rsqrt_fast(float x) { return __builtin_amdgcn_rsqf(x); }

// Sticky status bits raised by the kernels (read and cleared by
// gdn_device_status through the accessor each HIP source defines with
// GDN_STATUS_ACCESSOR; every source has its own word, the query ORs them).
constexpr uint32_t kStatusWaitExpired = 1u;  // a bounded wait between waves or workgroups gave up
constexpr uint32_t kStatusBadIndex = 2u;     // a read or write block outside the pool was skipped
static __device__ uint32_t g_status;
__device__ __forceinline__ void raise_status(uint32_t bit) {
  __hip_atomic_fetch_or(&g_status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
#define GDN_STATUS_ACCESSOR(fn)                                                                      \
  hipError_t fn(uint32_t* bits, int clear) {                                                         \
    uint32_t v = 0;                                                                                  \
    hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_status), sizeof(v), 0, hipMemcpyDeviceToHost); \
    if (e == hipSuccess && clear && v) {                                                             \
      const uint32_t z = 0;                                                                          \
      e = hipMemcpyToSymbol(HIP_SYMBOL(g_status), &z, sizeof(z), 0, hipMemcpyHostToDevice);          \
    }                                                                                                \
    *bits |= v;                                                                                      \
    return e;                                                                                        \
  }
hipError_t status_chunk(uint32_t* bits, int clear);
hipError_t status_conv(uint32_t* bits, int clear);
hipError_t status_recurrent(uint32_t* bits, int clear);
hipError_t status_ssd(uint32_t* bits, int clear);
hipError_t status_kda(uint32_t* bits, int clear);

// A sequence takes part in a call when it has a write block inside the pool and
// a read block inside the pool; anything else is skipped without memory access
// (a negative write block is a padding sequence; any other index outside the
// pool raises kStatusBadIndex).
__device__ __forceinline__ bool seq_active(const int32_t* read_idx, const int32_t* write_idx,
                                           int s, int num_blocks) {
  int rb = read_idx[s], wb = write_idx[s];
  const bool ok = wb >= 0 && wb < num_blocks && rb >= 0 && rb < num_blocks;
  if (!ok && wb >= 0) raise_status(kStatusBadIndex);
  return ok;
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
  const int32_t* skip;  // device plan: the whole launch does nothing when *skip != 0 (NULL: never)
};

struct TailArgs {
  const void* x;
  const int32_t* cu;
  const int32_t* read_idx;
  const int32_t* write_idx;
  char* conv_pool;
  int64_t conv_stride;
  int num_seqs, num_blocks, channels;
  int max_len;  // sequences longer than this are committed elsewhere (the chunk kernel)
  const int32_t* fused;  // device plan: when *fused != 0, max_len is 1 (NULL: use max_len)
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
  int kda;               // token path: g is [T][H_v][d_k], a decay per key channel (Kimi delta attention)
};

// Sequences of the chunked launch, longest first (one workgroup row per entry).
constexpr int kMaxOrder = 1024;
struct SeqOrder {
  int32_t n;                    // entries used; 0 means "every sequence, in index order"
  uint16_t seq[kMaxOrder];
};

// silu: SiLU after the conv; q/k normalisation of the channels below 2 * qk_channels
hipError_t launch_conv(const ConvArgs& a, int width, bool bf16, bool silu, hipStream_t st);
hipError_t launch_tail_commit(const TailArgs& a, int width, bool bf16, hipStream_t st);

// Fork copy: both states of block src[i] to block dst[i].  Sizes and strides
// are multiples of 16 bytes; pairs with an index outside [0, num_blocks) or
// src == dst are skipped.
struct StateCopyArgs {
  char* ssm_pool;
  char* conv_pool;
  int64_t ssm_stride, conv_stride, ssm_bytes, conv_bytes;
  const int32_t* src;
  const int32_t* dst;
  int num_blocks;
};
hipError_t launch_state_copy(const StateCopyArgs& a, int n, hipStream_t st);

// Mamba2 scan (ssd_scan.hip): x, B, C bf16 rows at the given strides (in
// elements, multiples of 8, 16-byte aligned bases), dt [T][H] fp32, y
// [T][H][P] bf16, states [H][P][N] fp32 per block.  One workgroup per
// (sequence, head); P = 64 and N = 128 only (ssd_supported).
struct SsdArgs {
  const uint16_t* x;
  const uint16_t* b;
  const uint16_t* c;
  int64_t x_stride, bc_stride;
  const float* dt;
  const float* dt_bias;  // may be null
  const float* A;
  const float* D;        // may be null
  const int32_t* cu;
  const int32_t* read_idx;
  const int32_t* write_idx;
  float* pool;
  int64_t pool_stride;   // floats between blocks
  int num_blocks, num_seqs, num_heads, num_groups, softplus;
  int total_tokens;      // sequences whose offsets leave [0, total_tokens] are skipped
  uint16_t* y;
};
bool ssd_supported(int head_dim, int state_dim);
// sequences of length >= 2; ord (n > 0): only the sequences it lists, one rank
// of workgroups each, in its order (ord.seq[r] < num_seqs)
hipError_t launch_ssd(const SsdArgs& a, const SeqOrder& ord, hipStream_t st);
hipError_t launch_ssd_token(const SsdArgs& a, hipStream_t st);  // sequences of length 0 and 1
hipError_t launch_recurrent(const ScanArgs& a, int dk, int dv, bool bf16, hipStream_t st);
// The conv of the chunked sequences run by the chunk-scan workgroups
// themselves, as tasks they claim before their scans.  Task t belongs to
// rank r of the launch order when first[r] <= t < first[r + 1]; it covers rows
// [cu[s] + b * kConvTaskRows, ...) of sequence s = order.seq[r] and channels
// [c * kConvTaskChannels, ...), with b = (t - first[r]) / slices and
// c = (t - first[r]) % slices.  n == 0: y was written by the conv kernel.
// Each of the workgroup's 8 waves converts kConvWaveRows rows of 512 channels
// of the task; the task is kConvTaskChannels / 512 such segments wide and as
// many 16-row parts deep as the waves fill: one 64-row chunk, so a chunk's
// rows are converted by exactly `slices` tasks.
constexpr int kConvTaskChannels = 1024;
constexpr int kConvWaveRows = 16;
constexpr int kConvTaskRows = kConvWaveRows * 8 * 512 / kConvTaskChannels;
static_assert(kConvTaskChannels % 512 == 0 && 8 * 512 % kConvTaskChannels == 0, "whole wave segments");
static_assert(kConvTaskRows == 64, "a task is one 64-row chunk deep");
constexpr int kMaxFusedRanks = 256;
// Times are in ticks of the 100 MHz real-time counter, counted from the start
// of a workgroup's conv phase.  A workgroup of a sequence with N chunks keeps
// claiming tasks beyond its own sequence's while it can still finish one more
// task and its scan by `target`: its scan is priced scan0 + N * scan1, a task
// `task`.  The figures only steer who converts which rows, never the result.
struct FusedConv {
  int32_t n;         // ranks (entries of the launch order), 0 = no fused conv
  int32_t slices;    // channel slices per row block
  int32_t* sync;     // [0] next task to claim, [1 + r] tasks of rank r finished, [1 + n + first[r] / slices + c]
                     // tasks of chunk c of rank r finished; zero before the launch
  int32_t target, task, scan0, scan1;
  int32_t first[kMaxFusedRanks + 1];
  // Device plan (launches planned on the device from cu_seqlens, see
  // plan_kernel): when non-NULL, n, target, first[] and the launch order come
  // from this array instead, laid out as below, for up to plan_seqs sequences.
  const int32_t* plan;
  int32_t plan_seqs;
  // Streaming (host plan only): the n * H_v scan workgroups start at once and
  // wait chunk by chunk, while `helpers` more workgroups convert rows just
  // ahead of them.  first[r] is then the first chunk of rank r in the ready
  // counters (first[n] = all chunks), and sync holds [0] the next task to
  // claim (in chunk-major order over the ranks), [1, 1 + first[n]) tasks
  // finished per chunk.
  int32_t stream;
  int32_t helpers;
  // 1: a workgroup claims at least until every task of its own sequence is
  // claimed (and beyond that by its time budget); 0: by its time budget alone,
  // except the last rank's workgroups, which claim until every task is claimed
  int32_t own_first;
};
constexpr size_t kFusedSyncBytes = 4096;  // room for sync[0 .. kMaxFusedRanks]

// Device plan layout (int32): [0] chunked sequences n, [1] conv inside the chunk
// kernel (0/1), [2] makespan target (ticks), [3] unused, [4, 4 + N) launch order
// (sequence of each rank), [4 + N, 5 + 2N) first task of each rank and the total.
constexpr int kPlanN = 0, kPlanFused = 1, kPlanTarget = 2, kPlanOrder = 4;
constexpr int kMaxPlanSeqs = 1024;  // one 1024-thread workgroup plans
inline size_t plan_ints(int num_seqs) { return 5 + 2 * (size_t)num_seqs; }

struct PlanArgs {
  const int32_t* cu;
  int num_seqs, num_v_heads, slices, conv_rows;
  int fused_allowed;  // every scan workgroup fits at once, the weights are aligned, no override against
  int fused_forced;   // the override asks for it whenever allowed
  double conv_us_per_token, task_us, scan0_us, scan1_us, margin;
  int cus;  // compute units: the per-chunk scan time after the conv kernel
  double plain_scan1_us, crowd_scan1_us, phased_scale;  // grows with the share of them scanning
  int beside_tokens;  // the token kernel runs beside on a side stream: with one-token sequences, conv inside
  int32_t* plan;
  int32_t* sync;      // zeroed: 1 + n + (chunks of the n chunked sequences) counters
};
hipError_t launch_plan(const PlanArgs& a, hipStream_t st);
hipError_t launch_zero_sync(int32_t* sync, int n, hipStream_t st);  // n counters to zero

hipError_t launch_chunk(const ScanArgs& a, const SeqOrder& order, const FusedConv& fc, int dk, int dv,
                        hipStream_t st);
bool chunk_supported(int dk, int dv);

// Chunked prefill for every other head size and the fp32 layer
// (gdn_chunk_generic.hip): sequences with min_len <= L <= max_len, launch order
// as for launch_chunk, reading the conv output y (act dtype, normalised); fp32
// arithmetic; d_k, d_v in {16, 32, 64, 128} (chunk_generic_supported).
hipError_t launch_chunk_generic(const ScanArgs& a, const SeqOrder& order, int dk, int dv, bool bf16,
                                hipStream_t st);
bool chunk_generic_supported(int dk, int dv);

// Measurement support (gdn_probe.hip): blocks x 256 threads issuing `iters`
// rounds of 8 independent MFMAs per wave (bf16 16x16x32 or fp32 16x16x4); a
// streaming copy of n16 16-byte elements, one 256-thread block per 32 KiB.
hipError_t launch_mfma_probe(bool bf16, int blocks, int iters, hipStream_t st);
hipError_t launch_copy_probe(const void* src, void* dst, int64_t n16, hipStream_t st);

// Kimi delta attention, chunked (kda_chunk.hip): sequences with min_len <= L <= max_len,
// launch order as for launch_chunk, reading the conv output y (bf16, normalised)
// and g [T][H_v][d_k]; d_k = d_v = 128 only (kda_chunk_supported).  fc.n > 0:
// the kernel's workgroups write y themselves first (phased, host plan only;
// fc.sync zeroed: 1 + n + the ranks' chunks counters).
hipError_t launch_kda_chunk(const ScanArgs& a, const SeqOrder& order, const FusedConv& fc, hipStream_t st);
bool kda_chunk_supported(int dk, int dv);

}  // namespace gdn
