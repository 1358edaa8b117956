// gdn_convtask.h -- the conv of the chunked rows run inside a chunk kernel, as
// tasks its own workgroups claim before their scans, and the per-chunk wait of
// the scans for the converted rows.  Shared by the gated delta rule's chunk
// kernel (gdn_chunk.hip) and the KDA chunk kernel (kda_chunk.hip), both one
// 512-thread workgroup per (sequence, value head).
//
// Page "Continuous batching for linear attention layers" (PR description): the
// varlen causal convolution continues every sequence of the packed row from its
// own conv state; SiLU follows, and q and k are L2-normalised per key head.
#pragma once
#include "gdn_device.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int kConvThreads = 512;  // threads per workgroup of the kernels that run the tasks
constexpr int kConvWaves = kConvThreads / 64;

// With the conv inside the kernel: waits until every conv task of chunk c of
// the sequence is counted in ready[c].  Bounded: streaming, the tasks are run
// by helper workgroups that never wait, and every helper has started before
// any scan (see chunk_scan_kernel); phased, every task of the sequence was
// claimed before its workgroups left their conv phase, and a claimed task
// never waits.  After a successful poll an agent-scope acquire fence drops any
// stale copy of the rows from this CU's caches (a workspace reused from an
// earlier call may still be cached from that call).  A wait that gives up
// raises kStatusWaitExpired.  Returns the first chunk from c on that is not
// known to be converted.
__device__ __forceinline__ int chunk_wait(const int32_t* ready, int slices, int L, int c, int upto, int lane) {
  if (c < upto) return upto;
  // lane l looks at chunk c + l: one round trip finds how many chunks from c on
  // are complete, and the scan polls again only after it has used them up
  const int cc = c + lane;
  const int want = slices;  // tasks are one chunk deep
  const bool mine = cc * BT < L;
  for (int it = 0; it < (1 << 24); ++it) {
    const bool ok = !mine || __hip_atomic_load(&ready[cc], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want;
    const uint64_t late = __ballot(!ok);
    if (!(late & 1)) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return c + (late ? __builtin_ctzll(late) : 64);
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (lane == 0) raise_status(kStatusWaitExpired);
  return c + 1;
}


// ---- the conv of the chunked rows, run by the scan workgroups as claimed tasks
//
// Every workgroup first claims conv tasks (kConvTaskRows rows x
// kConvTaskChannels channels of one sequence, each wave converting 16 rows of
// 512 channels) from a counter in global memory, while its scan, priced by
// the host's time model, can still end by the host's estimate of the balanced
// finish.  Two orders (FusedConv::own_first): sequence-major, the longest
// sequence's tasks first, with every workgroup claiming at least until its own
// sequence's tasks are all claimed (the gated delta rule, whose scans would
// catch up with rows converted by others); or chunk-major, every sequence's
// chunk 0 first, then every chunk 1, and so on, by the time budget alone (KDA,
// whose slower scans the conversion stays ahead of).  In both, the last
// sequence's workgroups claim until every task is claimed.  It then starts
// its scan, which waits for each chunk's rows when it first needs them (each
// task is counted for its sequence and for its chunk), so later chunks may
// still be converting by other workgroups while it scans.  A workgroup only
// ever waits for tasks that are already claimed, and a claimed task never
// waits for anything, so every wait ends whatever the number of resident
// workgroups.  The rows are computed exactly as by the conv kernel
// (same tap order, SiLU, and head reduction across the 16 lanes of a key
// head), so y is bitwise the same either way.
//
// Visibility across XCDs without writing back whole L2 caches: the rows are
// stored with device-scope coherence (the SC1 bit, as the compiler emits for an
// agent-scope atomic store), every wave waits for its stores to complete, the
// workgroup meets at a barrier, and only then is the task counted.  A scan
// that has seen a chunk's count complete invalidates its caches (an
// agent-scope acquire fence) before it reads the chunk's rows.
constexpr int kStoreDeviceScope = 16 | 2;  // buffer store cache policy: SC1 (device scope) | NT (streaming)

// The launch order and the conv task plan: from the kernel arguments (planned
// on the host, DP = false), or from the device plan array (planned by
// plan_kernel, DP = true).  Two instantiations, so that the host-planned
// kernel carries no trace of the device plan (registers are at the limit).
template <bool DP>
__device__ __forceinline__ int plan_n(const SeqOrder& ord, const FusedConv& fc) {
  if constexpr (DP) return fc.plan[kPlanN];
  else return ord.n;
}
template <bool DP>
__device__ __forceinline__ int plan_fused_n(const FusedConv& fc) {
  if constexpr (DP) return fc.plan[kPlanFused] ? fc.plan[kPlanN] : 0;
  else return fc.n;
}
template <bool DP>
__device__ __forceinline__ int plan_seq(const SeqOrder& ord, const FusedConv& fc, int r) {
  if constexpr (DP) return fc.plan[kPlanOrder + r];
  else return (int)ord.seq[r];
}
template <bool DP>
__device__ __forceinline__ int plan_first(const FusedConv& fc, int r) {
  if constexpr (DP) return fc.plan[kPlanOrder + fc.plan_seqs + r];
  else return fc.first[r];
}
template <bool DP>
__device__ __forceinline__ int32_t plan_target(const FusedConv& fc) {
  if constexpr (DP) return fc.plan[kPlanTarget];
  else return fc.target;
}

// One task as one wave sees it: the wave's rows [r0, r0 + n) of sequence s
// (rows from seq0; n <= 0 past the sequence's end) at channels c0..c0+7 of
// each thread; `on` is false for the threads past the channel count or the
// sequence's end.  `row` is the task's first row group (in kConvTaskRows).
struct ConvTask {
  int rank, s, seq0, r0, n, c0, row;
  bool on;
};

// Wave wv's part of the task at row group b and channel slice c of sequence s:
// 16 rows of 512 channels.  Every value but c0 is uniform over the wave.
__device__ __forceinline__ void conv_part(const ScanArgs& a, ConvTask& k, int b, int c) {
  constexpr int kSegWaves = kConvTaskChannels / 512;  // waves across the task's channels
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  k.row = b;
  k.r0 = k.seq0 + b * kConvTaskRows + (wv / kSegWaves) * kConvWaveRows;
  k.n = min(kConvWaveRows, a.cu[k.s + 1] - k.r0);
  k.c0 = c * kConvTaskChannels + (wv % kSegWaves) * 512 + ((int)threadIdx.x & 63) * 8;
  k.on = k.c0 < a.channels && k.n > 0;
}

template <bool DP>
__device__ __forceinline__ ConvTask conv_decode(const ScanArgs& a, const SeqOrder& ord, const FusedConv& fc, int t) {
  int lo = 0, loc = 0;
  if (!DP && !fc.own_first) {
    // chunk-major: every rank's chunk 0, then every rank's chunk 1, ...  The
    // ranks run longest first, so those that still hold chunk c are a prefix
    const int S = fc.slices;
    int c0 = 0, g = t;
    for (int act = fc.n; act >= 1; --act) {  // chunks [c0, c1) are held by ranks 0 .. act-1
      const int c1 = (fc.first[act] - fc.first[act - 1]) / S;
      const int span = (c1 - c0) * act * S;
      if (g < span) {
        const int c = c0 + g / (act * S), j = g % (act * S);
        lo = j / S;
        loc = c * S + j % S;
        break;
      }
      g -= span;
      c0 = c1;
    }
  } else {
    int hi = plan_fused_n<DP>(fc);  // rank of task t: first[r] <= t < first[r + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (plan_first<DP>(fc, mid) <= t) lo = mid; else hi = mid;
    }
    loc = t - plan_first<DP>(fc, lo);
  }
  ConvTask k;
  k.rank = lo;
  k.s = plan_seq<DP>(ord, fc, lo);
  k.seq0 = a.cu[k.s];
  conv_part(a, k, loc / fc.slices, loc % fc.slices);
  return k;
}

// Halo and taps of a task in registers: the W-1 inputs before r0 (earlier rows
// of the sequence, else its conv state, else zero) and w[c][j] (8 channels x W
// contiguous).  The task's rows go through LDS (conv_prefetch).
template <int W>
struct ConvSide {
  u32x4 hx[W > 1 ? W - 1 : 1];
  u32x4 wr[W];
};

// During the conv phase the LDS of the scan is free: it stages the rows of the
// next task.  Wave w's 512-channel segment of row r sits at (8 r + w) KiB,
// lane l's 16 bytes at + 16 l, so every wave reads back only what it loaded.
// SM: the kernel's LDS struct, at least 128 KiB with an int `task` past them.
template <typename SM>
__device__ __forceinline__ u32x4* conv_stage(SM& sm) { return reinterpret_cast<u32x4*>(&sm); }

// Issues the loads of task k: halo and taps into `sd`, the rows straight into
// LDS (no registers), all in flight while the current task is computed.
template <int W, typename SM>
__device__ __forceinline__ void conv_prefetch(SM& sm, const ScanArgs& a, const ConvTask& k, ConvSide<W>& sd) {
  if (!k.on) return;
  const int C = a.channels;
  const int64_t cq = k.c0 / 8;  // 16-byte column of this thread
  const gptr<const u32x4> x = as_global(reinterpret_cast<const u32x4*>(a.x));
  const bool act = seq_active(a.read_idx, a.write_idx, k.s, a.num_blocks);
#pragma unroll
  for (int j = 1; j < W; ++j) {
    const int p = k.r0 - j;
    sd.hx[j - 1] = u32x4{0u, 0u, 0u, 0u};
    if (p >= k.seq0) {
      sd.hx[j - 1] = x[(int64_t)p * (C / 8) + cq];
    } else if (act) {
      const gptr<const u32x4> tail =
          as_global(reinterpret_cast<const u32x4*>(a.conv_pool + (int64_t)a.read_idx[k.s] * a.conv_stride));
      sd.hx[j - 1] = tail[(int64_t)(W - 1 + p - k.seq0) * (C / 8) + cq];
    }
  }
  const gptr<const u32x4> wp =
      as_global(reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.w) + (int64_t)k.c0 * W));
#pragma unroll
  for (int i = 0; i < W; ++i) sd.wr[i] = wp[i];
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int r0 = __builtin_amdgcn_readfirstlane(k.r0), n = __builtin_amdgcn_readfirstlane(k.n);
  const __amdgpu_buffer_rsrc_t xs =
      make_rsrc(reinterpret_cast<const uint16_t*>(a.x) + (int64_t)r0 * C, (uint32_t)(n * C * 2));
  u32x4* st = conv_stage(sm);
#pragma unroll
  for (int r = 0; r < kConvWaveRows; ++r)  // rows past the wave's end load its last row again
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (__attribute__((address_space(3))) void*)(st + (r * kConvWaves + wv) * 64),
                                             16, (min(r, n - 1) * C + k.c0) * 2, 0, 0, 0);
}

// Sum over the 16 lanes of a key head (a DPP row): the same pairings as a
// butterfly over lane xor 1, 2, 4, 8, and the same steps as the conv kernel's
// group_sum, so every lane ends with the bits the conv kernel computes (each
// step adds two equal partial sums of the two halves, and the order of the
// two does not change a float sum).
__device__ __forceinline__ float head_sum(float v) {
  v += dpp_move<0xB1, 0xf>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_move<0x4E, 0xf>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_move<0x141, 0xf>(v);  // row_half_mirror: lane 7 - i within 8, the other quad
  v += dpp_move<0x140, 0xf>(v);  // row_mirror: lane 15 - i, the other half row
  return v;
}

// Computes and stores task k from its rows (registers) and its halo and taps.
template <int W>
__device__ __forceinline__ void conv_compute(const ScanArgs& a, const ConvTask& k, const ConvSide<W>& sd,
                                             const u32x4 (&rx)[kConvWaveRows]) {
  if (!k.on) return;  // whole 16-lane head groups (the channel count is a multiple of 128)
  const int C = a.channels;
  float wt[8][W];
#pragma unroll
  for (int i = 0; i < 8 * W; ++i) {
    const uint32_t word = sd.wr[i / 8][(i % 8) / 2];
    wt[i / W][i % W] = __uint_as_float((i & 1) ? (word & 0xffff0000u) : (word << 16));
  }
  const bool do_norm = k.c0 < 2 * a.num_k_heads * D;
  const float scale = k.c0 < a.num_k_heads * D ? a.q_scale : 1.0f;
  float xw[4][8];  // the last 4 inputs, slot (row mod 4)
#pragma unroll
  for (int j = 1; j < W; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xw[(4 - j) & 3][2 * i] = __uint_as_float(sd.hx[j - 1][i] << 16);
      xw[(4 - j) & 3][2 * i + 1] = __uint_as_float(sd.hx[j - 1][i] & 0xffff0000u);
    }
  // the task is the same for the whole workgroup: its rows in scalar registers
  // keep the descriptor scalar
  const int r0 = __builtin_amdgcn_readfirstlane(k.r0), n = __builtin_amdgcn_readfirstlane(k.n);
  const __amdgpu_buffer_rsrc_t ys =
      make_rsrc(reinterpret_cast<const uint16_t*>(a.y) + (int64_t)r0 * C, (uint32_t)(n * C * 2));
#pragma unroll
  for (int r = 0; r < kConvWaveRows; ++r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xw[r & 3][2 * i] = __uint_as_float(rx[r][i] << 16);
      xw[r & 3][2 * i + 1] = __uint_as_float(rx[r][i] & 0xffff0000u);
    }
    float yv[8];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = wt[e][W - 1] * xw[r & 3][e];
#pragma unroll
      for (int j = 1; j < W; ++j) acc += wt[e][W - 1 - j] * xw[(r - j) & 3][e];
      yv[e] = silu(acc);
      ss += yv[e] * yv[e];
    }
    ss = head_sum(ss);
    if (do_norm) {
      const float inv = scale * rsqrt_fast(ss + a.eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[e] *= inv;
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(yv[2 * i], yv[2 * i + 1]);
    if (r < n) __builtin_amdgcn_raw_buffer_store_b128(o, ys, (r * C + k.c0) * 2, 0, kStoreDeviceScope);
  }
}

// Thread 0: claim one more task after the newest claimed one, while my rank
// has unclaimed tasks or there is time for it before my scan.
__device__ __forceinline__ int claim_after(const FusedConv& fc, int newest, int total, int last, int32_t latest,
                                           uint64_t t_begin) {
  if (newest >= total) return total;
  if (newest < last - 1 || (int64_t)(__builtin_amdgcn_s_memrealtime() - t_begin) <= latest)
    return __hip_atomic_fetch_add(fc.sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return total;
}

// Claims and runs conv tasks, at least until every task of `rank` is claimed
// (the scan then waits for them chunk by chunk).  All threads of the workgroup
// call it.  While a task is computed from registers, the rows of the next
// claimed task are loading into LDS, and a third task is being claimed.  On
// return no LDS access or load of the phase is outstanding.
template <bool DP, int W, typename SM>
__device__ void conv_phase(SM& sm, const ScanArgs& a, const SeqOrder& ord, const FusedConv& fc, int rank) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_ranks = plan_fused_n<DP>(fc);
  const int total = plan_first<DP>(fc, n_ranks);
  // claim at least until this task index (my rank's tasks end there; with
  // own_first off, only the last rank holds to it, every task then)
  const int last = (fc.own_first || rank == n_ranks - 1) ? plan_first<DP>(fc, rank + 1) : 0;
  // latest claim of a task that two more precede before my scan
  const int my_s = plan_seq<DP>(ord, fc, rank);
  const int32_t latest =
      plan_target<DP>(fc) - fc.scan0 - fc.scan1 * ((a.cu[my_s + 1] - a.cu[my_s] + BT - 1) / BT) - 3 * fc.task;
  const uint64_t t_begin = __builtin_amdgcn_s_memrealtime();
  // the first claim as the later ones (with own_first set, always taken)
  if (tid == 0) sm.task = claim_after(fc, -1, total, last, latest, t_begin);
  lds_barrier();
  int t = __builtin_amdgcn_readfirstlane(sm.task);
  lds_barrier();  // every thread has read sm.task before thread 0 writes it again
  ConvTask k{};
  ConvSide<W> cur, nxt;
  if (t < total) {
    k = conv_decode<DP>(a, ord, fc, t);
    conv_prefetch<W>(sm, a, k, nxt);
  }
  if (tid == 0) sm.task = claim_after(fc, t, total, last, latest, t_begin);
  lds_barrier();
  int u = __builtin_amdgcn_readfirstlane(sm.task);
  u32x4 rx[kConvWaveRows];
  const u32x4* st = conv_stage(sm);
  while (t < total) {
    // this task's rows and halo have arrived; read the rows back from LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    cur = nxt;
    if (k.on) {
#pragma unroll
      for (int r = 0; r < kConvWaveRows; ++r) rx[r] = st[(r * kConvWaves + wv) * 64 + lane];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the next rows overwrite them
    lds_barrier();  // every thread has read sm.task (u)
    ConvTask kn{};
    if (u < total) {
      kn = conv_decode<DP>(a, ord, fc, u);
      conv_prefetch<W>(sm, a, kn, nxt);
    }
    int v = total;
    if (tid == 0) v = claim_after(fc, u, total, last, latest, t_begin);
    conv_compute<W>(a, k, cur, rx);
    if (tid == 0) sm.task = v;
    // this task's device-scope stores complete (and the next task's loads),
    // then the counts: its rank's, and its chunk's (the scans wait on these)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (tid == 0) {
      __hip_atomic_fetch_add(&fc.sync[1 + k.rank], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&fc.sync[1 + n_ranks + plan_first<DP>(fc, k.rank) / fc.slices + k.row], 1,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    k = kn;
    t = u;
    u = __builtin_amdgcn_readfirstlane(sm.task);
  }
}

// Waits until every conv task of `rank` is counted, then makes their rows
// visible to this workgroup.  Bounded: every task counted here is claimed (the
// workgroup claimed past them before it stopped) and finishes without waiting.
template <bool DP>
__device__ __forceinline__ void conv_wait(const FusedConv& fc, int rank) {
  if (threadIdx.x == 0) {
    const int need = plan_first<DP>(fc, rank + 1) - plan_first<DP>(fc, rank);
    bool done = false;
    for (int it = 0; it < (1 << 24) && !done; ++it) {
      done = __hip_atomic_load(&fc.sync[1 + rank], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need;
      if (!done) __builtin_amdgcn_s_sleep(2);
    }
    if (!done) raise_status(kStatusWaitExpired);
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

template <bool DP, typename SM>
__device__ __forceinline__ void conv_phase_w(SM& sm, const ScanArgs& a, const SeqOrder& ord, const FusedConv& fc,
                                             int rank) {
  switch (a.width) {
    case 1: conv_phase<DP, 1>(sm, a, ord, fc, rank); break;
    case 2: conv_phase<DP, 2>(sm, a, ord, fc, rank); break;
    case 3: conv_phase<DP, 3>(sm, a, ord, fc, rank); break;
    default: conv_phase<DP, 4>(sm, a, ord, fc, rank); break;
  }
}

}  // namespace
}  // namespace gdn
