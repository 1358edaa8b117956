// gdn_api.cpp -- the C ABI (include/gdn.h): argument checks, launch planning
// from the host copy of cu_seqlens, and the kernel launches on the caller's
// stream.  No device memory is allocated and nothing synchronises with the host.
//
// Planning follows the page "Continuous batching for linear attention layers":
// the linear layers' state indices hold one entry per sequence (allocator
// commit), the prefill path must not sync with the host (the PR notes the fla
// chunked kernel does, which keeps accelerator graphs off), and the engine's
// batch preparation (page input_ouputs.py, prepare_batch_tensors) builds
// cu_seqlens on the host and rejects an empty batch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_device.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool pow2_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

int check_desc(const gdn_layer_desc* d) {
  if (!d) return fail(GDN_EINVAL, "layer descriptor is NULL");
  if (d->num_k_heads < 1 || d->num_v_heads < 1)
    return fail(GDN_EINVAL, "head counts must be >= 1 (H_k=%d, H_v=%d)", d->num_k_heads, d->num_v_heads);
  if (d->num_v_heads % d->num_k_heads != 0)
    return fail(GDN_EINVAL, "H_v=%d is not a multiple of H_k=%d", d->num_v_heads, d->num_k_heads);
  if (d->act_dtype != GDN_F32 && d->act_dtype != GDN_BF16)
    return fail(GDN_EINVAL, "act_dtype %d is neither GDN_F32 nor GDN_BF16", d->act_dtype);
  if (!(d->l2norm_eps >= 0.0f)) return fail(GDN_EINVAL, "l2norm_eps must be >= 0");
  if (d->head_k_dim < 1 || d->head_v_dim < 1)
    return fail(GDN_EINVAL, "head dims must be >= 1 (d_k=%d, d_v=%d)", d->head_k_dim, d->head_v_dim);
  if (d->conv_width < 1) return fail(GDN_EINVAL, "conv_width must be >= 1 (got %d)", d->conv_width);
  if (!pow2_dim(d->head_k_dim) || !pow2_dim(d->head_v_dim))
    return fail(GDN_EUNSUPPORTED, "head dims must be 16, 32, 64 or 128 (d_k=%d, d_v=%d)", d->head_k_dim,
                d->head_v_dim);
  if (d->conv_width > 4) return fail(GDN_EUNSUPPORTED, "conv_width %d > 4 is not built", d->conv_width);
  const int64_t C = 2LL * d->num_k_heads * d->head_k_dim + (int64_t)d->num_v_heads * d->head_v_dim;
  if (C > INT_MAX / 8) return fail(GDN_EUNSUPPORTED, "too many conv channels (%lld)", (long long)C);
  return GDN_OK;
}

int64_t channels(const gdn_layer_desc* d) {
  return 2LL * d->num_k_heads * d->head_k_dim + (int64_t)d->num_v_heads * d->head_v_dim;
}

int64_t act_size(const gdn_layer_desc* d) { return d->act_dtype == GDN_BF16 ? 2 : 4; }

int64_t conv_state_bytes(const gdn_layer_desc* d) { return (int64_t)(d->conv_width - 1) * channels(d) * act_size(d); }

int64_t ssm_state_bytes(const gdn_layer_desc* d) {
  return (int64_t)d->num_v_heads * d->head_k_dim * d->head_v_dim * 4;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The workspace holds the conv output of the packed row for the chunked
// prefill, the task counters of the conv run inside the scan kernel, and the
// device plan (used when the launch is planned on the device).
struct WsLayout {
  size_t sync, plan, total;
};
WsLayout ws_layout(const gdn_layer_desc* d, int64_t total_tokens, int64_t num_seqs) {
  WsLayout l{0, 0, 0};
  if (total_tokens <= 0) return l;
  l.sync = round_up((size_t)total_tokens * (size_t)channels(d) * (size_t)act_size(d), 256);
  // counters: phased conv 1 + N; streaming 1 + chunks (at most T/64 + N)
  const size_t ns = (size_t)std::max<int64_t>(num_seqs, 0);
  const size_t sync_bytes = std::max(gdn::kFusedSyncBytes, 4 * (2 + 3 * ns + (size_t)total_tokens / 64));
  l.plan = l.sync + round_up(sync_bytes, 256);
  l.total = l.plan + round_up(4 * gdn::plan_ints((int)std::min<int64_t>(std::max<int64_t>(num_seqs, 0), INT_MAX / 4)), 256);
  return l;
}
size_t workspace_bytes_for(const gdn_layer_desc* d, int64_t total_tokens, int64_t num_seqs) {
  return ws_layout(d, total_tokens, num_seqs).total;
}

// Time model of the fused prefill (microseconds, measured on MI355X with the
// 128 x 128 head): a scan takes kScan0Us + kScan1Us per chunk; a conv task
// moves its rows in and out at about 17 GB/s per workgroup; the conv kernel
// runs at about 4.2 TB/s; the makespan target sits 3% past the even spread of
// all conv and scan work over the workgroups (3% measured best of 0-10%).
constexpr double kScan0Us = 11.0, kScan1Us = 2.8, kTaskBytesPerUs = 17e3, kConvBytesPerUs = 4.2e6;
constexpr double kTargetMargin = 1.03;

// Choice of the conv placement, fitted to a sweep over 1-8 equal sequences of
// 1024-32768 tokens, one long sequence beside short ones, and the prefill mix:
// - conv kernel first: a scan then takes kScanPlainUs per chunk while at most
//   half the CUs scan, rising by up to kScanCrowdUs with every CU scanning;
// - phased: the estimate above runs about 5% high on long sequences
//   (kPhasedScale);
// - streamed: kStreamStartUs of start-up and kStreamScanScale on the longest
//   scan (it runs beside the helpers' traffic), unless the helpers are the
//   bound: each converts a task's rows at about kHelperBytesPerUs.
constexpr double kScanPlainUs = 2.55, kScanCrowdUs = 0.65, kPhasedScale = 0.95;
constexpr double kStreamStartUs = 40.0, kStreamScanScale = 1.06, kHelperBytesPerUs = 18.7e3;
// The claim rule of the phased conv, chosen per batch.  Sequence-major with
// every workgroup claiming until its own sequence's tasks are claimed (the
// constants above) suits batches of similar lengths; chunk-major by time budget
// alone (FusedConv::own_first = 0) lets the long sequences start their scans
// at once while the short ones convert, which suits skewed batches.  The
// budgets of the latter take the per-workgroup timeline's constants: a scan
// of kCalScan0Us + kCalScan1Us per chunk, a task of kCalTaskUs, and a target
// kBudgetSlackTasks tasks past the larger of the even spread and the longest
// scan (a multiple of the even spread fails small batches, whose target sits
// at that bound: every budget would go negative).  Measured (ms, own tasks ->
// budget): 4 x 4096 beside 4 x 128 0.312 -> 0.250; 4096, 4096, 2048, 2048,
// 1024, 1024, 512, 256: 0.261 -> 0.246; 4 x 2048 beside 4 x 64 0.170 -> 0.152;
// but the prefill mix 0.281 -> 0.283, eight of 2500 0.280 -> 0.281 and the
// mixed step 0.093 -> 0.096, which the estimates below keep on their own tasks.
constexpr double kCalScan0Us = 4.5, kCalScan1Us = 2.95, kCalTaskUs = 12.5, kBudgetSlackTasks = 2.0;
// The KDA chunk kernel's scan: kKdaScan0Us + kKdaScan1Us per chunk (measured on
// MI355X, 128 x 128 head); the conv inside it is placed by the phased rule.
constexpr double kKdaScan0Us = 10.0, kKdaScan1Us = 8.3;

double plain_scan1(int64_t wgs, int cus) {
  const double half = std::max(cus, 2) / 2.0;
  return kScanPlainUs + kScanCrowdUs * std::min(1.0, std::max(0.0, (wgs - half) / half));
}

double task_us(int C, const gdn_layer_desc* d) {
  return 2.0 * gdn::kConvTaskRows * std::min(C, gdn::kConvTaskChannels) * act_size(d) / kTaskBytesPerUs;
}

// GDN_CONV_IN_SCAN: "always" runs the conv inside the chunk kernel (phased)
// whenever its workgroups all fit on the device, "stream" streams it from
// helper workgroups whenever at least 32 CUs are left for them, "never" always
// runs the conv kernel, anything else (or unset) lets the time model choose.  The result is the same
// bit for bit either way; the override exists for tests and tuning.
int conv_in_scan_mode() {
  const char* v = getenv("GDN_CONV_IN_SCAN");
  if (!v) return 0;
  if (!strcmp(v, "always")) return 1;   // the phased conv inside the chunk kernel
  if (!strcmp(v, "stream")) return 2;   // streaming, when there are spare CUs for helpers
  if (!strcmp(v, "never")) return -1;
  return 0;
}

// GDN_CONV_CLAIM: "own" keeps the phased conv's workgroups claiming until
// their own sequence's tasks are claimed, "budget" makes them claim by time
// budget alone; unset (or anything else), the host's estimates choose.
int conv_claim_mode() {
  const char* v = getenv("GDN_CONV_CLAIM");
  if (!v) return 0;
  if (!strcmp(v, "own")) return 1;
  if (!strcmp(v, "budget")) return 2;
  return 0;
}

// Compute units of the device that owns `st` (0 if unknown), looked up once per device.
int device_cus(hipStream_t st) {
  static std::mutex mu;
  static std::vector<int> cus;
  int dev = 0;
  if (hipStreamGetDevice(st, &dev) != hipSuccess || dev < 0) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cus.size() <= dev) cus.resize(dev + 1, -1);
  if (cus[dev] < 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
  }
  return cus[dev];
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// ---- optional per-kernel event timing (measurement only)
enum { K_CONV = 0, K_CHUNK, K_TOKEN, K_TAIL, K_COPY, K_ZERO, K_PLAN, K_SSD, K_SSD_TOKEN, K_KDA_CHUNK, K_CHUNK_GEN,
       K_COUNT };
const char* const kKernelNames[K_COUNT] = {"conv_silu_norm", "chunk_scan", "token_recurrent", "conv_state_commit",
                                           "state_copy", "task_counter_reset", "device_plan", "ssd_scan",
                                           "ssd_token", "kda_chunk", "chunk_generic"};

struct Timing {
  std::mutex mu;
  bool on = false;
  struct Rec { int k; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> spare;
  double total_ms[K_COUNT] = {};
  int64_t launches[K_COUNT] = {};
};
Timing g_timing;

hipEvent_t take_event() {
  if (!g_timing.spare.empty()) {
    hipEvent_t e = g_timing.spare.back();
    g_timing.spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  // timing only: no system-scope fence, which would write back and invalidate
  // the caches between the kernels it brackets and slow the step down
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` (which enqueues one kernel on st), bracketed by events when timing is on.
template <class F>
hipError_t timed(int k, hipStream_t st, F launch) {
  if (!g_timing.on) return launch();
  std::lock_guard<std::mutex> lock(g_timing.mu);
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) {
    if (a) g_timing.spare.push_back(a);
    if (b) g_timing.spare.push_back(b);
    return launch();
  }
  if (hipEventRecord(a, st) != hipSuccess) {  // this launch goes untimed
    g_timing.spare.push_back(a);
    g_timing.spare.push_back(b);
    return launch();
  }
  const hipError_t e = launch();
  if (hipEventRecord(b, st) != hipSuccess) {
    g_timing.spare.push_back(a);
    g_timing.spare.push_back(b);
    return e;
  }
  g_timing.pending.push_back({k, a, b});
  return e;
}

}  // namespace

extern "C" int gdn_kernel_timing(int enable) {
  std::lock_guard<std::mutex> lock(g_timing.mu);
  if (enable) {
    for (auto& r : g_timing.pending) {
      if (hipEventSynchronize(r.b) == hipSuccess) {
        g_timing.spare.push_back(r.a);
        g_timing.spare.push_back(r.b);
      } else {  // not reused: an event in an error state would spoil later timings
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
      }
    }
    g_timing.pending.clear();
    for (int k = 0; k < K_COUNT; ++k) { g_timing.total_ms[k] = 0; g_timing.launches[k] = 0; }
  }
  g_timing.on = enable != 0;
  return GDN_OK;
}

extern "C" int gdn_mfma_peak_probe(int32_t dtype, int32_t iters, double* tflops, void* stream) {
  if (!tflops) return fail(GDN_EINVAL, "tflops is NULL");
  if (dtype != GDN_BF16 && dtype != GDN_F32) return fail(GDN_EINVAL, "dtype %d is neither GDN_BF16 nor GDN_F32", dtype);
  if (iters < 1 || iters > (1 << 20)) return fail(GDN_EINVAL, "iters=%d outside [1, 2^20]", iters);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int cus = device_cus(st);
  if (cus <= 0) return fail(GDN_EHIP, "could not read the device's compute unit count");
  const int blocks = 4 * cus;  // 16 waves per CU, four per SIMD
  const bool bf16 = dtype == GDN_BF16;
  hipEvent_t ev[2] = {nullptr, nullptr};
  hipError_t e = hipEventCreate(&ev[0]);
  if (e == hipSuccess) e = hipEventCreate(&ev[1]);
  if (e == hipSuccess) e = gdn::launch_mfma_probe(bf16, blocks, iters, st);  // warm-up
  if (e == hipSuccess) e = hipEventRecord(ev[0], st);
  if (e == hipSuccess) e = gdn::launch_mfma_probe(bf16, blocks, iters, st);
  if (e == hipSuccess) e = hipEventRecord(ev[1], st);
  if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
  for (hipEvent_t v : ev)
    if (v) (void)hipEventDestroy(v);  // clean-up: the probe's own status is e
  if (e != hipSuccess) return fail(GDN_EHIP, "MFMA probe: %s", hipGetErrorString(e));
  const double flop_per = bf16 ? 16.0 * 16 * 32 * 2 : 16.0 * 16 * 4 * 2;
  *tflops = (double)blocks * 4 * iters * 8 * flop_per / (ms * 1e-3) / 1e12;
  return GDN_OK;
}

extern "C" int gdn_hbm_copy_probe(const void* src, void* dst, int64_t bytes, int32_t reps, double* gbs,
                                  void* stream) {
  if (!gbs) return fail(GDN_EINVAL, "gbs is NULL");
  if (!src || !dst) return fail(GDN_EINVAL, "src or dst is NULL");
  if (bytes <= 0 || bytes % 16 != 0 || bytes > ((int64_t)1 << 36))
    return fail(GDN_EINVAL, "bytes=%lld is not a positive multiple of 16 up to 2^36", (long long)bytes);
  if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return fail(GDN_EINVAL, "src or dst is not 16-byte aligned");
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes) return fail(GDN_EINVAL, "src and dst overlap");
  if (reps < 1 || reps > 1000) return fail(GDN_EINVAL, "reps=%d outside [1, 1000]", reps);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t n16 = bytes / 16;
  hipEvent_t ev[2] = {nullptr, nullptr};
  hipError_t e = hipEventCreate(&ev[0]);
  if (e == hipSuccess) e = hipEventCreate(&ev[1]);
  if (e == hipSuccess) e = gdn::launch_copy_probe(src, dst, n16, st);  // warm-up
  if (e == hipSuccess) e = hipEventRecord(ev[0], st);
  for (int r = 0; r < reps && e == hipSuccess; ++r) e = gdn::launch_copy_probe(src, dst, n16, st);
  if (e == hipSuccess) e = hipEventRecord(ev[1], st);
  if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
  for (hipEvent_t v : ev)
    if (v) (void)hipEventDestroy(v);  // clean-up: the probe's own status is e
  if (e != hipSuccess) return fail(GDN_EHIP, "copy probe: %s", hipGetErrorString(e));
  *gbs = 2.0 * (double)bytes * reps / (ms * 1e-3) / 1e9;
  return GDN_OK;
}

extern "C" int gdn_kernel_times(gdn_kernel_time* out, int32_t max, int32_t* count) {
  std::lock_guard<std::mutex> lock(g_timing.mu);
  for (auto& r : g_timing.pending) {
    hipError_t e = hipEventSynchronize(r.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return fail(GDN_EHIP, "kernel timing: %s", hipGetErrorString(e));
    g_timing.total_ms[r.k] += ms;
    g_timing.launches[r.k] += 1;
    g_timing.spare.push_back(r.a);
    g_timing.spare.push_back(r.b);
  }
  g_timing.pending.clear();
  int n = 0;
  for (int k = 0; k < K_COUNT; ++k) {
    if (!g_timing.launches[k]) continue;
    if (out && n < max) {
      memset(&out[n], 0, sizeof(out[n]));
      snprintf(out[n].name, sizeof(out[n].name), "%s", kKernelNames[k]);
      out[n].total_ms = g_timing.total_ms[k];
      out[n].launches = g_timing.launches[k];
    }
    ++n;
  }
  if (count) *count = n;
  return GDN_OK;
}

extern "C" int gdn_state_spec(const gdn_layer_desc* desc, gdn_state_decl out[2]) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!out) return fail(GDN_EINVAL, "output array is NULL");
  memset(out, 0, 2 * sizeof(gdn_state_decl));
  snprintf(out[0].name, sizeof(out[0].name), "conv");
  out[0].ndim = 2;
  out[0].shape[0] = desc->conv_width - 1;
  out[0].shape[1] = channels(desc);
  out[0].dtype = desc->act_dtype;
  out[0].bytes = conv_state_bytes(desc);
  out[0].align = 128;
  snprintf(out[1].name, sizeof(out[1].name), "recurrent");
  out[1].ndim = 3;
  out[1].shape[0] = desc->num_v_heads;
  out[1].shape[1] = desc->head_k_dim;
  out[1].shape[2] = desc->head_v_dim;
  out[1].dtype = GDN_F32;
  out[1].bytes = ssm_state_bytes(desc);
  out[1].align = 128;
  return GDN_OK;
}

extern "C" int gdn_workspace_size(const gdn_layer_desc* desc, int32_t total_tokens, int32_t num_seqs,
                                  size_t* bytes) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!bytes) return fail(GDN_EINVAL, "bytes is NULL");
  if (total_tokens < 0 || num_seqs < 0) return fail(GDN_EINVAL, "negative token or sequence count");
  *bytes = workspace_bytes_for(desc, total_tokens, num_seqs);
  return GDN_OK;
}

extern "C" const char* gdn_last_error(void) { return g_last_error.c_str(); }

extern "C" int gdn_device_status(int clear, uint32_t* bits, void* stream) {
  hipError_t e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GDN_EHIP, "device status: %s", hipGetErrorString(e));
  uint32_t v = 0;
  for (auto fn : {gdn::status_chunk, gdn::status_conv, gdn::status_recurrent, gdn::status_ssd, gdn::status_kda}) {
    e = fn(&v, clear);
    if (e != hipSuccess) return fail(GDN_EHIP, "device status: %s", hipGetErrorString(e));
  }
  if (bits) *bits = v;
  if (!v) return GDN_OK;
  return fail(GDN_EDEVICE, "device status 0x%x:%s%s", v,
              (v & GDN_DEV_WAIT_EXPIRED) ? " a bounded wait gave up (that call's results are not valid);" : "",
              (v & GDN_DEV_BAD_INDEX) ? " a state block index outside the pool was skipped;" : "");
}

namespace {

// A mixed step (decode tokens beside chunked sequences) runs the token path on
// a side stream beside the conv and chunk kernels: they touch disjoint
// sequences and blocks, and the token kernel is HBM-bound while the chunk
// kernel is latency-bound, so the two overlap.  One side stream and one pair of
// events per device, created on first use (default priority, non-blocking);
// fork and join are event records and waits, so the call stays asynchronous
// and capturable.  Each record and its wait are made under one lock, so calls
// from several threads never wait on each other's records.
struct Side {
  std::mutex mu;
  std::vector<hipStream_t> stream;
  std::vector<hipEvent_t> fork_ev, join_ev;
};
Side g_side;

hipError_t fork_side(hipStream_t st, hipStream_t* side) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_side.mu);
  if ((int)g_side.stream.size() <= dev) {
    g_side.stream.resize(dev + 1, nullptr);
    g_side.fork_ev.resize(dev + 1, nullptr);
    g_side.join_ev.resize(dev + 1, nullptr);
  }
  if (!g_side.stream[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    hipStream_t s = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    const unsigned fl = hipEventDisableTiming | hipEventDisableSystemFence;
    e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&a, fl);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&b, fl);
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) {  // nothing half-made is kept
      if (b) (void)hipEventDestroy(b);
      if (a) (void)hipEventDestroy(a);
      if (s) (void)hipStreamDestroy(s);
      return e;
    }
    g_side.stream[dev] = s;
    g_side.fork_ev[dev] = a;
    g_side.join_ev[dev] = b;
    if (back != hipSuccess) return back;  // the caller's device could not be restored
  }
  *side = g_side.stream[dev];
  if ((e = hipEventRecord(g_side.fork_ev[dev], st)) != hipSuccess) return e;
  return hipStreamWaitEvent(*side, g_side.fork_ev[dev], 0);
}

hipError_t join_side(hipStream_t st, hipStream_t side) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(side, &dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_side.mu);
  if ((e = hipEventRecord(g_side.join_ev[dev], side)) != hipSuccess) return e;
  return hipStreamWaitEvent(st, g_side.join_ev[dev], 0);
}

}  // namespace

namespace {
// The whole forward with the scratch it needs at `workspace`; `noalloc` says
// the scratch is the library's static buffer (looked up only once every host
// check has passed, so a rejected call touches no device).
int forward_impl(const gdn_layer_desc* desc, const void* x, const void* conv_weight, const float* g,
                 const float* beta, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t num_seqs,
                 int32_t total_tokens, const int32_t* read_idx, const int32_t* write_idx, void* conv_pool,
                 int64_t conv_block_stride, float* ssm_pool, int64_t ssm_block_stride, int32_t num_blocks,
                 void* out, void* workspace, size_t workspace_bytes, void* stream, bool noalloc);
}  // namespace

extern "C" int gdn_varlen_forward(const gdn_layer_desc* desc, const void* x, const void* conv_weight,
                                  const float* g, const float* beta, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t total_tokens,
                                  const int32_t* read_idx, const int32_t* write_idx, void* conv_pool,
                                  int64_t conv_block_stride, float* ssm_pool, int64_t ssm_block_stride,
                                  int32_t num_blocks, void* out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return forward_impl(desc, x, conv_weight, g, beta, cu_seqlens, cu_seqlens_host, num_seqs, total_tokens, read_idx,
                      write_idx, conv_pool, conv_block_stride, ssm_pool, ssm_block_stride, num_blocks, out,
                      workspace, workspace_bytes, stream, false);
}

namespace {

// Scratch of the allocation-free entry point: one static device buffer, which
// every device the library runs on holds (at its own address) until the
// process ends.  In host code `scratch` only names the symbol; its device
// address on each device comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is ever passed on.
static __device__ __align__(256) unsigned char scratch[GDN_STATIC_SCRATCH_BYTES];

hipError_t scratch_address(hipStream_t st, void** ptr) {
  static std::mutex mu;
  static std::vector<void*> addr;
  int dev = 0;
  hipError_t e = hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int gdn_varlen_forward_noalloc(const gdn_layer_desc* desc, const void* x, const void* conv_weight,
                                          const float* g, const float* beta, const int32_t* cu_seqlens,
                                          const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t total_tokens,
                                          const int32_t* read_idx, const int32_t* write_idx, void* conv_pool,
                                          int64_t conv_block_stride, float* ssm_pool, int64_t ssm_block_stride,
                                          int32_t num_blocks, void* out, void* stream) {
  return forward_impl(desc, x, conv_weight, g, beta, cu_seqlens, cu_seqlens_host, num_seqs, total_tokens, read_idx,
                      write_idx, conv_pool, conv_block_stride, ssm_pool, ssm_block_stride, num_blocks, out, nullptr,
                      GDN_STATIC_SCRATCH_BYTES, stream, true);
}

namespace {
int forward_impl(const gdn_layer_desc* desc, const void* x, const void* conv_weight, const float* g,
                 const float* beta, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t num_seqs,
                 int32_t total_tokens, const int32_t* read_idx, const int32_t* write_idx, void* conv_pool,
                 int64_t conv_block_stride, float* ssm_pool, int64_t ssm_block_stride, int32_t num_blocks,
                 void* out, void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
  int rc = check_desc(desc);
  if (rc) return rc;
  const int W = desc->conv_width;
  const bool bf16 = desc->act_dtype == GDN_BF16;

  // ---- host-side checks; nothing below reads device memory
  if (num_seqs < 1) return fail(GDN_EINVAL, "no sequences in batch (num_seqs=%d)", num_seqs);
  if (total_tokens < 0) return fail(GDN_EINVAL, "total_tokens=%d is negative", total_tokens);
  const bool dev_plan = cu_seqlens_host == nullptr;  // plan on the device (graph capture)
  if (dev_plan) {
    if (num_seqs > gdn::kMaxPlanSeqs)
      return fail(GDN_EUNSUPPORTED, "planning on the device takes at most %d sequences (num_seqs=%d)",
                  gdn::kMaxPlanSeqs, num_seqs);
  } else {
    if (cu_seqlens_host[0] != 0) return fail(GDN_EINVAL, "cu_seqlens[0]=%d, expected 0", cu_seqlens_host[0]);
    for (int i = 0; i < num_seqs; ++i)
      if (cu_seqlens_host[i + 1] < cu_seqlens_host[i])
        return fail(GDN_EINVAL, "cu_seqlens decreases at %d (%d -> %d)", i, cu_seqlens_host[i],
                    cu_seqlens_host[i + 1]);
    if (cu_seqlens_host[num_seqs] != total_tokens)
      return fail(GDN_EINVAL, "cu_seqlens[%d]=%d differs from total_tokens=%d", num_seqs,
                  cu_seqlens_host[num_seqs], total_tokens);
  }
  if (!cu_seqlens || !read_idx || !write_idx) return fail(GDN_EINVAL, "device cu_seqlens/read_idx/write_idx is NULL");
  if (!ssm_pool) return fail(GDN_EINVAL, "ssm_pool is NULL");
  if (W > 1 && !conv_pool) return fail(GDN_EINVAL, "conv_pool is NULL but conv_width=%d > 1", W);
  if (total_tokens > 0 && (!x || !g || !beta || !out))
    return fail(GDN_EINVAL, "x, g, beta and out must be non-NULL when total_tokens > 0");
  if (!conv_weight && total_tokens > 0) return fail(GDN_EINVAL, "conv_weight is NULL");
  if (num_blocks < 2) return fail(GDN_EINVAL, "num_blocks=%d; the pool needs the trash block and one more", num_blocks);
  if (ssm_block_stride < ssm_state_bytes(desc) || ssm_block_stride % 16)
    return fail(GDN_EINVAL, "ssm_block_stride=%lld must be a multiple of 16 and >= %lld", (long long)ssm_block_stride,
                (long long)ssm_state_bytes(desc));
  if (W > 1 && (conv_block_stride < conv_state_bytes(desc) || conv_block_stride % 16))
    return fail(GDN_EINVAL, "conv_block_stride=%lld must be a multiple of 16 and >= %lld",
                (long long)conv_block_stride, (long long)conv_state_bytes(desc));
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ssm_pool, 16) || !aligned(conv_pool, 16) ||
      !aligned(g, 4) || !aligned(beta, 4))
    return fail(GDN_EINVAL, "x, out and the pools must be 16-byte aligned");
  const WsLayout wl = ws_layout(desc, total_tokens, num_seqs);
  const size_t need = wl.total;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (noalloc) {
    if (need > workspace_bytes)
      return fail(GDN_EWORKSPACE,
                  "the batch needs %zu bytes of scratch, more than the %zu of the static buffer "
                  "(gdn_varlen_forward_noalloc); call gdn_varlen_forward with a workspace instead",
                  need, workspace_bytes);
    const hipError_t e = scratch_address(st, &workspace);
    if (e != hipSuccess) return fail(GDN_EHIP, "static scratch buffer: %s", hipGetErrorString(e));
  }
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(GDN_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  if (workspace && !aligned(workspace, 256)) return fail(GDN_EINVAL, "workspace must be 256-byte aligned");

  const int C = (int)channels(desc);
  hipError_t e = hipSuccess;

  gdn::ScanArgs sa{};
  sa.y = workspace; sa.x = x; sa.w = conv_weight;
  sa.conv_pool = W > 1 ? reinterpret_cast<const char*>(conv_pool) : nullptr;
  sa.conv_stride = conv_block_stride; sa.width = W; sa.eps = desc->l2norm_eps;
  sa.q_scale = desc->q_scale > 0.f ? desc->q_scale : 1.0f / sqrtf((float)desc->head_k_dim);
  sa.g = g; sa.beta = beta; sa.cu = cu_seqlens; sa.read_idx = read_idx;
  sa.write_idx = write_idx; sa.ssm_pool = ssm_pool; sa.ssm_stride = ssm_block_stride; sa.out = out;
  sa.num_seqs = num_seqs; sa.num_blocks = num_blocks; sa.num_k_heads = desc->num_k_heads;
  sa.num_v_heads = desc->num_v_heads; sa.channels = C;
  const bool chunked = bf16 && gdn::chunk_supported(desc->head_k_dim, desc->head_v_dim);
  // every other head size, and the fp32 layer: the fp32 chunk kernel
  const bool generic = !chunked && gdn::chunk_generic_supported(desc->head_k_dim, desc->head_v_dim);

  gdn::TailArgs ta{};
  ta.x = x; ta.cu = cu_seqlens; ta.read_idx = read_idx; ta.write_idx = write_idx;
  ta.conv_pool = reinterpret_cast<char*>(conv_pool); ta.conv_stride = conv_block_stride;
  ta.num_seqs = num_seqs; ta.num_blocks = num_blocks; ta.channels = C;
  ta.max_len = INT_MAX;

  gdn::ConvArgs ca{};
  ca.x = x; ca.w = conv_weight; ca.cu = cu_seqlens; ca.read_idx = read_idx; ca.write_idx = write_idx;
  ca.conv_pool = reinterpret_cast<const char*>(conv_pool); ca.conv_stride = conv_block_stride;
  ca.y = workspace;
  ca.num_seqs = num_seqs; ca.total_tokens = total_tokens; ca.num_blocks = num_blocks; ca.channels = C;
  ca.qk_channels = desc->num_k_heads * desc->head_k_dim; ca.head_k_dim = desc->head_k_dim;
  {  // about 4096 one-wave blocks (16 per CU): rows per block a multiple of the 4 rows in flight
    const int groups = (C + 511) / 512;
    const int slices = std::max(1, 4096 / groups);
    const int rows = (total_tokens + slices - 1) / slices;
    ca.rows_per_block = std::min(256, std::max(4, (rows + 3) / 4 * 4));
  }
  ca.eps = sa.eps;
  ca.q_scale = sa.q_scale;

  // ---- plan on the device: every launch size depends on num_seqs and
  // total_tokens only, so a captured graph replays for any offsets and indices
  if (dev_plan) {
    // the token path (which skips the chunked sequences itself) on the side
    // stream beside the chunked path; captured graphs keep the fork
    const bool fork = !noalloc && chunked && total_tokens > 0;
    hipStream_t side = nullptr;
    if (fork) {
      e = fork_side(st, &side);
      if (e != hipSuccess) return fail(GDN_EHIP, "side stream: %s", hipGetErrorString(e));
      gdn::ScanArgs ts = sa;
      ts.min_len = 0; ts.max_len = 1;
      e = timed(K_TOKEN, side, [&] { return gdn::launch_recurrent(ts, desc->head_k_dim, desc->head_v_dim, bf16, side); });
      if (e != hipSuccess) return fail(GDN_EHIP, "token path launch: %s", hipGetErrorString(e));
    }
    if (chunked && total_tokens > 0) {
      int32_t* plan = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + wl.plan);
      int32_t* sync = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + wl.sync);
      const int mode = conv_in_scan_mode();
      gdn::PlanArgs pa{};
      pa.cu = cu_seqlens; pa.num_seqs = num_seqs; pa.num_v_heads = desc->num_v_heads;
      pa.slices = (C + gdn::kConvTaskChannels - 1) / gdn::kConvTaskChannels; pa.conv_rows = gdn::kConvTaskRows;
      pa.fused_allowed = mode >= 0 && aligned(conv_weight, 16) &&
                         (int64_t)num_seqs * desc->num_v_heads <= device_cus(st);
      pa.fused_forced = mode > 0;
      pa.conv_us_per_token = 2.0 * C * act_size(desc) / kConvBytesPerUs;
      pa.task_us = task_us(C, desc);
      pa.scan0_us = kScan0Us; pa.scan1_us = kScan1Us; pa.margin = kTargetMargin * 100.0;
      pa.cus = device_cus(st); pa.plain_scan1_us = kScanPlainUs; pa.crowd_scan1_us = kScanCrowdUs;
      pa.phased_scale = kPhasedScale;
      pa.beside_tokens = fork;
      pa.plan = plan; pa.sync = sync;
      e = timed(K_PLAN, st, [&] { return gdn::launch_plan(pa, st); });
      if (e != hipSuccess) return fail(GDN_EHIP, "plan launch: %s", hipGetErrorString(e));
      ca.skip = plan + gdn::kPlanFused;
      e = timed(K_CONV, st, [&] { return gdn::launch_conv(ca, W, bf16, true, st); });
      if (e != hipSuccess) return fail(GDN_EHIP, "conv launch: %s", hipGetErrorString(e));
      static thread_local gdn::SeqOrder none;
      none.n = 0;
      static thread_local gdn::FusedConv fc;
      fc.n = 0; fc.slices = pa.slices; fc.sync = sync; fc.own_first = 1;
      fc.target = 0; fc.task = (int32_t)(pa.task_us * 100.0);
      fc.scan0 = (int32_t)(kScan0Us * 100.0); fc.scan1 = (int32_t)(kScan1Us * 100.0);
      fc.plan = plan; fc.plan_seqs = num_seqs;
      sa.min_len = 2; sa.max_len = INT_MAX;
      e = timed(K_CHUNK, st, [&] { return gdn::launch_chunk(sa, none, fc, desc->head_k_dim, desc->head_v_dim, st); });
      if (e != hipSuccess) return fail(GDN_EHIP, "chunk scan launch: %s", hipGetErrorString(e));
      ta.fused = plan + gdn::kPlanFused;
    } else if (generic && total_tokens > 0) {
      e = timed(K_CONV, st, [&] { return gdn::launch_conv(ca, W, bf16, true, st); });
      if (e != hipSuccess) return fail(GDN_EHIP, "conv launch: %s", hipGetErrorString(e));
      static thread_local gdn::SeqOrder none_g;
      none_g.n = 0;
      sa.min_len = 2; sa.max_len = INT_MAX;
      e = timed(K_CHUNK_GEN, st, [&] {
        return gdn::launch_chunk_generic(sa, none_g, desc->head_k_dim, desc->head_v_dim, bf16, st);
      });
      if (e != hipSuccess) return fail(GDN_EHIP, "chunk scan launch: %s", hipGetErrorString(e));
    }
    if (fork) {
      e = join_side(st, side);
      if (e != hipSuccess) return fail(GDN_EHIP, "side stream: %s", hipGetErrorString(e));
    } else {
      sa.min_len = 0; sa.max_len = (chunked || generic) ? 1 : INT_MAX;
      e = timed(K_TOKEN, st, [&] { return gdn::launch_recurrent(sa, desc->head_k_dim, desc->head_v_dim, bf16, st); });
      if (e != hipSuccess) return fail(GDN_EHIP, "token path launch: %s", hipGetErrorString(e));
    }
    if (W > 1) {
      e = timed(K_TAIL, st, [&] { return gdn::launch_tail_commit(ta, W, bf16, st); });
      if (e != hipSuccess) return fail(GDN_EHIP, "conv state commit launch: %s", hipGetErrorString(e));
    }
    return GDN_OK;
  }

  // ---- plan from the host offsets
  int n_long = 0, n_short = 0;
  for (int i = 0; i < num_seqs; ++i) {
    const int L = cu_seqlens_host[i + 1] - cu_seqlens_host[i];
    if (L >= 2) ++n_long; else ++n_short;
  }

  // Order on the stream: (1) conv + SiLU + norm of the packed row into the
  // workspace for the chunked prefill (its own kernel, or inside the chunk
  // kernel ahead of the scans), (2) chunked prefill, (3) the token path
  // (decode, or everything in fp32 / other head sizes), which runs its own conv
  // from the conv states, (4) conv-state commit, last, once every reader of the
  // old conv states has been enqueued (when the chunk kernel ran the conv, it
  // also wrote the chunked sequences' states, and this covers the rest).
  bool tails_done = false;  // the chunk kernel has written the chunked sequences' conv states
  // a mixed batch: the token path on the side stream, beside the chunked path
  // (not for the allocation-free entry point, which creates nothing).  The
  // chunk kernel is enqueued first: each of its workgroups needs a whole CU,
  // and token workgroups already spread over every CU would hold it back
  // (measured: its kernel 0.105 -> 0.072 ms on 64 decode tokens beside
  // 4 x 512 prefill tokens).  With the conv kernel first, the token path does
  // not wait for it (it runs its own conv) and starts at once as before.
  const bool fork = !noalloc && chunked && n_long > 0 && n_short > 0;
  hipStream_t side = nullptr;
  gdn::ScanArgs ts = sa;
  ts.min_len = 0; ts.max_len = 1;
  // the side stream starts from the work enqueued so far (the fork), and the
  // token kernel goes on it once the chunk kernel is enqueued after the fork
  auto fork_here = [&]() -> int {
    const hipError_t fe = fork_side(st, &side);
    return fe == hipSuccess ? GDN_OK : fail(GDN_EHIP, "side stream: %s", hipGetErrorString(fe));
  };
  auto launch_side = [&]() -> int {
    const hipError_t fe =
        timed(K_TOKEN, side, [&] { return gdn::launch_recurrent(ts, desc->head_k_dim, desc->head_v_dim, bf16, side); });
    return fe == hipSuccess ? GDN_OK : fail(GDN_EHIP, "token path launch: %s", hipGetErrorString(fe));
  };
  if (chunked && n_long > 0) {
    sa.min_len = 2; sa.max_len = INT_MAX;
    // longest sequences first, so the longest chains start before the short ones
    static thread_local gdn::SeqOrder order;
    order.n = 0;
    if (n_long <= gdn::kMaxOrder && num_seqs <= 65535) {
      std::vector<std::pair<int, int>> lens;
      lens.reserve(n_long);
      for (int i = 0; i < num_seqs; ++i) {
        const int L = cu_seqlens_host[i + 1] - cu_seqlens_host[i];
        if (L >= 2) lens.push_back({-L, i});
      }
      std::stable_sort(lens.begin(), lens.end());
      for (size_t i = 0; i < lens.size(); ++i) order.seq[i] = (uint16_t)lens[i].second;
      order.n = (int32_t)lens.size();
    }
    // The conv of the chunked rows runs inside the scan kernel when every
    // workgroup of the scan is resident at once (one per CU): the workgroups
    // convert rows, longest sequence first, until their own sequence's rows are
    // all taken, and start their scans while the others go on converting.
    // Otherwise the conv kernel writes all of y first.
    static thread_local gdn::FusedConv fc;
    fc.n = 0;
    fc.plan = nullptr;
    fc.plan_seqs = 0;
    fc.stream = 0;
    fc.helpers = 0;
    fc.own_first = 1;  // a scan of 2.8 us per chunk would catch up with rows converted by others
    const int mode = conv_in_scan_mode();
    const int cus = device_cus(st);
    if (mode >= 0 && order.n > 0 && order.n <= gdn::kMaxFusedRanks && aligned(conv_weight, 16) &&
        (int64_t)order.n * desc->num_v_heads <= cus) {
      fc.slices = (C + gdn::kConvTaskChannels - 1) / gdn::kConvTaskChannels;
      fc.first[0] = 0;
      const double scan0 = kScan0Us, scan1 = kScan1Us;
      const double task_us = ::task_us(C, desc);
      double scans = 0.0;
      for (int r = 0; r < order.n; ++r) {
        const int L = cu_seqlens_host[order.seq[r] + 1] - cu_seqlens_host[order.seq[r]];
        fc.first[r + 1] = fc.first[r] + (L + gdn::kConvTaskRows - 1) / gdn::kConvTaskRows * fc.slices;
        scans += scan0 + scan1 * ((L + 63) / 64);
      }
      const int L0 = cu_seqlens_host[order.seq[0] + 1] - cu_seqlens_host[order.seq[0]];
      const int chunks0 = (L0 + 63) / 64;
      const double longest = scan0 + scan1 * chunks0;
      // work spread evenly over the workgroups, but no earlier than the longest scan allows
      const double fused = std::max((fc.first[order.n] * task_us + desc->num_v_heads * scans) /
                                    ((double)order.n * desc->num_v_heads), longest + 2.0 * task_us);
      const int64_t wgs = (int64_t)order.n * desc->num_v_heads;
      const double apart = 2.0 * (double)total_tokens * C * act_size(desc) / kConvBytesPerUs + scan0 +
                           plain_scan1(wgs, cus) * chunks0 + 3.0;
      // streaming: spare CUs run helper workgroups that convert rows just
      // ahead of the scans, which all start at once; it ends when both the
      // longest scan and the helpers' share of the conv are done
      const int helpers = (cus - (int)wgs) / 8 * 8;  // a multiple of the 8 XCDs
      const bool stream_ok = helpers >= 32 && mode != 1;
      const double helper_task_us = task_us * kTaskBytesPerUs / kHelperBytesPerUs;
      const double streamed = std::max(kStreamScanScale * (scan0 + kScanPlainUs * chunks0) + kStreamStartUs,
                                       fc.first[order.n] * helper_task_us / std::max(helpers, 1) + 25.0);
      const double phased = kPhasedScale * fused;
      // With one-token sequences in the batch the token kernel runs beside
      // this path on the side stream, and a separate conv kernel would share
      // the HBM and the CUs with it: the conv then runs inside the chunk
      // kernel (measured on 64 decode tokens beside 4 x 512 prefill tokens:
      // 0.093 against 0.114 ms per step).
      const bool use_stream =
          stream_ok && (mode == 2 || (mode == 0 && !fork && streamed < std::min(phased, apart)));
      const bool use_phased = !use_stream && (mode == 1 || (mode == 0 && (fork || phased < apart)));
      if (use_stream || use_phased) {
        fc.n = order.n;
        fc.sync = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + wl.sync);
        fc.target = (int32_t)(fused * kTargetMargin * 100.0);  // 100 ticks per microsecond
        fc.task = (int32_t)(task_us * 100.0);
        fc.scan0 = (int32_t)(scan0 * 100.0);
        fc.scan1 = (int32_t)(scan1 * 100.0);
      }
      if (use_phased && fc.n > 0) {
        // own tasks: sequence r scans once the tasks up to its own are claimed,
        // at the rate of every workgroup converting; by budget: the target
        // below.  A task of a narrower layer is priced in proportion.
        const double task_cal =
            kCalTaskUs * task_us / (2.0 * gdn::kConvTaskRows * gdn::kConvTaskChannels * 2.0 / kTaskBytesPerUs);
        const double rate = (double)wgs / task_cal;
        double own_end = 0.0, scans_cal = 0.0;
        for (int r = 0; r < order.n; ++r) {
          const int n_r = (fc.first[r + 1] - fc.first[r]) / fc.slices;
          own_end = std::max(own_end, fc.first[r + 1] / rate + kCalScan0Us + kCalScan1Us * n_r);
          scans_cal += kCalScan0Us + kCalScan1Us * n_r;
        }
        const double even = (fc.first[order.n] * task_cal + desc->num_v_heads * scans_cal) / (double)wgs;
        const double budget_end = std::max(even, kCalScan0Us + kCalScan1Us * chunks0 + 2.0 * task_cal) +
                                  kBudgetSlackTasks * task_cal;
        const int claim = conv_claim_mode();
        if (claim == 2 || (claim == 0 && own_end >= budget_end)) {
          fc.own_first = 0;
          fc.target = (int32_t)(budget_end * 100.0);
          fc.task = (int32_t)(task_cal * 100.0);
          fc.scan0 = (int32_t)(kCalScan0Us * 100.0);
          fc.scan1 = (int32_t)(kCalScan1Us * 100.0);
        }
      }
      if (use_stream) {  // first[r]: the first chunk counter of rank r
        fc.stream = 1;
        fc.helpers = helpers;
        fc.first[0] = 0;
        for (int r = 0; r < order.n; ++r) {
          const int L = cu_seqlens_host[order.seq[r] + 1] - cu_seqlens_host[order.seq[r]];
          fc.first[r + 1] = fc.first[r] + (L + 63) / 64;
        }
      }
    }
    if (fc.n == 0) {
      if (fork && ((rc = fork_here()) != GDN_OK || (rc = launch_side()) != GDN_OK)) return rc;
      e = timed(K_CONV, st, [&] { return gdn::launch_conv(ca, W, bf16, true, st); });
      if (e != hipSuccess) return fail(GDN_EHIP, "conv launch: %s", hipGetErrorString(e));
    } else {
      // streaming: the task counter, the chunk counters and the role ticket;
      // phased: the task counter, one per rank and one per chunk of each rank
      const int counters = fc.stream ? 2 + fc.first[fc.n] : 1 + fc.n + fc.first[fc.n] / fc.slices;
      e = timed(K_ZERO, st, [&] { return gdn::launch_zero_sync(fc.sync, counters, st); });
      if (e != hipSuccess) return fail(GDN_EHIP, "counter reset launch: %s", hipGetErrorString(e));
      if (fork && (rc = fork_here()) != GDN_OK) return rc;
    }
    e = timed(K_CHUNK, st, [&] { return gdn::launch_chunk(sa, order, fc, desc->head_k_dim, desc->head_v_dim, st); });
    if (e != hipSuccess) return fail(GDN_EHIP, "chunk scan launch: %s", hipGetErrorString(e));
    if (fork && fc.n > 0 && (rc = launch_side()) != GDN_OK) return rc;
    tails_done = fc.n > 0;
  }
  if (generic && n_long > 0) {
    // conv kernel first (the fp32 kernel reads y), longest sequences first
    e = timed(K_CONV, st, [&] { return gdn::launch_conv(ca, W, bf16, true, st); });
    if (e != hipSuccess) return fail(GDN_EHIP, "conv launch: %s", hipGetErrorString(e));
    static thread_local gdn::SeqOrder order_g;
    order_g.n = 0;
    if (n_long <= gdn::kMaxOrder && num_seqs <= 65535) {
      std::vector<std::pair<int, int>> lens;
      lens.reserve(n_long);
      for (int i = 0; i < num_seqs; ++i) {
        const int L = cu_seqlens_host[i + 1] - cu_seqlens_host[i];
        if (L >= 2) lens.push_back({-L, i});
      }
      std::stable_sort(lens.begin(), lens.end());
      for (size_t i = 0; i < lens.size(); ++i) order_g.seq[i] = (uint16_t)lens[i].second;
      order_g.n = (int32_t)lens.size();
    }
    sa.min_len = 2; sa.max_len = INT_MAX;
    e = timed(K_CHUNK_GEN, st, [&] {
      return gdn::launch_chunk_generic(sa, order_g, desc->head_k_dim, desc->head_v_dim, bf16, st);
    });
    if (e != hipSuccess) return fail(GDN_EHIP, "chunk scan launch: %s", hipGetErrorString(e));
  }
  const bool any_chunk = (chunked || generic) && n_long > 0;
  if (fork) {
    e = join_side(st, side);
    if (e != hipSuccess) return fail(GDN_EHIP, "side stream: %s", hipGetErrorString(e));
  } else if (!any_chunk || n_short > 0) {
    sa.min_len = 0; sa.max_len = any_chunk ? 1 : INT_MAX;
    e = timed(K_TOKEN, st, [&] { return gdn::launch_recurrent(sa, desc->head_k_dim, desc->head_v_dim, bf16, st); });
    if (e != hipSuccess) return fail(GDN_EHIP, "token path launch: %s", hipGetErrorString(e));
  }
  if (W > 1 && (!tails_done || n_short > 0)) {
    ta.max_len = tails_done ? 1 : INT_MAX;
    e = timed(K_TAIL, st, [&] { return gdn::launch_tail_commit(ta, W, bf16, st); });
    if (e != hipSuccess) return fail(GDN_EHIP, "conv state commit launch: %s", hipGetErrorString(e));
  }
  return GDN_OK;
}
}  // namespace

extern "C" int gdn_varlen_conv(int32_t channels, int32_t conv_width, int32_t act_dtype, int32_t silu,
                               const void* x, const void* conv_weight, const int32_t* cu_seqlens,
                               const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t total_tokens,
                               const int32_t* read_idx, const int32_t* write_idx, void* conv_pool,
                               int64_t conv_block_stride, int32_t num_blocks, void* y, void* stream) {
  if (act_dtype != GDN_F32 && act_dtype != GDN_BF16)
    return fail(GDN_EINVAL, "act_dtype %d is neither GDN_F32 nor GDN_BF16", act_dtype);
  if (channels < 1 || conv_width < 1) return fail(GDN_EINVAL, "channels and conv_width must be >= 1");
  if (channels % 8) return fail(GDN_EUNSUPPORTED, "channels=%d is not a multiple of 8", channels);
  if (channels > INT_MAX / 8) return fail(GDN_EUNSUPPORTED, "too many channels (%d)", channels);
  if (conv_width > 4) return fail(GDN_EUNSUPPORTED, "conv_width %d > 4 is not built", conv_width);
  const int W = conv_width;
  const bool bf16 = act_dtype == GDN_BF16;
  const int64_t esz = bf16 ? 2 : 4;
  if (num_seqs < 1) return fail(GDN_EINVAL, "no sequences in batch (num_seqs=%d)", num_seqs);
  if (total_tokens < 0) return fail(GDN_EINVAL, "total_tokens=%d is negative", total_tokens);
  if (!cu_seqlens_host) return fail(GDN_EINVAL, "cu_seqlens_host is NULL");
  if (cu_seqlens_host[0] != 0) return fail(GDN_EINVAL, "cu_seqlens[0]=%d, expected 0", cu_seqlens_host[0]);
  for (int i = 0; i < num_seqs; ++i)
    if (cu_seqlens_host[i + 1] < cu_seqlens_host[i])
      return fail(GDN_EINVAL, "cu_seqlens decreases at %d (%d -> %d)", i, cu_seqlens_host[i], cu_seqlens_host[i + 1]);
  if (cu_seqlens_host[num_seqs] != total_tokens)
    return fail(GDN_EINVAL, "cu_seqlens[%d]=%d differs from total_tokens=%d", num_seqs, cu_seqlens_host[num_seqs],
                total_tokens);
  if (!cu_seqlens || !read_idx || !write_idx) return fail(GDN_EINVAL, "device cu_seqlens/read_idx/write_idx is NULL");
  if (W > 1 && !conv_pool) return fail(GDN_EINVAL, "conv_pool is NULL but conv_width=%d > 1", W);
  if (total_tokens > 0 && (!x || !conv_weight || !y)) return fail(GDN_EINVAL, "x, conv_weight and y must be non-NULL");
  if (num_blocks < 2) return fail(GDN_EINVAL, "num_blocks=%d; the pool needs the trash block and one more", num_blocks);
  if (W > 1 && (conv_block_stride < (W - 1) * (int64_t)channels * esz || conv_block_stride % 16))
    return fail(GDN_EINVAL, "conv_block_stride=%lld must be a multiple of 16 and >= %lld", (long long)conv_block_stride,
                (long long)((W - 1) * (int64_t)channels * esz));
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(conv_pool, 16))
    return fail(GDN_EINVAL, "x, y and conv_pool must be 16-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (total_tokens > 0) {
    gdn::ConvArgs ca{};
    ca.x = x; ca.w = conv_weight; ca.cu = cu_seqlens; ca.read_idx = read_idx; ca.write_idx = write_idx;
    ca.conv_pool = reinterpret_cast<const char*>(conv_pool); ca.conv_stride = conv_block_stride;
    ca.y = y;
    ca.num_seqs = num_seqs; ca.total_tokens = total_tokens; ca.num_blocks = num_blocks; ca.channels = channels;
    ca.qk_channels = 0;   // no normalisation
    ca.head_k_dim = 128;  // lanes of the (unused) head sums
    ca.eps = 0.f;
    ca.q_scale = 1.f;
    const int groups = (channels + 511) / 512;
    const int slices = std::max(1, 4096 / groups);
    const int rows = (total_tokens + slices - 1) / slices;
    ca.rows_per_block = std::min(256, std::max(4, (rows + 3) / 4 * 4));
    e = timed(K_CONV, st, [&] { return gdn::launch_conv(ca, W, bf16, silu != 0, st); });
    if (e != hipSuccess) return fail(GDN_EHIP, "conv launch: %s", hipGetErrorString(e));
  }
  if (W > 1) {
    gdn::TailArgs ta{};
    ta.x = x; ta.cu = cu_seqlens; ta.read_idx = read_idx; ta.write_idx = write_idx;
    ta.conv_pool = reinterpret_cast<char*>(conv_pool); ta.conv_stride = conv_block_stride;
    ta.num_seqs = num_seqs; ta.num_blocks = num_blocks; ta.channels = channels;
    ta.max_len = INT_MAX;
    e = timed(K_TAIL, st, [&] { return gdn::launch_tail_commit(ta, W, bf16, st); });
    if (e != hipSuccess) return fail(GDN_EHIP, "conv state commit launch: %s", hipGetErrorString(e));
  }
  return GDN_OK;
}

extern "C" int gdn_state_copy(const gdn_layer_desc* desc, void* conv_pool, int64_t conv_block_stride,
                              float* ssm_pool, int64_t ssm_block_stride, int32_t num_blocks, const int32_t* src,
                              const int32_t* dst, int32_t n, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  const int W = desc->conv_width;
  if (n < 0) return fail(GDN_EINVAL, "n=%d is negative", n);
  if (n == 0) return GDN_OK;
  if (!src || !dst) return fail(GDN_EINVAL, "src or dst is NULL");
  if (!ssm_pool) return fail(GDN_EINVAL, "ssm_pool is NULL");
  if (W > 1 && !conv_pool) return fail(GDN_EINVAL, "conv_pool is NULL but conv_width=%d > 1", W);
  if (num_blocks < 1) return fail(GDN_EINVAL, "num_blocks=%d", num_blocks);
  if (ssm_block_stride < ssm_state_bytes(desc) || ssm_block_stride % 16)
    return fail(GDN_EINVAL, "ssm_block_stride=%lld must be a multiple of 16 and >= %lld", (long long)ssm_block_stride,
                (long long)ssm_state_bytes(desc));
  if (W > 1 && (conv_block_stride < conv_state_bytes(desc) || conv_block_stride % 16))
    return fail(GDN_EINVAL, "conv_block_stride=%lld must be a multiple of 16 and >= %lld",
                (long long)conv_block_stride, (long long)conv_state_bytes(desc));
  if (!aligned(ssm_pool, 16) || !aligned(conv_pool, 16)) return fail(GDN_EINVAL, "the pools must be 16-byte aligned");
  gdn::StateCopyArgs ca{};
  ca.ssm_pool = reinterpret_cast<char*>(ssm_pool);
  ca.conv_pool = reinterpret_cast<char*>(conv_pool);
  ca.ssm_stride = ssm_block_stride;
  ca.conv_stride = conv_block_stride;
  ca.ssm_bytes = ssm_state_bytes(desc);
  ca.conv_bytes = W > 1 ? conv_state_bytes(desc) : 0;
  ca.src = src;
  ca.dst = dst;
  ca.num_blocks = num_blocks;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = timed(K_COPY, st, [&] { return gdn::launch_state_copy(ca, n, st); });
  if (e != hipSuccess) return fail(GDN_EHIP, "state copy launch: %s", hipGetErrorString(e));
  return GDN_OK;
}

extern "C" int ssd_varlen_scan(const ssd_layer_desc* desc, const void* x, int64_t x_row_stride, const void* B,
                               const void* C, int64_t bc_row_stride, const float* dt, const float* dt_bias,
                               const float* A, const float* D, const int32_t* cu_seqlens,
                               const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t total_tokens,
                               const int32_t* read_idx, const int32_t* write_idx, float* ssm_pool,
                               int64_t ssm_block_stride, int32_t num_blocks, void* y, void* stream) {
  if (!desc) return fail(GDN_EINVAL, "layer descriptor is NULL");
  const int H = desc->num_heads, P = desc->head_dim, G = desc->num_groups, N = desc->state_dim;
  if (H < 1 || G < 1 || P < 1 || N < 1) return fail(GDN_EINVAL, "H=%d, P=%d, G=%d, N=%d must be >= 1", H, P, G, N);
  if (H % G) return fail(GDN_EINVAL, "H=%d is not a multiple of G=%d", H, G);
  if (!gdn::ssd_supported(P, N))
    return fail(GDN_EUNSUPPORTED, "head_dim=%d, state_dim=%d: this build runs head_dim 64 with state_dim 128", P, N);
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_EINVAL, "num_seqs=%d, total_tokens=%d", num_seqs, total_tokens);
  if (num_seqs == 0) return GDN_OK;
  if (!cu_seqlens || !read_idx || !write_idx || !A || !ssm_pool) return fail(GDN_EINVAL, "a required pointer is NULL");
  if (total_tokens > 0 && (!x || !B || !C || !dt || !y)) return fail(GDN_EINVAL, "x, B, C, dt or y is NULL");
  if (num_blocks < 1) return fail(GDN_EINVAL, "num_blocks=%d", num_blocks);
  const int64_t state_bytes = (int64_t)H * P * N * 4;
  if (ssm_block_stride < state_bytes || ssm_block_stride % 16)
    return fail(GDN_EINVAL, "ssm_block_stride=%lld must be a multiple of 16 and >= %lld", (long long)ssm_block_stride,
                (long long)state_bytes);
  if (x_row_stride < (int64_t)H * P || x_row_stride % 8 || bc_row_stride < (int64_t)G * N || bc_row_stride % 8)
    return fail(GDN_EINVAL, "row strides (x %lld, B/C %lld) must be multiples of 8 and cover a row",
                (long long)x_row_stride, (long long)bc_row_stride);
  // the kernel's buffer offsets are 32-bit: 64 rows of either stride must fit
  if (x_row_stride > (1LL << 23) || bc_row_stride > (1LL << 23))
    return fail(GDN_EUNSUPPORTED, "row strides above 2^23 elements");
  if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) || !aligned(ssm_pool, 16))
    return fail(GDN_EINVAL, "x, B, C, y and ssm_pool must be 16-byte aligned");
  // with the host offsets, a kernel with no sequence of its kind is not launched
  bool any_long = true, any_short = true;
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] != 0 || cu_seqlens_host[num_seqs] != total_tokens)
      return fail(GDN_EINVAL, "cu_seqlens must run from 0 to total_tokens=%d", total_tokens);
    any_long = any_short = false;
    for (int i = 0; i < num_seqs; ++i) {
      const int L = cu_seqlens_host[i + 1] - cu_seqlens_host[i];
      if (L < 0) return fail(GDN_EINVAL, "cu_seqlens decreases at %d", i);
      if (L >= 2) any_long = true; else any_short = true;
    }
  }
  gdn::SsdArgs a{};
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.b = reinterpret_cast<const uint16_t*>(B);
  a.c = reinterpret_cast<const uint16_t*>(C);
  a.x_stride = x_row_stride;
  a.bc_stride = bc_row_stride;
  a.dt = dt;
  a.dt_bias = dt_bias;
  a.A = A;
  a.D = D;
  a.cu = cu_seqlens;
  a.read_idx = read_idx;
  a.write_idx = write_idx;
  a.pool = ssm_pool;
  a.pool_stride = ssm_block_stride / 4;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.num_heads = H;
  a.num_groups = G;
  a.softplus = desc->dt_softplus != 0;
  a.total_tokens = total_tokens;
  a.y = reinterpret_cast<uint16_t*>(y);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // sequences of length >= 2 in chunks, those of length 0 and 1 in the token
  // kernel; they touch disjoint blocks, so the two launches need no order
  if (any_long) {
    // with the host offsets: the sequences of length >= 2 only, longest first
    // (a pair of heads fills a CU, so the grid runs in rounds; on 8 sequences
    // of 256-4096 tokens the longest chains otherwise started in the second)
    static thread_local gdn::SeqOrder order;
    order.n = 0;
    if (cu_seqlens_host && num_seqs <= gdn::kMaxOrder) {
      std::vector<std::pair<int, int>> lens;
      for (int i = 0; i < num_seqs; ++i) {
        const int L = cu_seqlens_host[i + 1] - cu_seqlens_host[i];
        if (L >= 2) lens.push_back({-L, i});
      }
      std::stable_sort(lens.begin(), lens.end());
      for (size_t i = 0; i < lens.size(); ++i) order.seq[i] = (uint16_t)lens[i].second;
      order.n = (int32_t)lens.size();
    }
    const hipError_t e = timed(K_SSD, st, [&] { return gdn::launch_ssd(a, order, st); });
    if (e != hipSuccess) return fail(GDN_EHIP, "ssd scan launch: %s", hipGetErrorString(e));
  }
  if (any_short) {
    const hipError_t e = timed(K_SSD_TOKEN, st, [&] { return gdn::launch_ssd_token(a, st); });
    if (e != hipSuccess) return fail(GDN_EHIP, "ssd token launch: %s", hipGetErrorString(e));
  }
  return GDN_OK;
}

extern "C" int kda_varlen_forward(const gdn_layer_desc* desc, const void* x, const void* conv_weight,
                                  const float* g, const float* beta, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t total_tokens,
                                  const int32_t* read_idx, const int32_t* write_idx, void* conv_pool,
                                  int64_t conv_block_stride, float* ssm_pool, int64_t ssm_block_stride,
                                  int32_t num_blocks, void* out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  const int W = desc->conv_width;
  const bool bf16 = desc->act_dtype == GDN_BF16;
  if (num_seqs < 1) return fail(GDN_EINVAL, "no sequences in batch (num_seqs=%d)", num_seqs);
  if (total_tokens < 0) return fail(GDN_EINVAL, "total_tokens=%d is negative", total_tokens);
  if (!cu_seqlens_host) return fail(GDN_EINVAL, "cu_seqlens_host is NULL");
  if (cu_seqlens_host[0] != 0) return fail(GDN_EINVAL, "cu_seqlens[0]=%d, expected 0", cu_seqlens_host[0]);
  for (int i = 0; i < num_seqs; ++i)
    if (cu_seqlens_host[i + 1] < cu_seqlens_host[i])
      return fail(GDN_EINVAL, "cu_seqlens decreases at %d (%d -> %d)", i, cu_seqlens_host[i], cu_seqlens_host[i + 1]);
  if (cu_seqlens_host[num_seqs] != total_tokens)
    return fail(GDN_EINVAL, "cu_seqlens[%d]=%d differs from total_tokens=%d", num_seqs, cu_seqlens_host[num_seqs],
                total_tokens);
  if (!cu_seqlens || !read_idx || !write_idx) return fail(GDN_EINVAL, "device cu_seqlens/read_idx/write_idx is NULL");
  if (!ssm_pool) return fail(GDN_EINVAL, "ssm_pool is NULL");
  if (W > 1 && !conv_pool) return fail(GDN_EINVAL, "conv_pool is NULL but conv_width=%d > 1", W);
  if (total_tokens > 0 && (!x || !g || !beta || !out || !conv_weight))
    return fail(GDN_EINVAL, "x, conv_weight, g, beta and out must be non-NULL when total_tokens > 0");
  if (num_blocks < 2) return fail(GDN_EINVAL, "num_blocks=%d; the pool needs the trash block and one more", num_blocks);
  if (ssm_block_stride < ssm_state_bytes(desc) || ssm_block_stride % 16)
    return fail(GDN_EINVAL, "ssm_block_stride=%lld must be a multiple of 16 and >= %lld", (long long)ssm_block_stride,
                (long long)ssm_state_bytes(desc));
  if (W > 1 && (conv_block_stride < conv_state_bytes(desc) || conv_block_stride % 16))
    return fail(GDN_EINVAL, "conv_block_stride=%lld must be a multiple of 16 and >= %lld",
                (long long)conv_block_stride, (long long)conv_state_bytes(desc));
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ssm_pool, 16) || !aligned(conv_pool, 16) ||
      !aligned(g, 4) || !aligned(beta, 4))
    return fail(GDN_EINVAL, "x, out and the pools must be 16-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int C = (int)channels(desc);
  gdn::ScanArgs sa{};
  sa.x = x; sa.w = conv_weight;
  sa.conv_pool = W > 1 ? reinterpret_cast<const char*>(conv_pool) : nullptr;
  sa.conv_stride = conv_block_stride; sa.width = W; sa.eps = desc->l2norm_eps;
  sa.q_scale = desc->q_scale > 0.f ? desc->q_scale : 1.0f / sqrtf((float)desc->head_k_dim);
  sa.g = g; sa.beta = beta; sa.cu = cu_seqlens; sa.read_idx = read_idx;
  sa.write_idx = write_idx; sa.ssm_pool = ssm_pool; sa.ssm_stride = ssm_block_stride; sa.out = out;
  sa.num_seqs = num_seqs; sa.num_blocks = num_blocks; sa.num_k_heads = desc->num_k_heads;
  sa.num_v_heads = desc->num_v_heads; sa.channels = C;
  sa.kda = 1;
  // Sequences of two or more tokens run chunked (bf16, d_k = d_v = 128, with a
  // workspace for the conv output): the normalised q, k and v rows are written
  // into the workspace, by the chunk kernel's own workgroups or by the conv
  // kernel before it, and the KDA chunk kernel walks each sequence 64 rows at
  // a time, longest first.  The others (and everything without a workspace or
  // in another shape) run token by token.  The new conv states come last, once
  // every reader of the old ones is enqueued.
  int n_long = 0;
  for (int i = 0; i < num_seqs; ++i) n_long += cu_seqlens_host[i + 1] - cu_seqlens_host[i] >= 2;
  const size_t y_bytes = (size_t)total_tokens * C * act_size(desc);
  const bool chunked = bf16 && n_long > 0 && workspace && gdn::kda_chunk_supported(desc->head_k_dim, desc->head_v_dim);
  if (chunked && workspace_bytes < y_bytes)
    return fail(GDN_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, y_bytes);
  if (workspace && !aligned(workspace, 256)) return fail(GDN_EINVAL, "workspace must be 256-byte aligned");
  hipError_t e = hipSuccess;
  if (chunked) {
    static thread_local gdn::SeqOrder order;
    order.n = 0;
    if (n_long <= gdn::kMaxOrder && num_seqs <= 65535) {
      std::vector<std::pair<int, int>> lens;
      for (int i = 0; i < num_seqs; ++i) {
        const int L = cu_seqlens_host[i + 1] - cu_seqlens_host[i];
        if (L >= 2) lens.push_back({-L, i});
      }
      std::stable_sort(lens.begin(), lens.end());
      for (size_t i = 0; i < lens.size(); ++i) order.seq[i] = (uint16_t)lens[i].second;
      order.n = (int32_t)lens.size();
    }
    // The conv of the chunked rows runs inside the KDA chunk kernel (phased, as
    // for the gated delta rule) when every workgroup of the kernel is resident
    // at once and the workspace holds the task counters; the workgroups of the
    // short sequences, whose scans end long before the longest one's, then
    // convert most of the rows.  Otherwise the conv kernel runs first.
    static thread_local gdn::FusedConv fc;
    fc.n = 0;
    fc.plan = nullptr;
    fc.plan_seqs = 0;
    fc.stream = 0;
    fc.helpers = 0;
    // A KDA scan takes 8.3 us per chunk, well behind the conversion of its rows
    // by the other workgroups: the tasks go chunk-major and each workgroup by
    // its time budget alone, so the long sequences start scanning after their
    // first chunks (0.556 -> 0.543 ms on the prefill workload)
    fc.own_first = 0;
    const WsLayout wl = ws_layout(desc, total_tokens, num_seqs);
    const int mode = conv_in_scan_mode();
    if (mode >= 0 && order.n > 0 && order.n <= gdn::kMaxFusedRanks && aligned(conv_weight, 16) &&
        workspace_bytes >= wl.plan && (int64_t)order.n * desc->num_v_heads <= device_cus(st)) {
      fc.slices = (C + gdn::kConvTaskChannels - 1) / gdn::kConvTaskChannels;
      fc.first[0] = 0;
      const double tus = ::task_us(C, desc);
      double scans = 0.0;
      for (int r = 0; r < order.n; ++r) {
        const int L = cu_seqlens_host[order.seq[r] + 1] - cu_seqlens_host[order.seq[r]];
        fc.first[r + 1] = fc.first[r] + (L + gdn::kConvTaskRows - 1) / gdn::kConvTaskRows * fc.slices;
        scans += kKdaScan0Us + kKdaScan1Us * ((L + 63) / 64);
      }
      const int L0 = cu_seqlens_host[order.seq[0] + 1] - cu_seqlens_host[order.seq[0]];
      const double longest = kKdaScan0Us + kKdaScan1Us * ((L0 + 63) / 64);
      const double fused = std::max((fc.first[order.n] * tus + desc->num_v_heads * scans) /
                                    ((double)order.n * desc->num_v_heads), longest + 2.0 * tus);
      const double apart = 2.0 * (double)total_tokens * C * act_size(desc) / kConvBytesPerUs + longest + 3.0;
      if (mode == 1 || mode == 2 || kPhasedScale * fused < apart) {
        fc.n = order.n;
        fc.sync = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + wl.sync);
        fc.target = (int32_t)(fused * kTargetMargin * 100.0);  // 100 ticks per microsecond
        fc.task = (int32_t)(tus * 100.0);
        fc.scan0 = (int32_t)(kKdaScan0Us * 100.0);
        fc.scan1 = (int32_t)(kKdaScan1Us * 100.0);
      }
    }
    if (fc.n > 0) {
      // the task counter, one per rank and one per chunk of each rank
      e = timed(K_ZERO, st, [&] { return gdn::launch_zero_sync(fc.sync, 1 + fc.n + fc.first[fc.n] / fc.slices, st); });
      if (e != hipSuccess) return fail(GDN_EHIP, "counter reset launch: %s", hipGetErrorString(e));
    } else {
      gdn::ConvArgs ca{};
      ca.x = x; ca.w = conv_weight; ca.cu = cu_seqlens; ca.read_idx = read_idx; ca.write_idx = write_idx;
      ca.conv_pool = reinterpret_cast<const char*>(conv_pool); ca.conv_stride = conv_block_stride;
      ca.y = workspace;
      ca.num_seqs = num_seqs; ca.total_tokens = total_tokens; ca.num_blocks = num_blocks; ca.channels = C;
      ca.qk_channels = desc->num_k_heads * desc->head_k_dim; ca.head_k_dim = desc->head_k_dim;
      const int groups = (C + 511) / 512;
      const int slices = std::max(1, 4096 / groups);
      const int rows = (total_tokens + slices - 1) / slices;
      ca.rows_per_block = std::min(256, std::max(4, (rows + 3) / 4 * 4));
      ca.eps = sa.eps;
      ca.q_scale = sa.q_scale;
      e = timed(K_CONV, st, [&] { return gdn::launch_conv(ca, W, bf16, true, st); });
      if (e != hipSuccess) return fail(GDN_EHIP, "conv launch: %s", hipGetErrorString(e));
    }
    gdn::ScanArgs ka = sa;
    ka.y = workspace;
    ka.min_len = 2; ka.max_len = INT_MAX;
    e = timed(K_KDA_CHUNK, st, [&] { return gdn::launch_kda_chunk(ka, order, fc, st); });
    if (e != hipSuccess) return fail(GDN_EHIP, "KDA chunk launch: %s", hipGetErrorString(e));
  }
  if (!chunked || n_long < num_seqs) {
    sa.min_len = 0; sa.max_len = chunked ? 1 : INT_MAX;
    e = timed(K_TOKEN, st, [&] { return gdn::launch_recurrent(sa, desc->head_k_dim, desc->head_v_dim, bf16, st); });
    if (e != hipSuccess) return fail(GDN_EHIP, "token path launch: %s", hipGetErrorString(e));
  }
  if (W > 1) {
    gdn::TailArgs ta{};
    ta.x = x; ta.cu = cu_seqlens; ta.read_idx = read_idx; ta.write_idx = write_idx;
    ta.conv_pool = reinterpret_cast<char*>(conv_pool); ta.conv_stride = conv_block_stride;
    ta.num_seqs = num_seqs; ta.num_blocks = num_blocks; ta.channels = C;
    ta.max_len = INT_MAX;
    e = timed(K_TAIL, st, [&] { return gdn::launch_tail_commit(ta, W, bf16, st); });
    if (e != hipSuccess) return fail(GDN_EHIP, "conv state commit launch: %s", hipGetErrorString(e));
  }
  return GDN_OK;
}
