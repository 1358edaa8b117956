/*
 * gdn.h -- C ABI of the MI355X (gfx950) library for the packed-batch (varlen)
 * forward of a gated-delta-net linear-attention layer under continuous batching.
 *
 * The operation (page "Continuous batching for linear attention layers", PR
 * description and the commit that adds the linear attention cache allocator):
 * many requests of different lengths are packed into one row of T tokens,
 * delimited by cu_seqlens.  Each request keeps a fixed-size state in one block
 * of a paged cache: the last W-1 inputs of its causal convolution ("conv"
 * state) and its recurrent state.  A request with no past reads the zeroed
 * trash block (block 0); every forward pass overwrites the request's own block
 * in place.  For every sequence the layer
 *   1. runs a depthwise causal conv1d of width W over the C = 2*H_k*d_k + H_v*d_v
 *      channels, continued from the conv state, followed by SiLU;
 *   2. splits the result into q (H_k heads of d_k), k (H_k heads of d_k) and
 *      v (H_v heads of d_v), in that channel order, L2-normalises q and k per
 *      head ( x / sqrt(sum x^2 + eps) ) and multiplies q by q_scale;
 *   3. runs the gated delta rule (Gated Delta Networks, Yang et al., ICLR 2025)
 *      for every value head m, reading key head m / (H_v / H_k):
 *         S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t,
 *      with a_t = exp(g_t), b_t = beta_t, S stored [d_k][d_v];
 *   4. writes o to out and the new conv state and recurrent state to the
 *      sequence's write block.
 *
 * All device work is enqueued on the caller's stream; no call synchronises
 * with the host, none allocates device memory, and host arrays passed in are
 * no longer needed when the call returns (so the warmup race that a commit on
 * the page fixes, inputs rewritten while a stream still read them, cannot arise
 * from this library).
 *
 * Errors: every function returns a gdn_status; gdn_last_error() gives a
 * readable message for the last non-OK status of the calling thread (the page's
 * allocator commit likewise refuses bad state declarations with a message).
 * Nothing aborts and no exception crosses this ABI.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_EINVAL = -1,        /* an argument is invalid (null, inconsistent, out of range) */
  GDN_EUNSUPPORTED = -2,  /* valid, but a shape or dtype this build does not run */
  GDN_EWORKSPACE = -3,    /* workspace missing or smaller than gdn_workspace_size() */
  GDN_EHIP = -4,          /* the HIP runtime reported an error (message has its text) */
  GDN_EDEVICE = -5        /* gdn_device_status only: a kernel raised a device-side status bit */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Shapes and numeric options of one layer; every shape is passed explicitly
 * (the page's allocator commit: shapes are declared by the layer, not read
 * from one model family's config). */
typedef struct {
  int32_t num_k_heads;  /* H_k >= 1 */
  int32_t num_v_heads;  /* H_v, a multiple of H_k */
  int32_t head_k_dim;   /* d_k in {16, 32, 64, 128} */
  int32_t head_v_dim;   /* d_v in {16, 32, 64, 128} */
  int32_t conv_width;   /* W in [1, 4] */
  int32_t act_dtype;    /* gdn_dtype of x, conv weight, conv pool and out; the
                           recurrent state, g and beta are always fp32 */
  float l2norm_eps;     /* eps of the q/k L2 normalisation, >= 0 (1e-6 usual) */
  float q_scale;        /* multiplies normalised q; <= 0 means 1/sqrt(d_k) */
} gdn_layer_desc;

/* One per-request state a layer declares (page "Continuous batching for linear
 * attention layers", commit declaring linear_attention_states: each state has a
 * shape and a dtype, and a block holds each on a 128-byte boundary). */
typedef struct {
  char name[16];      /* "conv" or "recurrent" */
  int32_t ndim;
  int64_t shape[4];
  int32_t dtype;      /* gdn_dtype */
  int64_t bytes;      /* product of shape times element size */
  int32_t align;      /* required alignment of the state inside a block: 128 */
} gdn_state_decl;

/* Fills out[0] = conv state [W-1][C] in act dtype (W-1 may be 0) and
 * out[1] = recurrent state [H_v][d_k][d_v] fp32.  Host only. */
int gdn_state_spec(const gdn_layer_desc* desc, gdn_state_decl out[2]);

/* Bytes of device workspace gdn_varlen_forward needs for a batch of
 * total_tokens packed tokens and num_seqs sequences (y, the conv task
 * counters and the device plan).  Host only. */
int gdn_workspace_size(const gdn_layer_desc* desc, int32_t total_tokens,
                       int32_t num_seqs, size_t* bytes);

/* The packed-batch forward (steps 1-4 above).
 *
 * Device pointers (all on the current HIP device, 16-byte aligned):
 *   x            [T][C] act dtype, row-major (the packed row of conv inputs)
 *   conv_weight  [C][W] act dtype
 *   g            [T][H_v] fp32, log of the decay (a = exp(g), g <= 0 expected)
 *   beta         [T][H_v] fp32, the delta-rule write strength
 *   cu_seqlens   [N+1] int32, cu_seqlens[0] = 0, non-decreasing, cu_seqlens[N] = T
 *   read_idx     [N] int32, block each sequence reads its states from (0 = trash
 *                block, for a request with no past)
 *   write_idx    [N] int32, block each sequence owns and overwrites; < 0 marks a
 *                padding sequence: nothing is read or written for it and its out
 *                rows are left as they are
 *   conv_pool    P blocks of the conv state, block i at conv_pool + i*conv_block_stride
 *                bytes; may be NULL when W == 1
 *   ssm_pool     P blocks of the recurrent state [H_v][d_k][d_v] fp32, block i at
 *                ssm_pool + i*ssm_block_stride bytes (the two pools may be views of
 *                one block buffer at different 128-byte aligned offsets, the
 *                placement gdn_state_spec asks for; the library itself needs both
 *                strides to be multiples of 16 bytes and at least the state size)
 *   out          [T][H_v][d_v] act dtype
 *   workspace    device scratch of at least gdn_workspace_size() bytes, 256-byte
 *                aligned; its contents on entry do not matter
 * Host pointer:
 *   cu_seqlens_host  the same N+1 offsets in host memory; the library plans its
 *                launches from it so that it never reads device memory back.
 *                NULL: the launch is planned on the device from cu_seqlens by a
 *                small planning kernel (at most 1024 sequences), and every launch
 *                size and argument depends only on N, total_tokens and the
 *                pointers, so a captured graph of the call replays correctly for
 *                any offsets, indices and data of the same N and total_tokens
 *                (the offsets are then not checked: they must be non-decreasing
 *                from 0 to total_tokens).  Results are bitwise the same as with
 *                the host plan.
 * Preconditions the library cannot check without a sync (violations give
 * undefined results, never out-of-bounds accesses for indices outside [0, P),
 * which are skipped and raise GDN_DEV_BAD_INDEX, see gdn_device_status): device
 * cu_seqlens equals cu_seqlens_host; write blocks are
 * distinct, never block 0 and never another sequence's read block; block 0 is
 * all zero.  read_idx[i] == write_idx[i] is the ordinary in-place continue.
 * stream is a hipStream_t (NULL = the default stream).
 *
 * Paths: sequences of two or more tokens run in chunks of 64 rows in the WY / UT
 * form, sequences of length 0 and 1 run token by token beside them.  The bf16
 * layer with d_k = d_v = 128 takes the bf16-operand MFMA chunk kernel
 * ("chunk_scan"); every other head size, and the all-fp32 layer, take a chunk
 * kernel that computes in fp32 on the fp32 MFMA ("chunk_generic"), after the
 * conv kernel has written the normalised rows into the workspace.
 *
 * Launch plan (bf16, 128 x 128 heads): the conv of the chunked rows runs in its
 * own kernel, inside the chunk kernel before the scans, or (host plan only, when the scans leave at
 * least 32 CUs free) streamed by helper workgroups of the chunk kernel while
 * the scans run (the first workgroups to start become the helpers, so no scan
 * waits for a workgroup that has not started); a time model chooses.  The environment variable
 * GDN_CONV_IN_SCAN=never|always|stream (read at every call) overrides the
 * choice ("stream" falls back to the others where it cannot run).  Inside the
 * chunk kernel (host plan), the workgroups claim the conv tasks either longest
 * sequence first, each until its own sequence's tasks are claimed, or chunk by
 * chunk across the sequences by a time budget alone (for batches whose lengths
 * are far apart); the host's estimates choose, and GDN_CONV_CLAIM=own|budget
 * overrides them.  Every output and state is the same bit for bit in all of
 * these.
 */
int gdn_varlen_forward(const gdn_layer_desc* desc, const void* x,
                       const void* conv_weight, const float* g, const float* beta,
                       const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                       int32_t num_seqs, int32_t total_tokens,
                       const int32_t* read_idx, const int32_t* write_idx,
                       void* conv_pool, int64_t conv_block_stride, float* ssm_pool,
                       int64_t ssm_block_stride, int32_t num_blocks, void* out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* gdn_varlen_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same arguments without the workspace; the scratch the call
 * needs (gdn_workspace_size for the batch) lives in a static device buffer of
 * GDN_STATIC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends.  No allocation of any kind, no host sync.
 *   A batch that needs more scratch than that is rejected with
 *   GDN_EWORKSPACE before any device work (64 MiB holds the scratch of a
 *   batch of up to about 4000 tokens of an 8192-channel bf16 layer).
 *   Every call on one device shares that device's buffer, and a call leaves
 *   its contents behind: calls that overlap in time on one device (on
 *   different streams, or from different threads) race and give undefined
 *   results.  Calls in stream order on one stream are always safe: each call
 *   resets what it needs at zero itself.
 * Results are bitwise those of gdn_varlen_forward. */
#define GDN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int gdn_varlen_forward_noalloc(const gdn_layer_desc* desc, const void* x,
                               const void* conv_weight, const float* g, const float* beta,
                               const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                               int32_t num_seqs, int32_t total_tokens,
                               const int32_t* read_idx, const int32_t* write_idx,
                               void* conv_pool, int64_t conv_block_stride, float* ssm_pool,
                               int64_t ssm_block_stride, int32_t num_blocks, void* out,
                               void* stream);

/* A standalone varlen conv layer (the tracker page lists models with conv-only
 * layers): step 1 above, with or without the SiLU, and the conv-state part of
 * step 4, without the split, normalisation and recurrence.  For every sequence
 * i of the packed row,
 *   y[t][c] = act( sum_j w[c][j] * xext[t + j][c] ),  xext = [conv state of
 *   read_idx[i] (W-1 rows); the sequence's x rows],
 * with act = SiLU when silu != 0, else the identity, w[c][W-1] multiplying the
 * current token; then the last W-1 rows of xext become the conv state of
 * write_idx[i].  A padding sequence (write_idx < 0) reads and writes nothing
 * and its y rows are left as they are.
 *   channels   C, a multiple of 8;  conv_width W in 1..4;  act_dtype GDN_F32 or GDN_BF16
 *   x          [T][C] act dtype, device, 16-byte aligned
 *   conv_weight [C][W] act dtype, device
 *   cu_seqlens, cu_seqlens_host, read_idx, write_idx, num_blocks: as for gdn_varlen_forward
 *   conv_pool  P blocks of [W-1][C] act dtype at conv_pool + i*conv_block_stride
 *              (stride a multiple of 16 and >= (W-1)*C*size); may be NULL when W == 1
 *   y          [T][C] act dtype, device, 16-byte aligned (may not alias x)
 * Enqueued on `stream`; no allocation, no host sync.  Preconditions as for
 * gdn_varlen_forward (block 0 all zero, distinct write blocks). */
int gdn_varlen_conv(int32_t channels, int32_t conv_width, int32_t act_dtype, int32_t silu,
                    const void* x, const void* conv_weight, const int32_t* cu_seqlens,
                    const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t total_tokens,
                    const int32_t* read_idx, const int32_t* write_idx, void* conv_pool,
                    int64_t conv_block_stride, int32_t num_blocks, void* y, void* stream);

/* Fork copy (the PR description: a request's states are copied when it forks):
 * for i < n, both states of block src[i] (its conv state and its recurrent
 * state) are copied bit for bit to block dst[i], so the child continues
 * exactly where the parent stands.
 *   conv_pool, conv_block_stride, ssm_pool, ssm_block_stride, num_blocks: as
 *       for gdn_varlen_forward (conv_pool may be NULL when W == 1)
 *   src, dst  [n] int32 block indices, device memory; a pair with an index
 *       outside [0, num_blocks), or with src[i] == dst[i], is skipped
 * Preconditions: the dst blocks are distinct and none is a src block of the
 * same call (pairs run in parallel).  Enqueued on `stream`; no allocation, no
 * host sync. */
int gdn_state_copy(const gdn_layer_desc* desc, void* conv_pool, int64_t conv_block_stride,
                   float* ssm_pool, int64_t ssm_block_stride, int32_t num_blocks,
                   const int32_t* src, const int32_t* dst, int32_t n, void* stream);

/* ---- Kimi delta attention (KDA) layer with per-sequence states.
 * The pages list KDA (Kimi Linear, GLM5-next) among the layers whose states
 * the cache holds, without a formula.  The recurrence is the published one
 * (Kimi Linear technical report, 2025): the gated delta rule with a decay per
 * key channel, S_t = (I - b_t k_t k_t^T) diag(a_t) S_{t-1} + b_t k_t v_t^T,
 * o_t = S_t^T q_t, a_t = exp(g_t) with g_t in R^{d_k} per value head.  The
 * rest of the layer (conv + SiLU from the conv state, q/k L2 norm, q scale,
 * GQA head map, paged states, padding and empty sequences) is that of
 * gdn_varlen_forward.
 *   g  [T][H_v][d_k] fp32 (log decay per key channel; <= 0 for a decay)
 *   workspace  device scratch of at least gdn_workspace_size() bytes, 256-byte
 *              aligned, or NULL (then every sequence runs token by token)
 *   every other argument as for gdn_varlen_forward; cu_seqlens_host is required
 * Sequences of two or more tokens run in chunks of 64 rows (bf16 with
 * d_k = d_v = 128 and a workspace): the normalised rows are written into the
 * workspace (by the chunk kernel's own workgroups before their scans when all
 * of them fit on the device at once and the workspace is gdn_workspace_size()
 * bytes, else by the conv kernel first), and a chunk kernel evaluates the WY / UT form with the
 * decay inside the channel sums of its block products (every exponentiated
 * decay difference <= 1, except on a diagonal 16-row block, bounded there by
 * that block's own decay; a block whose decay passes e^80 on some channel is
 * computed in fp32 without that factor).  Sequences of length 0 and 1, and
 * every sequence in other shapes or in fp32, run token by token (one workgroup
 * per sequence and value head, the conv, norms and recurrence in one pass).
 * Then the conv-state commit.  No allocation, no host sync. */
int kda_varlen_forward(const gdn_layer_desc* desc, const void* x, const void* conv_weight,
                       const float* g, const float* beta, const int32_t* cu_seqlens,
                       const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t total_tokens,
                       const int32_t* read_idx, const int32_t* write_idx, void* conv_pool,
                       int64_t conv_block_stride, float* ssm_pool, int64_t ssm_block_stride,
                       int32_t num_blocks, void* out, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ---- Mamba2 scan with per-sequence states.
 * The model-support tracker page (continuous batching for the remaining
 * linear-attention and state-space hybrids) names a varlen scan with
 * per-sequence states for the Mamba2 mixers as groundwork, beside the varlen
 * conv (gdn_varlen_conv runs that conv: SiLU, no normalisation).  The pages
 * give no formula; the recurrence is Mamba2's selective state space model with
 * a scalar decay per head (Dao and Gu, "Transformers are SSMs", ICML 2024):
 *   d_t = softplus(dt_t + dt_bias_m) (or dt_t + dt_bias_m), a_t = exp(d_t A_m),
 *   h_t = a_t h_{t-1} + d_t x_t B_t^T (h [P][N] fp32), y_t = h_t C_t + D_m x_t.
 * Sequence i starts from ssm_pool block read_idx[i] (block 0 is the all-zero
 * trash block) and its final h overwrites block write_idx[i]; write_idx[i] < 0
 * marks a padding sequence (nothing read or written); a sequence of length 0
 * copies its state.  The same paging rules as gdn_varlen_forward apply. */
typedef struct {
  int32_t num_heads;    /* H */
  int32_t head_dim;     /* P: this build runs 64 */
  int32_t num_groups;   /* G, divides H; head m reads the B and C of group m / (H / G) */
  int32_t state_dim;    /* N: this build runs 128 */
  int32_t dt_softplus;  /* nonzero: d = softplus(dt + dt_bias) */
} ssd_layer_desc;

/*   x          bf16, row t of head m at x + t*x_row_stride + m*P (elements)
 *   B, C       bf16, row t of group g at B + t*bc_row_stride + g*N (same for C);
 *              x, B and C may be views into one conv output row [x | B | C]
 *   x_row_stride, bc_row_stride  in elements, multiples of 8, at most 2^23
 *   dt         [T][H] fp32; dt_bias [H] fp32 or NULL (0); A [H] fp32 (negative
 *              for a decay); D [H] fp32 or NULL (no skip term)
 *   cu_seqlens [num_seqs+1] int32, device; cu_seqlens_host: the same on the
 *              host, or NULL (then not checked: non-decreasing from 0 to
 *              total_tokens; sequences whose offsets leave [0, total_tokens]
 *              are skipped)
 *   read_idx, write_idx [num_seqs] int32, device
 *   ssm_pool   num_blocks blocks of [H][P][N] fp32 at ssm_pool + i*ssm_block_stride
 *              bytes (a multiple of 16, >= H*P*N*4)
 *   y          [T][H][P] bf16 (rows of padding sequences are left as they are)
 * All device pointers 16-byte aligned.  Returns GDN_EUNSUPPORTED for other
 * head or state sizes.  Enqueued on `stream` (a chunked kernel for sequences
 * of length >= 2, a token kernel for lengths 0 and 1; with cu_seqlens_host
 * only the kernels some sequence needs); no allocation, no host sync.
 * Precision: chunks take bf16 operands into fp32 products; the token step is
 * fp32; the state is fp32. */
int ssd_varlen_scan(const ssd_layer_desc* desc, const void* x, int64_t x_row_stride, const void* B,
                    const void* C, int64_t bc_row_stride, const float* dt, const float* dt_bias,
                    const float* A, const float* D, const int32_t* cu_seqlens,
                    const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t total_tokens,
                    const int32_t* read_idx, const int32_t* write_idx, float* ssm_pool,
                    int64_t ssm_block_stride, int32_t num_blocks, void* y, void* stream);

/* Message of the last non-OK status returned on this thread ("" if none). */
const char* gdn_last_error(void);

/* Device-side status of the current device.  Some failures happen where no
 * return value can carry them, so the kernels of every entry point raise
 * sticky bits instead:
 *   GDN_DEV_WAIT_EXPIRED  a bounded wait between the waves or workgroups of a
 *       kernel gave up (no kernel can hang, but the outputs and states of that
 *       call are then not valid);
 *   GDN_DEV_BAD_INDEX  a device-resident read or write block outside [0, P)
 *       was skipped (a negative write block marks padding and raises nothing);
 *       the page's allocator commit likewise refuses bad states with a readable
 *       error rather than running on them.
 * The call waits for `stream` (a host sync: a check for tests and debugging,
 * not for the step itself), then reads the bits raised since the last clear
 * into *bits (may be NULL); clear != 0 resets them.  Returns GDN_OK when no bit
 * is set, GDN_EDEVICE with a message naming them otherwise, GDN_EHIP when the
 * device could not be read. */
#define GDN_DEV_WAIT_EXPIRED 1u
#define GDN_DEV_BAD_INDEX 2u
int gdn_device_status(int clear, uint32_t* bits, void* stream);

/* Measurement support (not needed to run the layer).
 * gdn_kernel_timing(1) makes every later gdn_varlen_forward, gdn_varlen_conv,
 * gdn_state_copy, kda_varlen_forward and ssd_varlen_scan in this process record a HIP event pair on the call's
 * stream around each kernel it launches,
 * and clears the totals; gdn_kernel_timing(0) stops recording.
 * gdn_kernel_times() waits for the recorded events (a host sync), adds their
 * elapsed times to per-kernel totals and copies up to `max` entries to `out`;
 * `count` receives the number of kernels with at least one timed launch.
 * The library creates the events it records and keeps them for reuse. */
typedef struct {
  char name[32];      /* kernel: "conv_silu_norm", "chunk_scan", "token_recurrent", "conv_state_commit",
                         "state_copy", "task_counter_reset", "device_plan", "ssd_scan", "ssd_token",
                         "kda_chunk", "chunk_generic" */
  double total_ms;    /* summed event-to-event time of its timed launches */
  int64_t launches;
} gdn_kernel_time;

int gdn_kernel_timing(int enable);
int gdn_kernel_times(gdn_kernel_time* out, int32_t max, int32_t* count);

/* Measurement support: the dense MFMA rate the device reaches on back-to-back
 * independent products (v_mfma_f32_16x16x32_bf16 for dtype GDN_BF16,
 * v_mfma_f32_16x16x4_f32 for GDN_F32; four waves per SIMD, eight accumulator
 * chains per wave, `iters` rounds in [1, 2^20]), in TFLOP/s, so kernel rates can
 * be quoted against a measured peak beside the published one.  Runs a warm-up
 * launch and a timed one on `stream` and waits for them (a host sync);
 * allocates nothing but two events, destroyed before it returns. */
int gdn_mfma_peak_probe(int32_t dtype, int32_t iters, double* tflops, void* stream);

/* Measurement support: the HBM rate of a plain streaming copy of `bytes` bytes
 * (a positive multiple of 16, at most 2^36) from device buffer `src` to device
 * buffer `dst` (both 16-byte aligned, not overlapping, each at least `bytes`
 * long; the caller owns them), in GB/s counting bytes read plus bytes written.
 * 16-byte non-temporal loads and stores, four in flight per thread, one
 * 256-thread block per 32 KiB span.  Runs a
 * warm-up copy and `reps` timed ones (in [1, 1000]) on `stream` and waits for
 * them (a host sync); allocates nothing but two events, destroyed before it
 * returns.  dst ends up equal to src. */
int gdn_hbm_copy_probe(const void* src, void* dst, int64_t bytes, int32_t reps, double* gbs, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
