/*
 * gdn_oracle.c -- plain, slow fp64 CPU oracle for the packed-batch (varlen)
 * forward of a gated-delta-net linear-attention layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file defines what the layer computes so the
 * GPU library can be checked against it.  It shares no code, header, table or
 * helper with the GPU library, and only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  The GPU library never calls it.
 *
 * What it follows
 * ---------------
 * Page "Continuous batching for linear attention layers" (PR description and
 * the commit that introduces the linear attention cache allocator):
 *   - a linear-attention layer keeps, per request, a fixed-size state made of
 *     the last inputs of its causal convolution and its recurrent state;
 *   - the state lives in one block per request, read from the zeroed trash
 *     block while the request has no past, and overwritten in place by every
 *     forward pass;
 *   - the packed batch runs as one row: a varlen causal convolution continues
 *     every sequence from its own conv state, and the recurrence continues
 *     every sequence from its own recurrent state, sequences delimited by
 *     cu_seqlens.
 * The recurrence is the gated delta rule (Gated Delta Networks, Yang et al.,
 * ICLR 2025), written here in the orientation where the state S of a value
 * head is stored [d_k][d_v] (d_v fastest) and read out as o = S^T q:
 *     S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t,
 * with a_t = exp(g_t) and b_t = beta_t given per token and value head.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - channel order of the conv input/output: [q | k | v], head-major;
 *   - value head m reads key head m / (H_v / H_k)               (parity unpinned);
 *   - conv taps: w[c][W-1] multiplies the current token (causal
 *     cross-correlation), no bias; the conv state is the last W-1 pre-conv
 *     inputs, oldest row first, stored [W-1][C];
 *   - SiLU on all channels after the conv; then q and k of each key head are
 *     L2-normalised as x / sqrt(sum x^2 + eps) and q is multiplied by q_scale;
 *   - o_t reads the state after the update of token t;
 *   - write_idx < 0 marks a padding sequence: nothing is read or written.
 *
 * Everything is computed in fp64 from the exact stored input values (bf16 and
 * fp32 widen exactly).  The oracle walks every sequence token by token.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t num_k_heads;
  int32_t num_v_heads;
  int32_t head_k_dim;
  int32_t head_v_dim;
  int32_t conv_width;
  int32_t act_bf16; /* 1: x, conv weight and conv pool hold bf16; 0: fp32 */
  double l2norm_eps;
  double q_scale; /* <= 0 means 1/sqrt(head_k_dim) */
} gdn_oracle_layer;

static double act_load(const void* base, int64_t i, int bf16) {
  if (bf16) {
    uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
  }
  return (double)((const float*)base)[i];
}

/* Depthwise causal convolution of one sequence followed by SiLU.
 * The sequence is extended on the left by its conv state:
 *   xext = [tail (W-1 rows); x (L rows)],  y[t][c] = SiLU(sum_j w[c][j] * xext[t+j][c]).
 * tail: [W-1][C], x: [L][C], w: [C][W], y: [L][C]. */
void gdn_oracle_conv_silu(int64_t C, int32_t W, int64_t L, const double* tail,
                          const double* x, const double* w, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < C; ++c) {
    for (int64_t t = 0; t < L; ++t) {
      double acc = 0.0;
      for (int32_t j = 0; j < W; ++j) {
        int64_t i = t + j; /* index into xext */
        double xv = (i < W - 1) ? tail[i * C + c] : x[(i - (W - 1)) * C + c];
        acc += w[c * W + j] * xv;
      }
      y[t * C + c] = acc / (1.0 + exp(-acc));
    }
  }
}

/* Standalone varlen conv layer over a packed row (the tracker page lists
 * models with conv-only layers; the mechanism is the varlen conv of the PR
 * description, without the split, normalisation and recurrence).  For every
 * sequence, with xext = [conv state of its read block; its x rows]:
 *   y[t][c] = act( sum_j w[c][j] * xext[t+j][c] ),  act = SiLU if silu else identity,
 * and the last W-1 rows of xext become the conv state of its write block
 * (raw storage copies).  write_idx < 0: the sequence is skipped (its y rows are
 * left as they are, NaN from the caller).
 *   x [T][C] act, w [C][W] act, conv_pool [P][W-1][C] act (updated), y [T][C] fp64.
 * Returns 0, or -1 on an index it cannot use. */
int gdn_oracle_varlen_conv(int64_t C, int32_t W, int32_t act_bf16, int32_t silu, const void* x,
                           const void* conv_weight, const int32_t* cu_seqlens, int32_t num_seqs,
                           const int32_t* read_idx, const int32_t* write_idx, void* conv_pool,
                           int32_t num_blocks, double* y) {
  const size_t esz = act_bf16 ? 2 : 4;
  const int64_t tail_elems = (int64_t)(W - 1) * C;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t r0 = cu_seqlens[s];
    const int64_t L = (int64_t)cu_seqlens[s + 1] - r0;
    const int32_t rb = read_idx[s], wb = write_idx[s];
    if (wb < 0) continue;
    if (L < 0 || rb < 0 || rb >= num_blocks || wb >= num_blocks) return -1;
    /* xext as raw storage: W-1 state rows then the L input rows */
    const int64_t rows = (W - 1) + L;
    char* ext = (char*)malloc(esz * (size_t)(rows * C > 0 ? rows * C : 1));
    if (tail_elems > 0)
      memcpy(ext, (char*)conv_pool + (size_t)rb * esz * (size_t)tail_elems, esz * (size_t)tail_elems);
    if (L > 0) memcpy(ext + esz * (size_t)tail_elems, (const char*)x + esz * (size_t)(r0 * C), esz * (size_t)(L * C));
    for (int64_t t = 0; t < L; ++t)
      for (int64_t c = 0; c < C; ++c) {
        double acc = 0.0;
        for (int32_t j = 0; j < W; ++j)
          acc += act_load(conv_weight, c * W + j, act_bf16) * act_load(ext, (t + j) * C + c, act_bf16);
        y[(r0 + t) * C + c] = silu ? acc / (1.0 + exp(-acc)) : acc;
      }
    if (tail_elems > 0)
      memcpy((char*)conv_pool + (size_t)wb * esz * (size_t)tail_elems, ext + esz * (size_t)(L * C),
             esz * (size_t)tail_elems);
    free(ext);
  }
  return 0;
}

/* In-place L2 normalisation of n values, then multiplication by scale. */
void gdn_oracle_l2norm(int64_t n, double* v, double eps, double scale) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += v[i] * v[i];
  double inv = 1.0 / sqrt(ss + eps);
  for (int64_t i = 0; i < n; ++i) v[i] = v[i] * inv * scale;
}

/* The gated delta rule over L tokens of one (sequence, value head).
 * q, k: [L][dk]; v: [L][dv]; g, beta: [L]; S: [dk][dv] in/out; o: [L][dv].
 * Token t:  a = exp(g[t]), b = beta[t]
 *           S <- a (I - b k k^T) S + b k v^T   with (I - b k k^T) S = S - b k (k^T S)
 *           o[t] = S^T q                        (the updated state)          */
void gdn_oracle_delta_rule(int32_t dk, int32_t dv, int64_t L, const double* q,
                           const double* k, const double* v, const double* g,
                           const double* beta, double* S, double* o) {
  double* kS = (double*)malloc(sizeof(double) * (size_t)dv);
  for (int64_t t = 0; t < L; ++t) {
    const double* qt = q + t * dk;
    const double* kt = k + t * dk;
    const double* vt = v + t * dv;
    double a = exp(g[t]);
    double b = beta[t];
    for (int32_t j = 0; j < dv; ++j) {
      double s = 0.0;
      for (int32_t i = 0; i < dk; ++i) s += kt[i] * S[i * dv + j];
      kS[j] = s;
    }
    for (int32_t i = 0; i < dk; ++i)
      for (int32_t j = 0; j < dv; ++j)
        S[i * dv + j] = a * (S[i * dv + j] - b * kt[i] * kS[j]) + b * kt[i] * vt[j];
    for (int32_t j = 0; j < dv; ++j) {
      double s = 0.0;
      for (int32_t i = 0; i < dk; ++i) s += S[i * dv + j] * qt[i];
      o[t * dv + j] = s;
    }
  }
  free(kS);
}

/* Packed-batch layer forward.
 *   x [T][C] act, conv_weight [C][W] act, g/beta [T][H_v] fp32,
 *   cu_seqlens [N+1], read_idx/write_idx [N],
 *   conv_pool [P][W-1][C] act (updated in place), ssm_pool [P][H_v][dk][dv]
 *   fp32 (updated in place, final state rounded to fp32),
 *   head_mask [H_v] or NULL (only value heads with a nonzero entry are computed;
 *   rows, states and pool slices of the other heads are left as they are),
 *   out [T][H_v][dv] fp64, final_ssm [N][H_v][dk][dv] fp64 or NULL.
 * Returns 0, or -1 on an argument it cannot use. */
int gdn_oracle_forward(const gdn_oracle_layer* d, const void* x,
                       const void* conv_weight, const float* g, const float* beta,
                       const int32_t* cu_seqlens, int32_t num_seqs,
                       const int32_t* read_idx, const int32_t* write_idx,
                       void* conv_pool, float* ssm_pool, int32_t num_blocks,
                       const uint8_t* head_mask, double* out, double* final_ssm,
                       int32_t nthreads) {
  const int64_t Hk = d->num_k_heads, Hv = d->num_v_heads;
  const int64_t dk = d->head_k_dim, dv = d->head_v_dim;
  const int32_t W = d->conv_width;
  const int bf16 = d->act_bf16;
  if (Hk <= 0 || Hv <= 0 || Hv % Hk != 0 || dk <= 0 || dv <= 0 || W < 1) return -1;
  const int64_t G = Hv / Hk;
  const int64_t C = 2 * Hk * dk + Hv * dv;
  const double qs = d->q_scale > 0.0 ? d->q_scale : 1.0 / sqrt((double)dk);
  const size_t esz = bf16 ? 2 : 4;
  const int64_t tail_elems = (int64_t)(W - 1) * C;
  const int64_t state_elems = Hv * dk * dv;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif

  double* w = (double*)malloc(sizeof(double) * (size_t)(C * W));
  for (int64_t i = 0; i < C * W; ++i) w[i] = act_load(conv_weight, i, bf16);

  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t r0 = cu_seqlens[s];
    const int64_t L = (int64_t)cu_seqlens[s + 1] - r0;
    const int32_t rb = read_idx[s], wb = write_idx[s];
    if (wb < 0) continue; /* padding sequence */
    if (L < 0 || rb < 0 || rb >= num_blocks || wb >= num_blocks) {
      free(w);
      return -1;
    }

    /* conv state of the read block, as values and as raw storage */
    char* tail_raw = (char*)malloc(esz * (size_t)(tail_elems > 0 ? tail_elems : 1));
    double* tail = (double*)malloc(sizeof(double) * (size_t)(tail_elems > 0 ? tail_elems : 1));
    if (tail_elems > 0) {
      memcpy(tail_raw, (char*)conv_pool + (size_t)rb * esz * (size_t)tail_elems,
             esz * (size_t)tail_elems);
      for (int64_t i = 0; i < tail_elems; ++i) tail[i] = act_load(tail_raw, i, bf16);
    }

    /* conv + SiLU over all channels of the sequence */
    double* xs = (double*)malloc(sizeof(double) * (size_t)(L * C > 0 ? L * C : 1));
    double* y = (double*)malloc(sizeof(double) * (size_t)(L * C > 0 ? L * C : 1));
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < L; ++t)
      for (int64_t c = 0; c < C; ++c) xs[t * C + c] = act_load(x, (r0 + t) * C + c, bf16);
    gdn_oracle_conv_silu(C, W, L, tail, xs, w, y);

    /* q and k of each key head: L2-normalise; q also scaled */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < L; ++t)
      for (int64_t h = 0; h < Hk; ++h) {
        gdn_oracle_l2norm(dk, y + t * C + h * dk, d->l2norm_eps, qs);
        gdn_oracle_l2norm(dk, y + t * C + Hk * dk + h * dk, d->l2norm_eps, 1.0);
      }

    /* recurrence per value head */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < Hv; ++m) {
      if (head_mask && !head_mask[m]) continue;
      const int64_t h = m / G;
      double* q = (double*)malloc(sizeof(double) * (size_t)(L * dk + 1));
      double* k = (double*)malloc(sizeof(double) * (size_t)(L * dk + 1));
      double* v = (double*)malloc(sizeof(double) * (size_t)(L * dv + 1));
      double* gg = (double*)malloc(sizeof(double) * (size_t)(L + 1));
      double* bb = (double*)malloc(sizeof(double) * (size_t)(L + 1));
      double* o = (double*)malloc(sizeof(double) * (size_t)(L * dv + 1));
      double* S = (double*)malloc(sizeof(double) * (size_t)(dk * dv));
      for (int64_t t = 0; t < L; ++t) {
        for (int64_t i = 0; i < dk; ++i) {
          q[t * dk + i] = y[t * C + h * dk + i];
          k[t * dk + i] = y[t * C + Hk * dk + h * dk + i];
        }
        for (int64_t j = 0; j < dv; ++j) v[t * dv + j] = y[t * C + 2 * Hk * dk + m * dv + j];
        gg[t] = (double)g[(r0 + t) * Hv + m];
        bb[t] = (double)beta[(r0 + t) * Hv + m];
      }
      const float* S0 = ssm_pool + (size_t)rb * (size_t)state_elems + (size_t)(m * dk * dv);
      for (int64_t i = 0; i < dk * dv; ++i) S[i] = (double)S0[i];
      gdn_oracle_delta_rule((int32_t)dk, (int32_t)dv, L, q, k, v, gg, bb, S, o);
      for (int64_t t = 0; t < L; ++t)
        for (int64_t j = 0; j < dv; ++j) out[((r0 + t) * Hv + m) * dv + j] = o[t * dv + j];
      float* S1 = ssm_pool + (size_t)wb * (size_t)state_elems + (size_t)(m * dk * dv);
      for (int64_t i = 0; i < dk * dv; ++i) S1[i] = (float)S[i];
      if (final_ssm)
        memcpy(final_ssm + ((size_t)s * (size_t)Hv + (size_t)m) * (size_t)(dk * dv), S,
               sizeof(double) * (size_t)(dk * dv));
      free(q); free(k); free(v); free(gg); free(bb); free(o); free(S);
    }

    /* new conv state: the last W-1 rows of xext = [old tail; x], copied bit for bit */
    if (tail_elems > 0) {
      char* dst = (char*)conv_pool + (size_t)wb * esz * (size_t)tail_elems;
      for (int64_t j = 0; j < W - 1; ++j) {
        int64_t i = L + j; /* row of xext */
        const char* src = (i < W - 1) ? tail_raw + esz * (size_t)(i * C)
                                      : (const char*)x + esz * (size_t)((r0 + i - (W - 1)) * C);
        memcpy(dst + esz * (size_t)(j * C), src, esz * (size_t)C);
      }
    }
    free(tail_raw); free(tail); free(xs); free(y);
  }
  free(w);
  return 0;
}
