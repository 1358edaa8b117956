"""fp64 CPU oracle for the packed-batch Mamba2 scan with per-sequence states.

TEST INFRASTRUCTURE ONLY: the test suite and ``__graft_entry__.smoke()`` may
import it; the GPU library never does, and it imports nothing from it.

The model-support tracker page (continuous batching for the remaining
linear-attention and state-space hybrids) names, as groundwork for the Mamba2
mixers, a varlen scan with per-sequence states beside the varlen causal conv.
The pages give no formula for that scan; this follows the published Mamba2
state space recurrence (Dao and Gu, "Transformers are SSMs", ICML 2024: the
selective SSM with A a scalar times the identity per head), token by token, in
the same packed-batch and paged-state setting as the gated delta rule:

    d_t   = softplus(dt_t + dt_bias)            (or dt_t + dt_bias without softplus)
    a_t   = exp(d_t * A)                         (A < 0 per head)
    h_t   = a_t h_{t-1} + d_t x_t B_t^T          (h: [P][N] per head)
    y_t   = h_t C_t + D x_t

x_t is the head's [P] input, B_t and C_t the [N] vectors of the head's group
(head m uses group m // (H / G), G groups of consecutive heads), D a per-head
skip weight.  Sequence i starts from ssm_pool[read_idx[i]] (block 0 is the
all-zero trash block for a sequence with no past) and its final h goes to
ssm_pool[write_idx[i]]; write_idx[i] < 0 marks a padding sequence, which
reads and writes nothing.  A sequence of length 0 copies its state.

Parity pins (tests/test_oracle_ssd_pins.py): the quadratic dual form written
out as a masked matrix product, the closed form without decay, one token
from the trash block, splitting a sequence over two calls, padding and empty
sequences.  The group map is a convention: parity unpinned for it.
"""
from __future__ import annotations

import numpy as np


def softplus(v):
    """log(1 + e^v), computed without overflow."""
    return np.logaddexp(0.0, v)


def varlen_scan(x, dt, A, B, C, D, dt_bias, cu_seqlens, read_idx, write_idx, ssm_pool, dt_softplus=True):
    """Runs every sequence of the packed batch through the recurrence.

    x [T][H][P], dt [T][H], A [H], B and C [T][G][N], D [H] or None, dt_bias [H]
    or None, cu_seqlens [N+1], read_idx / write_idx [N], ssm_pool [nb][H][P][N].
    Returns (y [T][H][P], new pool), both float64; rows of padding sequences
    are left zero in y.
    """
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    pool = np.array(ssm_pool, dtype=np.float64)
    T, H, P = x.shape
    G = B.shape[1]
    Dv = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    bias = np.zeros(H) if dt_bias is None else np.asarray(dt_bias, dtype=np.float64)
    grp = np.arange(H) // (H // G)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    y = np.zeros((T, H, P))
    # every sequence reads its start state before any is written (the write
    # blocks are distinct and never another sequence's read block)
    starts = [pool[int(r)].copy() if int(w) >= 0 else None for r, w in zip(read_idx, write_idx)]
    for s in range(len(cu) - 1):
        if int(write_idx[s]) < 0:
            continue
        h = starts[s]
        for t in range(int(cu[s]), int(cu[s + 1])):
            d = dt[t] + bias
            if dt_softplus:
                d = softplus(d)
            a = np.exp(d * A)
            h = a[:, None, None] * h + (d[:, None] * x[t])[:, :, None] * B[t][grp][:, None, :]
            y[t] = np.einsum("hpn,hn->hp", h, C[t][grp]) + Dv[:, None] * x[t]
        pool[int(write_idx[s])] = h
    return y, pool
