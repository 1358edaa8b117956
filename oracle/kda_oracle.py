"""fp64 CPU oracle for the packed-batch Kimi delta attention (KDA) layer.

TEST INFRASTRUCTURE ONLY: the test suite may import it; the GPU library never
does, and it imports nothing from it.

The pages list KDA (Kimi Linear, GLM5-next) among the layers whose per-request
states the cache holds, but give no formula.  This follows the published KDA
recurrence (Kimi Linear technical report, 2025), the gated delta rule with a
decay per key channel instead of one per head, per sequence and value head m:

    S_t = (I - b_t k_t k_t^T) diag(a_t) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t,
    a_t = exp(g_t),  g_t in R^{d_k}

with S stored [d_k][d_v] as for the gated delta rule.  Everything around the
recurrence is the gated-delta-net layer's: depthwise causal conv + SiLU
continued from the conv state (``oracle.varlen_conv``, pinned with the rest of
that oracle), q and k L2-normalised per head with q scaled, key head
m // (H_v / H_k), the paged states (block 0 the zero trash block, write blocks
overwritten in place, write_idx < 0 a padding sequence).

Parity pins (tests/test_oracle_kda_pins.py): a hand-worked 2 x 2 example with
two different channel decays per token (tests/golden/kda_hand.txt), whose first
key does not commute with the decay, so the order of decay and projection is
fixed; brute force with the explicit d_k x d_k transition (I - b k k^T)
diag(exp(g)); a decay equal across the channels reduces to the gated-delta-rule
oracle; without the delta term (b = 0) the state decays row by row in closed
form; one token from the trash block; a sequence split over two calls.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def recurrence(q, k, v, g, beta, S0):
    """KDA over one sequence and value head: q, k [L][d_k] (normalised), v
    [L][d_v], g [L][d_k], beta [L], S0 [d_k][d_v].  Returns (o [L][d_v], S_L)."""
    S = np.array(S0, dtype=np.float64)
    L = q.shape[0]
    o = np.zeros((L, v.shape[1]))
    for t in range(L):
        S = np.exp(g[t])[:, None] * S                   # diag(a_t) S_{t-1}
        u = beta[t] * (v[t] - S.T @ k[t])               # b (v - (diag(a) S)^T k)
        S = S + np.outer(k[t], u)
        o[t] = S.T @ q[t]
    return o, S


def forward(layer, x, conv_weight, g, beta, cu_seqlens, read_idx, write_idx, conv_pool, ssm_pool, heads=None):
    """Packed-batch KDA layer on the CPU.  CPU torch tensors as for
    ``oracle.forward`` except g [T][H_v][d_k].  ``heads``: value heads to run
    (default all).  Returns (out [T][H_v][d_v] float64, NaN where not run or
    padding; conv_pool_new; ssm_pool_new float64)."""
    Hk, Hv, dk, dv = layer.num_k_heads, layer.num_v_heads, layer.head_k_dim, layer.head_v_dim
    y, conv_new = oracle.varlen_conv(x, conv_weight, cu_seqlens, read_idx, write_idx, conv_pool, silu=True)
    T = x.shape[0]
    heads = list(range(Hv)) if heads is None else list(heads)
    scale = layer.q_scale if layer.q_scale > 0 else 1.0 / np.sqrt(dk)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    pool = np.asarray(ssm_pool, dtype=np.float64)
    new = pool.copy()
    out = np.full((T, Hv, dv), np.nan)
    cu = [int(c) for c in cu_seqlens]
    for s in range(len(cu) - 1):
        wb, rb = int(write_idx[s]), int(read_idx[s])
        if wb < 0:
            continue
        r0, r1 = cu[s], cu[s + 1]
        for m in heads:
            h = m // (Hv // Hk)
            q = y[r0:r1, h * dk:(h + 1) * dk]
            k = y[r0:r1, Hk * dk + h * dk:Hk * dk + (h + 1) * dk]
            v = y[r0:r1, 2 * Hk * dk + m * dv:2 * Hk * dk + (m + 1) * dv]
            qn = np.stack([oracle.l2norm(r, layer.l2norm_eps, scale) for r in q]) if r1 > r0 else q
            kn = np.stack([oracle.l2norm(r, layer.l2norm_eps, 1.0) for r in k]) if r1 > r0 else k
            o, S = recurrence(qn, kn, v, g[r0:r1, m], beta[r0:r1, m], pool[rb, m])
            out[r0:r1, m] = o
            new[wb, m] = S
    return out, conv_new, new


def with_scalar_decay(g_head, dk):
    """A per-channel decay that equals the per-head one on every channel."""
    g_head = torch.as_tensor(g_head, dtype=torch.float32)
    return g_head[:, :, None].expand(-1, -1, dk).contiguous()
