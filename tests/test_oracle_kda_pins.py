"""Pins of the KDA oracle (oracle/kda_oracle.py) to facts that do not come from
it: a hand-worked 2 x 2 example with two different channel decays per token
(tests/golden/kda_hand.txt); brute force with the explicit d_k x d_k transition
matrix (I - b k k^T) diag(exp(g)) for d_k != d_v and decays that differ across
the channels; a decay equal on every channel is the gated delta rule (its own
oracle, pinned in tests/test_oracle_pins.py); without the delta term the state
decays row by row in closed form; one token from the trash block has a closed
form; a sequence split over two calls equals one call.  The recurrence is the
published KDA one (Kimi Linear technical report, 2025).

A decay applied to columns instead of rows fails the decay-only pin and the
golden; the decay applied after the projection, diag(a) (I - b k k^T) S, fails
the golden (token 1) and the brute force, whose keys do not commute with the
decays; reading o from S_{t-1} fails the golden.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import kda_oracle

LAYER = workloads.Layer(2, 4, 16, 8, 4, "f32")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rec = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                parts = line.split()
                rec[parts[0]] = np.array([float(v) for v in parts[1:]])
    return rec


def test_hand_worked_example_with_channel_decays():
    """tests/golden/kda_hand.txt: three tokens, d_k = d_v = 2, worked by hand."""
    r = _golden("kda_hand.txt")
    k, v, q = r["k"].reshape(3, 2), r["v"].reshape(3, 2), r["q"].reshape(3, 2)
    g = np.log(r["a"].reshape(3, 2))
    o, S = kda_oracle.recurrence(q, k, v, g, r["b"], r["S0"].reshape(2, 2))
    np.testing.assert_allclose(o, r["o"].reshape(3, 2), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, r["S3"].reshape(2, 2), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("dk,dv", [(5, 3), (3, 4)])
def test_brute_force_transition_matrix(dk, dv):
    """Brute force on tiny inputs: the d_k x d_k transition (I - b k k^T) diag(exp(g_t))
    built explicitly and multiplied, with decays spread across the channels and
    keys that are neither unit nor axis-aligned."""
    rng = np.random.default_rng(40 + dk)
    L = 8
    q, k = rng.standard_normal((L, dk)), rng.standard_normal((L, dk))
    v = rng.standard_normal((L, dv))
    g = -3.0 * rng.random((L, dk))           # channel decays from 1 down to e^-3
    b = rng.random(L)
    S0 = rng.standard_normal((dk, dv))
    o, S = kda_oracle.recurrence(q, k, v, g, b, S0)
    Sref = S0.copy()
    for t in range(L):
        M = (np.eye(dk) - b[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t]))
        Sref = M @ Sref + b[t] * np.outer(k[t], v[t])
        np.testing.assert_allclose(o[t], Sref.T @ q[t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, Sref, rtol=1e-12, atol=1e-13)


def _g_channels(b, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    T = b.total_tokens
    raw = rng.standard_normal((T, LAYER.num_v_heads, LAYER.head_k_dim)) * spread
    return torch.tensor(-np.logaddexp(0.0, raw), dtype=torch.float32)


def _qkv(b):
    """Normalised q, k and v of every row (conv + SiLU, then the L2 norms)."""
    y, _ = oracle.varlen_conv(b.x, b.conv_weight, b.cu_seqlens, b.read_idx, b.write_idx, b.conv_pool, silu=True)
    Hk, dk, dv = LAYER.num_k_heads, LAYER.head_k_dim, LAYER.head_v_dim
    scale = 1.0 / math.sqrt(dk)
    q = np.stack([[oracle.l2norm(y[t, h * dk:(h + 1) * dk], LAYER.l2norm_eps, scale) for h in range(Hk)]
                  for t in range(y.shape[0])])
    k = np.stack([[oracle.l2norm(y[t, Hk * dk + h * dk:Hk * dk + (h + 1) * dk], LAYER.l2norm_eps, 1.0)
                   for h in range(Hk)] for t in range(y.shape[0])])
    v = y[:, 2 * Hk * dk:].reshape(y.shape[0], LAYER.num_v_heads, dv)
    return q, k, v


def test_uniform_decay_is_the_gated_delta_rule():
    b = workloads.random_batch(LAYER, [9, 1, 20], seed=1, fresh=[0, 1, 0])
    g = kda_oracle.with_scalar_decay(b.g, LAYER.head_k_dim)
    out, cp, sp = kda_oracle.forward(LAYER, b.x, b.conv_weight, g, b.beta, b.cu_seqlens, b.read_idx, b.write_idx,
                                     b.conv_pool, b.ssm_pool)
    ro, fin, rcp, _ = oracle.forward(LAYER, b.x, b.conv_weight, b.g, b.beta, b.cu_seqlens, b.read_idx,
                                     b.write_idx, b.conv_pool, b.ssm_pool)
    np.testing.assert_allclose(out, ro, rtol=1e-10, atol=1e-12)
    for s in range(3):  # the fp64 final states (the returned pool is stored in fp32)
        np.testing.assert_allclose(sp[int(b.write_idx[s])], fin[s], rtol=1e-10, atol=1e-12)
    assert torch.equal(cp, rcp)


def test_no_delta_term_decays_rows_in_closed_form():
    """b = 0: S_t = diag(exp(sum_{s<=t} g_s)) S_0 and o_t = S_t^T q_t."""
    b = workloads.random_batch(LAYER, [11], seed=2)
    beta = torch.zeros_like(b.beta)
    g = _g_channels(b, 3)
    out, _, sp = kda_oracle.forward(LAYER, b.x, b.conv_weight, g, beta, b.cu_seqlens, b.read_idx, b.write_idx,
                                    b.conv_pool, b.ssm_pool)
    q, _, _ = _qkv(b)
    S0 = b.ssm_pool[int(b.read_idx[0])].double().numpy()
    cum = np.cumsum(g.double().numpy(), axis=0)  # [T][Hv][dk]
    for m in range(LAYER.num_v_heads):
        h = m // (LAYER.num_v_heads // LAYER.num_k_heads)
        for t in range(11):
            St = np.exp(cum[t, m])[:, None] * S0[m]
            np.testing.assert_allclose(out[t, m], St.T @ q[t, h], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(sp[int(b.write_idx[0]), m], np.exp(cum[-1, m])[:, None] * S0[m], rtol=1e-10)


def test_one_token_from_the_trash_block():
    """S_0 = 0: S_1 = b k v^T and o = b (q . k) v, whatever the decay."""
    b = workloads.random_batch(LAYER, [1], seed=4, fresh=[1])
    g = _g_channels(b, 5)
    out, _, sp = kda_oracle.forward(LAYER, b.x, b.conv_weight, g, b.beta, b.cu_seqlens, b.read_idx, b.write_idx,
                                    b.conv_pool, b.ssm_pool)
    q, k, v = _qkv(b)
    for m in range(LAYER.num_v_heads):
        h = m // (LAYER.num_v_heads // LAYER.num_k_heads)
        bm = float(b.beta[0, m])
        np.testing.assert_allclose(out[0, m], bm * float(q[0, h] @ k[0, h]) * v[0, m], rtol=1e-10, atol=1e-14)
        np.testing.assert_allclose(sp[int(b.write_idx[0]), m], bm * np.outer(k[0, h], v[0, m]), rtol=1e-10,
                                   atol=1e-14)


def test_split_over_two_calls():
    b = workloads.random_batch(LAYER, [13], seed=6)
    g = _g_channels(b, 7)
    out, cp, sp = kda_oracle.forward(LAYER, b.x, b.conv_weight, g, b.beta, b.cu_seqlens, b.read_idx, b.write_idx,
                                     b.conv_pool, b.ssm_pool)
    m = 5
    cu1 = torch.tensor([0, m], dtype=torch.int32)
    cu2 = torch.tensor([0, 13 - m], dtype=torch.int32)
    o1, cp1, sp1 = kda_oracle.forward(LAYER, b.x[:m], b.conv_weight, g[:m], b.beta[:m], cu1, b.read_idx,
                                      b.write_idx, b.conv_pool, b.ssm_pool)
    o2, cp2, sp2 = kda_oracle.forward(LAYER, b.x[m:], b.conv_weight, g[m:], b.beta[m:], cu2, b.write_idx,
                                      b.write_idx, cp1, torch.from_numpy(sp1))
    np.testing.assert_allclose(np.concatenate([o1, o2]), out, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(sp2[int(b.write_idx[0])], sp[int(b.write_idx[0])], rtol=1e-9, atol=1e-12)
    assert torch.equal(cp2, cp)
