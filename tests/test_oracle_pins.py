"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test ties one part of the oracle to a library routine, a closed form, an
invariant of the method, brute force on tiny inputs, or the hand-worked example
in tests/golden/.  The cases are chosen so that a plausible slip (a transposed
state, a wrong tap order, a dropped decay, o read before the update, a wrong
channel offset) fails at least one of them.

Sources: the gated delta rule (Gated Delta Networks, Yang et al., ICLR 2025);
the per-request conv and recurrent states, the trash block and in-place
overwrite from the page "Continuous batching for linear attention layers" (PR
description and the linear attention cache allocator commit).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- conv + SiLU

@pytest.mark.parametrize("W,L", [(4, 9), (4, 1), (4, 2), (3, 5), (2, 1), (1, 6)])
def test_conv_matches_torch_conv1d(W, L):
    """Library routine: depthwise causal conv == torch conv1d (groups=C) on the
    state-extended sequence, then torch SiLU.  Pins tap order and tail order."""
    rng = _rng(W * 100 + L)
    C = 7
    tail = rng.standard_normal((max(W - 1, 0), C))
    x = rng.standard_normal((L, C))
    w = rng.standard_normal((C, W))
    y = oracle.conv_silu(tail, x, w)
    xext = torch.from_numpy(np.concatenate([tail, x], axis=0).T[None])  # [1, C, W-1+L]
    ref = torch.nn.functional.conv1d(xext, torch.from_numpy(w)[:, None, :], groups=C)
    ref = torch.nn.functional.silu(ref)[0].T.numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_conv_width1_identity_silu():
    """Special case: width-1 conv with weight 1 is SiLU of the input."""
    rng = _rng(3)
    x = rng.standard_normal((5, 4))
    y = oracle.conv_silu(np.zeros((0, 4)), x, np.ones((4, 1)))
    np.testing.assert_allclose(y, x / (1 + np.exp(-x)), rtol=1e-15)


# ------------------------------------------------------------------- l2norm

def test_l2norm_unit_and_direction():
    rng = _rng(4)
    for n in (2, 16, 128):
        v = rng.standard_normal(n)
        u = oracle.l2norm(v, eps=1e-6)
        nv = np.linalg.norm(v)
        assert abs(np.linalg.norm(u) - 1.0) < 1e-6 / nv**2 + 1e-14
        cos = u @ v / (np.linalg.norm(u) * nv)
        assert abs(cos - 1.0) < 1e-14
        s = oracle.l2norm(v, eps=1e-6, scale=0.25)
        np.testing.assert_allclose(s, 0.25 * u, rtol=1e-15)
    assert np.all(oracle.l2norm(np.zeros(8)) == 0.0)


# --------------------------------------------------------------- delta rule

def test_delta_rule_hand_example():
    rec = {}
    with open(os.path.join(GOLDEN, "delta_rule_hand.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, *vals = line.split()
                rec[name] = np.array([float(v) for v in vals])
    q, k, v = rec["q"].reshape(3, 2), rec["k"].reshape(3, 2), rec["v"].reshape(3, 2)
    o, S = oracle.delta_rule(q, k, v, np.log(rec["a"]), rec["b"], rec["S0"].reshape(2, 2))
    np.testing.assert_allclose(o.ravel(), rec["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S.ravel(), rec["S3"], rtol=0, atol=1e-14)


def test_delta_rule_pure_decay():
    """beta = 0: S_L = exp(sum g) S_0 and o_t = exp(sum_{s<=t} g_s) S_0^T q_t."""
    rng = _rng(5)
    dk, dv, L = 5, 3, 9
    q, k = rng.standard_normal((L, dk)), rng.standard_normal((L, dk))
    v = rng.standard_normal((L, dv))
    g = -rng.random(L)
    S0 = rng.standard_normal((dk, dv))
    o, S = oracle.delta_rule(q, k, v, g, np.zeros(L), S0)
    np.testing.assert_allclose(S, math.exp(g.sum()) * S0, rtol=1e-13)
    gam = np.cumsum(g)
    for t in range(L):
        np.testing.assert_allclose(o[t], math.exp(gam[t]) * (S0.T @ q[t]), rtol=1e-12, atol=1e-14)


def test_delta_rule_orthonormal_keys_store_values():
    """a = 1, b = 1, distinct orthonormal keys: S_L = (I - sum k k^T) S_0 + sum k v^T,
    so S_L^T k_j = v_j, and directions no key touched keep S_0."""
    rng = _rng(6)
    dk, dv, L = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :L].T                      # L orthonormal keys
    v = rng.standard_normal((L, dv))
    S0 = rng.standard_normal((dk, dv))
    q = rng.standard_normal((L, dk))
    o, S = oracle.delta_rule(q, keys, v, np.zeros(L), np.ones(L), S0)
    for j in range(L):
        np.testing.assert_allclose(S.T @ keys[j], v[j], rtol=1e-12, atol=1e-12)
    for u in Qm[:, L:].T:
        np.testing.assert_allclose(S.T @ u, S0.T @ u, rtol=1e-12, atol=1e-12)
    # o_t reads the state after token t: retrieving with q = k_t returns v_t
    o2, _ = oracle.delta_rule(keys, keys, v, np.zeros(L), np.ones(L), S0)
    np.testing.assert_allclose(o2, v, rtol=1e-12, atol=1e-12)


def test_delta_rule_single_step_interpolates():
    """One step with unit k: S_1^T k = a (1 - b) S_0^T k + b v; S_1^T u = a S_0^T u for u _|_ k."""
    rng = _rng(7)
    dk, dv = 6, 4
    for _ in range(5):
        k = rng.standard_normal(dk)
        k /= np.linalg.norm(k)
        v = rng.standard_normal(dv)
        S0 = rng.standard_normal((dk, dv))
        a, b = rng.random(), rng.random()
        u = rng.standard_normal(dk)
        u -= (u @ k) * k
        _, S = oracle.delta_rule(k[None], k[None], v[None], np.log([a]), np.array([b]), S0)
        np.testing.assert_allclose(S.T @ k, a * (1 - b) * (S0.T @ k) + b * v, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S.T @ u, a * (S0.T @ u), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("dk,dv", [(3, 2), (2, 3), (4, 4)])
def test_delta_rule_brute_force_matrix_form(dk, dv):
    """Brute force on tiny inputs: build the d_k x d_k transition matrix
    a (I - b k k^T) explicitly and multiply (keys need not be unit)."""
    rng = _rng(10 * dk + dv)
    L = 7
    q, k = rng.standard_normal((L, dk)), rng.standard_normal((L, dk))
    v = rng.standard_normal((L, dv))
    g, b = -rng.random(L), rng.random(L)
    S0 = rng.standard_normal((dk, dv))
    o, S = oracle.delta_rule(q, k, v, g, b, S0)
    Sref = S0.copy()
    for t in range(L):
        A = math.exp(g[t]) * (np.eye(dk) - b[t] * np.outer(k[t], k[t]))
        Sref = A @ Sref + b[t] * np.outer(k[t], v[t])
        np.testing.assert_allclose(o[t], Sref.T @ q[t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, Sref, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------- layer forward

def _run(batch, **kw):
    return oracle.forward(batch.layer, batch.x, batch.conv_weight, batch.g, batch.beta,
                          batch.cu_seqlens, batch.read_idx, batch.write_idx,
                          batch.conv_pool, batch.ssm_pool, **kw)


def _sub_batch(batch, s):
    """Sequence s of a packed batch as a batch of its own (same pools)."""
    cu = batch.cu_seqlens.tolist()
    r0, r1 = cu[s], cu[s + 1]
    return workloads.Batch(
        name="one", layer=batch.layer, x=batch.x[r0:r1].contiguous(),
        conv_weight=batch.conv_weight, g=batch.g[r0:r1].contiguous(),
        beta=batch.beta[r0:r1].contiguous(),
        cu_seqlens=torch.tensor([0, r1 - r0], dtype=torch.int32),
        read_idx=batch.read_idx[s:s + 1].clone(), write_idx=batch.write_idx[s:s + 1].clone(),
        conv_pool=batch.conv_pool, ssm_pool=batch.ssm_pool)


SMALL_BF16 = workloads.Layer(2, 4, 16, 8, 4, "bf16")


@pytest.mark.parametrize("which", ["cfg0", "bf16"])
def test_packed_equals_per_sequence(which):
    """Packing: the packed call equals one call per sequence, bit for bit, and
    blocks nobody writes are untouched; the trash block stays zero."""
    if which == "cfg0":
        b = workloads.config(0)
    else:
        b = workloads.random_batch(SMALL_BF16, [3, 1, 0, 12, 2], seed=11, fresh=[0, 1, 0, 0, 1])
    out, fin, cp, sp = _run(b)
    cu = b.cu_seqlens.tolist()
    for s in range(len(cu) - 1):
        one = _sub_batch(b, s)
        o1, f1, cp1, sp1 = _run(one)
        assert np.array_equal(out[cu[s]:cu[s + 1]], o1)
        assert np.array_equal(fin[s], f1[0])
        wb = int(b.write_idx[s])
        assert torch.equal(cp[wb], cp1[wb]) and torch.equal(sp[wb], sp1[wb])
    written = set(b.write_idx.tolist())
    for blk in range(b.ssm_pool.shape[0]):
        if blk not in written:
            assert torch.equal(cp[blk], b.conv_pool[blk]) and torch.equal(sp[blk], b.ssm_pool[blk])
    assert not cp[0].any() and not sp[0].any()


@pytest.mark.parametrize("split", [1, 2, 3, 7, 16])
def test_split_and_carry(split):
    """Checkpoint/resume: running a sequence in two calls, the second reading the
    block the first wrote, equals one pass (conv state bit-exact; outputs and
    recurrent state up to the fp32 rounding of the stored state)."""
    b = workloads.random_batch(SMALL_BF16, [17], seed=12)
    out, fin, cp, sp = _run(b)
    L = 17
    first = _sub_batch(b, 0)
    first.x, first.g, first.beta = b.x[:split].contiguous(), b.g[:split].contiguous(), b.beta[:split].contiguous()
    first.cu_seqlens = torch.tensor([0, split], dtype=torch.int32)
    o1, f1, cp1, sp1 = _run(first)
    second = _sub_batch(b, 0)
    second.x, second.g, second.beta = b.x[split:].contiguous(), b.g[split:].contiguous(), b.beta[split:].contiguous()
    second.cu_seqlens = torch.tensor([0, L - split], dtype=torch.int32)
    second.read_idx = b.write_idx.clone()
    second.conv_pool, second.ssm_pool = cp1, sp1
    o2, f2, cp2, sp2 = _run(second)
    wb = int(b.write_idx[0])
    assert torch.equal(cp2[wb], cp[wb])
    both = np.concatenate([o1, o2], axis=0)
    np.testing.assert_allclose(both, out, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(f2, fin, rtol=1e-5, atol=1e-7)


def test_trash_block_equals_zero_state():
    """A sequence with no past reads the zeroed trash block: same result as a
    block that holds zeros explicitly."""
    b = workloads.random_batch(SMALL_BF16, [6, 9], seed=13, fresh=[1, 1])
    out, fin, _, _ = _run(b)
    b2 = workloads.random_batch(SMALL_BF16, [6, 9], seed=13, fresh=[1, 1])
    spare = [blk for blk in range(1, b2.ssm_pool.shape[0]) if blk not in b2.write_idx.tolist()][0]
    b2.conv_pool[spare] = 0
    b2.ssm_pool[spare] = 0
    b2.read_idx = torch.tensor([spare, spare], dtype=torch.int32)
    out2, fin2, _, _ = _run(b2)
    assert np.array_equal(out, out2) and np.array_equal(fin, fin2)


def test_padding_sequence_untouched():
    b = workloads.random_batch(SMALL_BF16, [4, 3, 5], seed=14)
    b.write_idx[1] = -2
    out, fin, cp, sp = _run(b)
    assert np.isnan(out[4:7]).all()
    assert not np.isnan(out[:4]).any() and not np.isnan(out[7:]).any()


def test_layer_orthonormal_keys_recall_values():
    """Layer-level delta case: W = 1 with weight 1 (conv is SiLU), a = 1, b = 1,
    the k input of each token is 8 e_{pi(t)} with distinct pi(t), the q input
    equals the k input, and the state starts at zero (trash block).  Then
    k_hat_t = e_{pi(t)} up to eps, and o_t = S_t^T q_hat_t = SiLU(v_in_t) / sqrt(d_k):
    pins the [q|k|v] split, the normalisation, the q scale, the key head shared
    by G value heads, and that o_t reads the updated state."""
    layer = workloads.Layer(2, 4, 8, 3, 1, "f32")
    Hk, Hv, dk, dv = 2, 4, 8, 3
    C = layer.conv_channels
    L = 6
    rng = _rng(15)
    x = np.zeros((L, C), dtype=np.float32)
    perms = [rng.permutation(dk)[:L] for _ in range(Hk)]
    for h in range(Hk):
        for t in range(L):
            x[t, h * dk + perms[h][t]] = 8.0                 # q input
            x[t, Hk * dk + h * dk + perms[h][t]] = 8.0       # k input
    xv = rng.standard_normal((L, Hv * dv)).astype(np.float32)
    x[:, 2 * Hk * dk:] = xv
    b = workloads.Batch(
        name="delta", layer=layer, x=torch.from_numpy(x), conv_weight=torch.ones(C, 1),
        g=torch.zeros(L, Hv), beta=torch.ones(L, Hv),
        cu_seqlens=torch.tensor([0, L], dtype=torch.int32),
        read_idx=torch.tensor([0], dtype=torch.int32), write_idx=torch.tensor([1], dtype=torch.int32),
        conv_pool=torch.zeros(2, 0, C), ssm_pool=torch.zeros(2, Hv, dk, dv))
    out, fin, _, _ = _run(b)
    s8 = 8.0 / (1.0 + math.exp(-8.0))
    knorm2 = s8 * s8 / (s8 * s8 + 1e-6)
    silu_v = (xv / (1 + np.exp(-xv.astype(np.float64)))).reshape(L, Hv, dv)
    np.testing.assert_allclose(out, silu_v * knorm2 / math.sqrt(dk), rtol=1e-12, atol=1e-14)
    # the state holds exactly the stored pairs: S^T e_{pi(t)} = v_t (times |k_hat|)
    for m in range(Hv):
        h = m // (Hv // Hk)
        for t in range(L):
            np.testing.assert_allclose(fin[0, m].T[:, perms[h][t]],
                                       silu_v[t, m] * math.sqrt(knorm2), rtol=1e-12)


def test_layer_pure_decay():
    """beta = 0 at layer level: the state only decays, S_L = exp(sum g) S_0,
    and the conv state still advances."""
    b = workloads.random_batch(SMALL_BF16, [5, 11], seed=16)
    b.beta.zero_()
    out, fin, cp, sp = _run(b)
    cu = b.cu_seqlens.tolist()
    for s in range(2):
        decay = np.exp(b.g[cu[s]:cu[s + 1]].double().sum(0).numpy())  # [H_v]
        S0 = b.ssm_pool[int(b.read_idx[s])].double().numpy()
        np.testing.assert_allclose(fin[s], decay[:, None, None] * S0, rtol=1e-12, atol=1e-15)


def test_conv_state_is_last_inputs():
    """The new conv state is the last W-1 inputs of [old state; x], bit for bit,
    including sequences shorter than W-1 and the empty sequence."""
    b = workloads.random_batch(SMALL_BF16, [0, 1, 2, 3, 9], seed=17)
    _, _, cp, _ = _run(b)
    cu = b.cu_seqlens.tolist()
    for s in range(5):
        old = b.conv_pool[int(b.read_idx[s])]
        ext = torch.cat([old, b.x[cu[s]:cu[s + 1]]], dim=0)
        assert torch.equal(cp[int(b.write_idx[s])], ext[-3:])


def test_empty_sequence_is_identity():
    b = workloads.random_batch(SMALL_BF16, [0], seed=18)
    out, fin, cp, sp = _run(b)
    rb, wb = int(b.read_idx[0]), int(b.write_idx[0])
    assert torch.equal(sp[wb], b.ssm_pool[rb]) and torch.equal(cp[wb], b.conv_pool[rb])


# ------------------------------------------------------- standalone varlen conv

def _vc_batch(C, W, lengths, seed, dtype=torch.float32, P=6):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    x = torch.tensor(rng.standard_normal((T, C)), dtype=torch.float32).to(dtype)
    w = torch.tensor(rng.standard_normal((C, W)) / math.sqrt(W), dtype=torch.float32).to(dtype)
    pool = torch.tensor(rng.standard_normal((P, W - 1, C)), dtype=torch.float32).to(dtype)
    pool[0] = 0
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return x, w, pool, cu


def test_varlen_conv_hand_example():
    """W = 2, one channel: x = 1, 2, 3 after a state of 4, taps (0.5, 2)."""
    x = torch.tensor([[1.0], [2.0], [3.0]])
    w = torch.tensor([[0.5, 2.0]])
    pool = torch.tensor([[[0.0]], [[4.0]], [[9.0]]])
    y, new = oracle.varlen_conv(x, w, torch.tensor([0, 3], dtype=torch.int32), torch.tensor([1], dtype=torch.int32),
                                torch.tensor([2], dtype=torch.int32), pool, silu=False)
    assert y[:, 0].tolist() == [4.0, 4.5, 7.0]
    assert new[2, 0, 0].item() == 3.0 and new[1, 0, 0].item() == 4.0


def test_varlen_conv_silu_closed_form():
    """A single tap of 1 on x = ln 3 gives SiLU(ln 3) = 0.75 ln 3."""
    x = torch.tensor([[math.log(3.0)]], dtype=torch.float32)
    y, _ = oracle.varlen_conv(x, torch.tensor([[1.0]]), torch.tensor([0, 1], dtype=torch.int32),
                              torch.tensor([0], dtype=torch.int32), torch.tensor([1], dtype=torch.int32),
                              torch.zeros(2, 0, 1), silu=True)
    xv = float(x[0, 0])
    assert abs(y[0, 0] - 0.75 * math.log(3.0)) < 1e-6
    assert abs(y[0, 0] - xv / (1.0 + math.exp(-xv))) < 1e-12


@pytest.mark.parametrize("W", [1, 2, 4])
def test_varlen_conv_matches_numpy_correlate(W):
    """Each sequence and channel is numpy's valid cross-correlation of
    [state; x] with the taps; sequences continue from their own blocks."""
    C, lengths = 5, [7, 1, 12]
    x, w, pool, cu = _vc_batch(C, W, lengths, seed=61)
    ri = torch.tensor([3, 0, 5], dtype=torch.int32)
    wi = torch.tensor([3, 1, 2], dtype=torch.int32)
    y, new = oracle.varlen_conv(x, w, cu, ri, wi, pool, silu=False)
    for s in range(3):
        xs = x[cu[s]:cu[s + 1]].double().numpy()
        ext = np.concatenate([pool[ri[s]].double().numpy().reshape(W - 1, C), xs], axis=0)
        for c in range(C):
            ref = np.correlate(ext[:, c], w[c].double().numpy(), mode="valid")
            assert np.allclose(y[cu[s]:cu[s + 1], c], ref, rtol=1e-12, atol=1e-12)
        # new state: the last W-1 rows of [state; x], copied bit for bit
        exp_tail = torch.cat([pool[ri[s]], x[cu[s]:cu[s + 1]]], dim=0)[-(W - 1):] if W > 1 else pool[wi[s]]
        assert torch.equal(new[wi[s]], exp_tail.reshape(new[wi[s]].shape))


def test_varlen_conv_silu_equals_layer_conv():
    """With SiLU, every sequence equals the layer oracle's conv_silu on its rows."""
    C, W, lengths = 6, 4, [9, 3]
    x, w, pool, cu = _vc_batch(C, W, lengths, seed=62, dtype=torch.bfloat16)
    ri = torch.tensor([2, 4], dtype=torch.int32)
    y, _ = oracle.varlen_conv(x, w, cu, ri, torch.tensor([2, 4], dtype=torch.int32), pool, silu=True)
    for s in range(2):
        ref = oracle.conv_silu(pool[ri[s]].float().numpy(), x[cu[s]:cu[s + 1]].float().numpy(), w.float().numpy())
        assert np.array_equal(y[cu[s]:cu[s + 1]], ref)


def test_varlen_conv_short_sequence_shifts_state_and_padding_is_skipped():
    C, W = 3, 4
    x, w, pool, cu = _vc_batch(C, W, [1, 2], seed=63)
    ri = torch.tensor([1, 2], dtype=torch.int32)
    wi = torch.tensor([4, -1], dtype=torch.int32)
    y, new = oracle.varlen_conv(x, w, cu, ri, wi, pool, silu=False)
    # one token: the new state drops the oldest row and appends the token
    assert torch.equal(new[4], torch.cat([pool[1][1:], x[0:1]], dim=0))
    # padding: its rows untouched (NaN), and no block changes other than block 4
    assert np.isnan(y[1:3]).all()
    for b in range(6):
        if b != 4:
            assert torch.equal(new[b], pool[b])
