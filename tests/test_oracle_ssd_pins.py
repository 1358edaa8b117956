"""Pins of the Mamba2 scan oracle (oracle/ssd_oracle.py) to facts that do not
come from the oracle itself: the hand-worked scalar example in tests/golden/,
the quadratic dual form of the recurrence written as a masked matrix product
(Dao and Gu, "Transformers are SSMs", ICML 2024), its closed form without
decay, one token from the trash block, a sequence split over two calls, and the
padding and empty-sequence rules of the paged states (page "Continuous batching
for linear attention layers": one block per request, zeroed trash block).

A dropped D term, a decay applied one token early or late, B and C swapped,
dt_bias or softplus left out, or a state written to the wrong block fails one
of them.
"""
import math
import os

import numpy as np

from oracle import ssd_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(seed, lengths, H=4, P=3, N=5, G=2, pool_blocks=None, fresh=None):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    n = len(lengths)
    nb = pool_blocks or n + 2
    x = rng.standard_normal((T, H, P))
    dt = rng.standard_normal((T, H))
    A = -np.exp(rng.standard_normal(H) * 0.5)
    B = rng.standard_normal((T, G, N))
    C = rng.standard_normal((T, G, N))
    D = rng.standard_normal(H)
    bias = rng.standard_normal(H) * 0.3
    pool = rng.standard_normal((nb, H, P, N))
    pool[0] = 0
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    blocks = list(range(1, n + 1))
    fresh = fresh or [False] * n
    ri = np.array([0 if f else b for f, b in zip(fresh, blocks)])
    wi = np.array(blocks)
    return x, dt, A, B, C, D, bias, cu, ri, wi, pool


def test_hand_worked_scalar_example():
    vals = {}
    for line in open(os.path.join(GOLDEN, "ssd_scalar_hand.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            vals[k] = np.array([float(e) for e in v])
    T = len(vals["x"])
    x = vals["x"].reshape(T, 1, 1)
    dt = vals["dt"].reshape(T, 1)
    B = vals["B"].reshape(T, 1, 1)
    C = vals["C"].reshape(T, 1, 1)
    pool = np.zeros((2, 1, 1, 1))
    pool[1] = 4.0
    y, new = so.varlen_scan(x, dt, np.array([-math.log(2.0)]), B, C, np.array([0.5]), None,
                            [0, T], [1], [1], pool, dt_softplus=False)
    np.testing.assert_allclose(y[:, 0, 0], vals["y"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(new[1, 0, 0, 0], vals["h"][0], rtol=0, atol=1e-12)


def _dual_form(x, d, A, B, C, D, h0, grp):
    """y and the final state of one sequence from the quadratic form: with
    cumulative log decay lam_t = sum_{i<=t} d_i A,
    y_t = sum_{j<=t} e^{lam_t - lam_j} d_j (C_t . B_j) x_j + e^{lam_t} h0 C_t + D x_t and
    h_L = e^{lam_L} h0 + sum_j e^{lam_L - lam_j} d_j x_j B_j^T."""
    L, H, P = x.shape
    y = np.zeros((L, H, P))
    hL = np.zeros_like(h0)
    for m in range(H):
        lam = np.cumsum(d[:, m] * A[m])
        decay = np.tril(np.exp(lam[:, None] - lam[None, :]))
        Bm, Cm = B[:, grp[m], :], C[:, grp[m], :]
        M = decay * (Cm @ Bm.T) * d[None, :, m]
        y[:, m, :] = M @ x[:, m, :] + np.exp(lam)[:, None] * (Cm @ h0[m].T) + D[m] * x[:, m, :]
        w = np.exp(lam[-1] - lam) * d[:, m]
        hL[m] = math.exp(lam[-1]) * h0[m] + (x[:, m, :] * w[:, None]).T @ Bm
    return y, hL


def test_matches_the_quadratic_dual_form():
    x, dt, A, B, C, D, bias, cu, ri, wi, pool = _case(1, [7, 1, 12], fresh=[False, True, False])
    y, new = so.varlen_scan(x, dt, A, B, C, D, bias, cu, ri, wi, pool)
    grp = np.arange(4) // 2
    for s in range(3):
        r = slice(cu[s], cu[s + 1])
        d = so.softplus(dt[r] + bias)
        yd, hd = _dual_form(x[r], d, A, B[r], C[r], D, pool[ri[s]], grp)
        np.testing.assert_allclose(y[r], yd, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(new[wi[s]], hd, rtol=1e-10, atol=1e-10)


def test_no_decay_is_a_running_sum():
    """A = 0: h_t = h_0 + sum_{j<=t} d_j x_j B_j^T (cumulative sum)."""
    x, dt, A, B, C, D, bias, cu, ri, wi, pool = _case(2, [9])
    A = np.zeros_like(A)
    y, new = so.varlen_scan(x, dt, A, B, C, D, None, cu, ri, wi, pool)
    d = so.softplus(dt)
    grp = np.arange(4) // 2
    outer = (d[:, :, None] * x)[:, :, :, None] * B[:, grp, None, :]
    h = pool[ri[0]][None] + np.cumsum(outer, axis=0)
    np.testing.assert_allclose(y, np.einsum("thpn,thn->thp", h, C[:, grp]) + D[None, :, None] * x, atol=1e-10)
    np.testing.assert_allclose(new[wi[0]], h[-1], atol=1e-10)


def test_one_token_from_the_trash_block():
    """h_0 = 0: y = d (B . C) x + D x with d = softplus(dt + dt_bias); at dt + bias = 0, d = ln 2."""
    x, dt, A, B, C, D, bias, cu, ri, wi, pool = _case(3, [1], fresh=[True])
    dt = -bias[None, :].copy()
    y, new = so.varlen_scan(x, dt, A, B, C, D, bias, cu, ri, wi, pool)
    grp = np.arange(4) // 2
    bc = np.sum(B[0, grp] * C[0, grp], axis=1)
    np.testing.assert_allclose(y[0], math.log(2.0) * bc[:, None] * x[0] + D[:, None] * x[0], atol=1e-12)
    np.testing.assert_allclose(new[wi[0]], math.log(2.0) * x[0][:, :, None] * B[0, grp][:, None, :], atol=1e-12)


def test_split_over_two_calls():
    """Tokens [0, m) and then [m, L) from the state the first call wrote equal one call over [0, L)."""
    x, dt, A, B, C, D, bias, cu, ri, wi, pool = _case(4, [11])
    y, new = so.varlen_scan(x, dt, A, B, C, D, bias, cu, ri, wi, pool)
    m = 4
    y1, p1 = so.varlen_scan(x[:m], dt[:m], A, B[:m], C[:m], D, bias, [0, m], ri, [2], pool)
    y2, p2 = so.varlen_scan(x[m:], dt[m:], A, B[m:], C[m:], D, bias, [0, 11 - m], [2], wi, p1)
    np.testing.assert_allclose(np.concatenate([y1, y2]), y, atol=1e-10)
    np.testing.assert_allclose(p2[wi[0]], new[wi[0]], atol=1e-10)


def test_padding_and_empty_sequences():
    x, dt, A, B, C, D, bias, cu, ri, wi, pool = _case(5, [3, 0, 4])
    wi, ri = wi.copy(), ri.copy()
    wi[2] = -1
    ri[1] = 4  # the empty sequence starts from another block than it writes
    y, new = so.varlen_scan(x, dt, A, B, C, D, bias, cu, ri, wi, pool)
    assert np.all(y[3:7] == 0)                       # padding: no output rows
    np.testing.assert_array_equal(new[3], pool[3])   # nor its would-be block
    np.testing.assert_array_equal(new[wi[1]], pool[ri[1]])  # empty: the state is carried over
    np.testing.assert_array_equal(new[0], pool[0])   # the trash block is never written
