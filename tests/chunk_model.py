"""fp64 NumPy model of the chunked (WY / UT-transform) form of the gated delta
rule, test-side only.

The GPU prefill kernel evaluates the recurrence chunk by chunk in this form.
This model states the same algebra in plain matrix code so that its agreement
with the token-by-token oracle (tests/test_chunk_model.py) checks the
derivation itself, independently of any kernel.  Optionally it rounds the
matrix-product operands to bf16 where the GPU kernel does, to estimate the
error that rounding alone causes.

Derivation (state stored [d_k][d_v], gamma = in-chunk cumulative sum of g):
  delta form        S_t = a_t S_{t-1} + k_t u_t^T,  u_t = b_t (v_t - a_t S_{t-1}^T k_t)
  unrolled          S_t = e^{gamma_t} S_0 + sum_{j<=t} e^{gamma_t-gamma_j} k_j u_j^T
  linear system     (I + A) U = diag(b) V - diag(b e^{gamma}) K S_0,
                    A_tj = b_t e^{gamma_t-gamma_j} k_t.k_j  (j < t)
  so with T = (I + A)^-1:  U = T diag(b) V - T diag(b e^gamma) K S_0 = U~ - W S_0
  outputs           O = diag(e^gamma) Q S_0 + (M * Q K^T) U,  M_tj = e^{gamma_t-gamma_j} (j <= t)
  carried state     S_c = e^{gamma_c} S_0 + (diag(e^{gamma_c-gamma}) K)^T U
"""
import numpy as np
import torch


def _bf(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).double().numpy()


def chunked_delta_rule(q, k, v, g, beta, S0, chunk=64, bf16=False):
    r = _bf if bf16 else (lambda a: a)
    L, dk = q.shape
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((L, v.shape[1]))
    for n0 in range(0, L, chunk):
        n1 = min(n0 + chunk, L)
        Q, K, V = q[n0:n1], k[n0:n1], v[n0:n1]
        gam = np.cumsum(g[n0:n1])
        b = beta[n0:n1]
        n = n1 - n0
        D = gam[:, None] - gam[None, :]
        low = np.tril(np.ones((n, n), dtype=bool), -1)
        lowd = np.tril(np.ones((n, n), dtype=bool), 0)
        E = np.exp(np.where(lowd, D, 0.0))
        A = np.where(low, b[:, None] * E * (K @ K.T), 0.0)
        T = np.linalg.inv(np.eye(n) + A)
        W = r(T * (b * np.exp(gam))[None, :]) @ K
        Ut = r(T * b[None, :]) @ V
        U = Ut - r(W) @ r(S)
        P = np.where(lowd, E * (Q @ K.T), 0.0)
        o[n0:n1] = np.exp(gam)[:, None] * (Q @ r(S)) + r(P) @ r(U)
        S = np.exp(gam[-1]) * S + K.T @ r(np.exp(gam[-1] - gam)[:, None] * U)
    return o, S
