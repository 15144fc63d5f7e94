"""Chunkwise (UT-transform) form of the gated delta rule, numpy, float64.

TEST INFRASTRUCTURE ONLY: a cross-check of the algebra the GPU prefill uses,
never a path the product calls.

The pages ("cherenkov qwen4_exp/cpu.rs" fn deltanet, "oxinfer 0.0.5
src/qwen.rs" DeltaRule::run) give the recurrence one token at a time:

    S_t = a_t S_{t-1} + k_t d_t^T,   d_t = b_t (v_t - a_t S_{t-1}^T k_t),
    o_t = S_t^T q_t,                 a_t = exp(g_t).

Within a chunk that starts from state S_0, let G_i = g_1 + ... + g_i.
Unrolling gives S_{i} = e^{G_i} S_0 + sum_{j<=i} e^{G_i - G_j} k_j d_j^T,
hence

    d_i + sum_{j<i} b_i e^{G_i-G_j} (k_i.k_j) d_j = b_i v_i - b_i e^{G_i} S_0^T k_i

i.e. (I + A) D = diag(b) (V - diag(e^G) K S_0) with A strictly lower
triangular, A_ij = b_i e^{G_i - G_j} k_i.k_j.  With T = (I + A)^{-1}:

    D   = T diag(b) (V - diag(e^G) K S_0)
    O   = diag(e^G) Q S_0 + (M o Q K^T) D,   M_ij = e^{G_i-G_j} for j <= i
    S_C = e^{G_C} S_0 + (diag(e^{G_C - G}) K)^T D

Only differences G_i - G_j with j <= i are ever exponentiated, so nothing
overflows however strong the decay.  The triangular system is solved with a
library routine; there is no other blocking or fusion.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunked_core(q, k, v, g, beta, S0, chunk):
    """Same contract as ``oracle.delta_core``, computed chunk by chunk."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    S = np.array(S0, np.float64, copy=True)
    L = q.shape[0]
    o = np.zeros((L, v.shape[1]))
    for s in range(0, L, chunk):
        e = min(s + chunk, L)
        Q, K, V = q[s:e], k[s:e], v[s:e]
        b = beta[s:e]
        G = np.cumsum(g[s:e])
        diff = G[:, None] - G[None, :]
        lower = np.tril(np.ones((e - s, e - s), dtype=bool))
        M = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
        A = np.tril(b[:, None] * M * (K @ K.T), -1)
        rhs = b[:, None] * (V - np.exp(G)[:, None] * (K @ S))
        D = solve_triangular(np.eye(e - s) + A, rhs, lower=True,
                             unit_diagonal=True)
        o[s:e] = np.exp(G)[:, None] * (Q @ S) + (M * (Q @ K.T)) @ D
        S = np.exp(G[-1]) * S + (np.exp(G[-1] - G)[:, None] * K).T @ D
    return o, S
