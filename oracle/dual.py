"""Chunked "dual form" of the TTT scan in fp64 numpy -- TEST INFRASTRUCTURE ONLY.

A second formulation of the same mini-batch gradient descent that the C
oracle computes token by token.  It is used only by the oracle's own tests,
to check the primal loops against the equivalence the pages state
("Test-Time Training Layers: How Inner-Loop Gradient Descent Replaces the
Transformer KV Cache ...", section "Hardware Parallelization: The Dual Form and
Mini-Batch GPU Acceleration": the chunk's inner-loop operations rewritten as
matrix products; the ren-xubin.github.io essay, paragraph on the dual form:
accumulated gradients substituted into the output without materialising every
intermediate W_t).

TTT-Linear, one chunk (rows = tokens, row-vector form z W):
    E      = K W - V                      residual at the chunk-start W
    Y      = Q W - eta * tril(Q K^T) E    tril keeps the diagonal: token t reads
                                          out after its own update
    W_next = W - eta * K^T E

TTT-Linear with momentum (the E2-TTT write-up on zhichai.net, sections
"E2-TTT's Breakthrough" and "Core Math": the chunk-end W and M computed in
closed form from the chunk-start W_k, M_k).  Token t of a chunk (0-based)
sees the weights after the chunk's first t tokens,
    W_(t) = W - eta c_t M - eta sum_{u<t} dsum_{t-1-u} k_u^T r_u,
    c_t = beta + ... + beta^t,   dsum_m = 1 + beta + ... + beta^m,
so with E = K W - V the exact token-level residuals solve the unit lower
triangular system
    (I + eta A) R = E - eta diag(c_t) K M,   A[t, u] = dsum_{t-1-u} (k_t . k_u), u < t
(with gradients at the chunk start instead, R = E), and then
    Y      = Q W - eta diag(c_{t+1}) Q M - eta (tril(Q K^T) o Dsum) R,
             Dsum[t, u] = dsum_{t-u}
    W_next = W - eta c_n M - eta K^T diag(dsum_{n-1-u}) R
    M_next = beta^n M + K^T diag(beta^{n-1-u}) R.
This is a derivation of this module, not a formula printed on the page.

TTT-MLP f(z) = SiLU(z W1) W2, one chunk, all gradients at the chunk start:
    Hk = K W1, Ak = SiLU(Hk), E = Ak W2 - V
    D  = (E W2^T) * SiLU'(Hk)
    Hq = Q W1 - eta * tril(Q K^T) D,   Aq = SiLU(Hq)
    Y  = Aq W2 - eta * tril(Aq Ak^T) E
    W1_next = W1 - eta K^T D,   W2_next = W2 - eta Ak^T E
"""
from __future__ import annotations

import numpy as np


def _silu(x):
    return x / (1.0 + np.exp(-x))


def _silu_grad(x):
    s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def linear_dual(Q, K, V, W0, eta, b):
    Q, K, V, W0, eta = (np.asarray(a, dtype=np.float64) for a in (Q, K, V, W0, eta))
    B, H, T, d = Q.shape
    Y = np.zeros_like(Q)
    W_out = np.zeros((B, H, d, d))
    for bi in range(B):
        for h in range(H):
            W = (W0[bi, h] if W0.ndim == 4 else W0[h]).copy()
            for s in range(0, T, b):
                e = min(s + b, T)
                Qc, Kc, Vc = Q[bi, h, s:e], K[bi, h, s:e], V[bi, h, s:e]
                E = Kc @ W - Vc
                Y[bi, h, s:e] = Qc @ W - eta[h] * np.tril(Qc @ Kc.T) @ E
                W = W - eta[h] * Kc.T @ E
            W_out[bi, h] = W
    return Y, W_out


def linear_momentum_dual(Q, K, V, W0, eta, beta, b, M0=None, grad_mode=0):
    Q, K, V, W0, eta, beta = (np.asarray(a, dtype=np.float64)
                              for a in (Q, K, V, W0, eta, beta))
    B, H, T, d = Q.shape
    Y = np.zeros_like(Q)
    W_out = np.zeros((B, H, d, d))
    M_out = np.zeros((B, H, d, d))
    for bi in range(B):
        for h in range(H):
            W = (W0[bi, h] if W0.ndim == 4 else W0[h]).copy()
            M = np.zeros((d, d)) if M0 is None else np.asarray(M0, np.float64)[bi, h].copy()
            bt, et = beta[h], eta[h]
            for s in range(0, T, b):
                e = min(s + b, T)
                n = e - s
                Qc, Kc, Vc = Q[bi, h, s:e], K[bi, h, s:e], V[bi, h, s:e]
                pw = bt ** np.arange(n + 1)                 # beta^0 .. beta^n
                c = np.concatenate([[0.0], np.cumsum(pw[1:])])   # c_0 .. c_n
                dsum = np.cumsum(pw)                        # dsum_0 .. dsum_n
                idx = np.arange(n)
                lag = idx[:, None] - idx[None, :]           # t - u
                E = Kc @ W - Vc
                if grad_mode == 0:
                    A = np.where(lag > 0, dsum[np.maximum(lag - 1, 0)], 0.0) * (Kc @ Kc.T)
                    rhs = E - et * c[:n, None] * (Kc @ M)
                    R = np.linalg.solve(np.eye(n) + et * A, rhs)
                else:
                    R = E
                S = np.where(lag >= 0, dsum[np.maximum(lag, 0)], 0.0) * (Qc @ Kc.T)
                Y[bi, h, s:e] = Qc @ W - et * c[1:, None] * (Qc @ M) - et * S @ R
                W = W - et * c[n] * M - et * Kc.T @ (dsum[n - 1 - idx][:, None] * R)
                M = pw[n] * M + Kc.T @ (pw[n - 1 - idx][:, None] * R)
            W_out[bi, h] = W
            M_out[bi, h] = M
    return Y, W_out, M_out


def mlp_dual(Q, K, V, W1, W2, eta, b):
    Q, K, V, W1, W2, eta = (np.asarray(a, dtype=np.float64) for a in (Q, K, V, W1, W2, eta))
    B, H, T, d = Q.shape
    m = W1.shape[-1]
    Y = np.zeros_like(Q)
    W1o = np.zeros((B, H, d, m))
    W2o = np.zeros((B, H, m, d))
    for bi in range(B):
        for h in range(H):
            A1 = (W1[bi, h] if W1.ndim == 4 else W1[h]).copy()
            A2 = (W2[bi, h] if W2.ndim == 4 else W2[h]).copy()
            for s in range(0, T, b):
                e = min(s + b, T)
                Qc, Kc, Vc = Q[bi, h, s:e], K[bi, h, s:e], V[bi, h, s:e]
                Hk = Kc @ A1
                Ak = _silu(Hk)
                E = Ak @ A2 - Vc
                D = (E @ A2.T) * _silu_grad(Hk)
                Hq = Qc @ A1 - eta[h] * np.tril(Qc @ Kc.T) @ D
                Aq = _silu(Hq)
                Y[bi, h, s:e] = Aq @ A2 - eta[h] * np.tril(Aq @ Ak.T) @ E
                A1 = A1 - eta[h] * Kc.T @ D
                A2 = A2 - eta[h] * Ak.T @ E
            W1o[bi, h] = A1
            W2o[bi, h] = A2
    return Y, W1o, W2o
