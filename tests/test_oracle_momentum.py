"""Pins of the momentum oracle (oracle.linear_momentum) against what the pages
and the mathematics fix.

The method: the E2-TTT write-up on zhichai.net, section "E2-TTT's
Breakthrough: A Closed-Form Solution" -- gradient descent or momentum gradient
descent on the squared loss, fast weights W and momentum M, the chunk-end W and
M computed exactly -- with the learning rate and momentum coefficient of its
"Core Math (Simplified)" section.  grad_mode 0 takes every gradient at the
token's own current weights (exact token-level steps); grad_mode 1 at the start
of the token's chunk ("The Curse of Efficiency").

None of these re-types the oracle's loop: each compares it with hand-worked
values, an independent closed form, torch autograd, the existing mini-batch
oracle (itself pinned in test_oracle.py) or the chunked triangular-solve form
in oracle/dual.py.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import dual

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac(x):
    return float(Fraction(x))


def _mat(rows):
    return np.array([[_frac(x) for x in r] for r in rows])


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


def _case(rng, B=2, H=3, T=37, d=6, m0=True):
    s = d ** -0.5
    Q, K, V = (rng.standard_normal((B, H, T, d)) * s for _ in range(3))
    W0 = rng.standard_normal((H, d, d)) * 0.1
    M0 = rng.standard_normal((B, H, d, d)) * 0.1 if m0 else None
    eta = rng.uniform(0.05, 0.4, size=H)
    beta = np.linspace(0.0, 0.9, H)
    return Q, K, V, W0, M0, eta, beta


# --------------------------------------------------------------------------
# 1. hand-worked exact d = 2 examples (tests/golden/momentum_d2_worked.json)
# --------------------------------------------------------------------------
def test_momentum_worked_examples_exact(oracle):
    g = json.load(open(os.path.join(GOLDEN, "momentum_d2_worked.json")))
    eta, beta = _frac(g["eta"]), _frac(g["beta"])
    k, v, q = (np.array(g[x], np.float64)[None, None] for x in ("k", "v", "q"))
    for case in g["cases"]:
        Y, W, M = oracle.linear_momentum(q, k, v, np.zeros((1, 2, 2)), np.array([eta]),
                                         np.array([beta]), case["b"],
                                         _mat(case["M0"])[None, None], case["grad_mode"])
        np.testing.assert_array_equal(Y[0, 0], _mat(case["Y"]), err_msg=str(case))
        np.testing.assert_array_equal(W[0, 0], _mat(case["W"]), err_msg=str(case))
        np.testing.assert_array_equal(M[0, 0], _mat(case["M"]), err_msg=str(case))


# --------------------------------------------------------------------------
# 2. heavy-ball closed form.  With every key the unit vector e_0 only row 0 of
# W receives gradients, and column j of it follows the scalar recursion of momentum GD on
# 1/2 (w - v_j)^2: the error x_t = w_t - v_j obeys
#     x_t = (1 - eta + beta) x_{t-1} - beta x_{t-2},
# solved by x_t = A l1^t + B l2^t with l1, l2 the roots of
# l^2 - (1 - eta + beta) l + beta (complex roots included).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("eta,beta", [(0.3, 0.2), (0.1, 0.5), (0.5, 0.0), (0.05, 0.9)])
def test_heavy_ball_closed_form(oracle, eta, beta):
    rng = np.random.default_rng(3)
    d, T = 3, 40
    K = np.zeros((1, 1, T, d))
    K[..., 0] = 1.0
    vrow = rng.standard_normal(d)
    V = np.broadcast_to(vrow, (1, 1, T, d)).copy()
    Q = rng.standard_normal((1, 1, T, d))
    W0 = rng.standard_normal((1, d, d))
    M0 = rng.standard_normal((1, 1, d, d))
    Y, W, M = oracle.linear_momentum(Q, K, V, W0, np.array([eta]), np.array([beta]), 1, M0, 0)
    l1, l2 = np.roots([1.0, -(1.0 - eta + beta), beta]).astype(complex)
    Wt = np.empty((T + 1, d, d))
    for j in range(d):
        x0 = W0[0, 0, j] - vrow[j]
        x1 = x0 - eta * (beta * M0[0, 0, 0, j] + x0)
        if abs(l1 - l2) > 1e-12:
            A = (x1 - l2 * x0) / (l1 - l2)
            Bc = x0 - A
            xs = np.array([(A * l1 ** t + Bc * l2 ** t).real for t in range(T + 1)])
        else:  # repeated root: x_t = (A + B t) l^t
            Bc = x1 / l1 - x0
            xs = np.array([((x0 + Bc * t) * l1 ** t).real for t in range(T + 1)])
        Wt[:, 0, j] = xs + vrow[j]
    # rows 1.. see no gradient; their momentum decays as beta^t M0, so they move
    # by -eta (beta + ... + beta^t) M0 = -eta beta (1 - beta^t) / (1 - beta) M0
    c = np.array([beta * (1.0 - beta ** t) / (1.0 - beta) for t in range(T + 1)])
    Wt[:, 1:, :] = W0[0, 1:, :][None] - eta * c[:, None, None] * M0[0, 0, 1:][None]
    np.testing.assert_allclose(W[0, 0], Wt[T], rtol=0, atol=1e-12)
    Yx = np.einsum("ti,tij->tj", Q[0, 0], Wt[1:])
    np.testing.assert_allclose(Y[0, 0], Yx, rtol=0, atol=1e-12)
    # rows other than 0 of M only decay: beta^T M0
    np.testing.assert_allclose(M[0, 0, 1:], beta ** T * M0[0, 0, 1:], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# 3. beta = 0 reduces to the mini-batch oracle: b = 1 for exact token steps
# (online GD), b for chunk-start gradients.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("b", [1, 5, 16])
def test_beta_zero_exact_steps_is_online_gd(oracle, b):
    rng = np.random.default_rng(4)
    Q, K, V, W0, _, eta, _ = _case(rng)
    H = W0.shape[0]
    Y, W, M = oracle.linear_momentum(Q, K, V, W0, eta, np.zeros(H), b, None, 0)
    Yr, Wr = oracle.linear_forward(Q, K, V, W0, eta, 1)
    assert _rel(Y, Yr) < 1e-13 and _rel(W, Wr) < 1e-13
    # with beta = 0 the momentum is the last token's gradient: (W_{T-1} - W_T) / eta
    T = Q.shape[2]
    _, Wp = oracle.linear_forward(Q[:, :, :T - 1], K[:, :, :T - 1], V[:, :, :T - 1], W0, eta, 1)
    assert _rel(M, (Wp - W) / eta[None, :, None, None]) < 1e-10


@pytest.mark.parametrize("b", [1, 4, 16])
def test_beta_zero_chunk_start_is_minibatch(oracle, b):
    rng = np.random.default_rng(5)
    Q, K, V, W0, _, eta, _ = _case(rng)
    Y, W, _ = oracle.linear_momentum(Q, K, V, W0, eta, np.zeros(W0.shape[0]), b, None, 1)
    Yr, Wr = oracle.linear_forward(Q, K, V, W0, eta, b)
    assert _rel(Y, Yr) < 1e-13 and _rel(W, Wr) < 1e-13


# --------------------------------------------------------------------------
# 4. torch autograd: gradients of 1/2 ||k W - v||^2 from autograd, at the
# current weights or at the chunk start, fed through momentum steps.
# --------------------------------------------------------------------------
def _autograd_reference(Q, K, V, W0, M0, eta, beta, b, grad_mode):
    B, H, T, d = Q.shape
    Y = np.zeros((B, H, T, d))
    Wo = np.zeros((B, H, d, d))
    Mo = np.zeros((B, H, d, d))
    for bi in range(B):
        for h in range(H):
            W = torch.tensor(W0[h])
            M = torch.zeros(d, d, dtype=torch.float64) if M0 is None else torch.tensor(M0[bi, h])
            Wc = W
            for t in range(T):
                if t % b == 0:
                    Wc = W.clone()
                Wg = (Wc if grad_mode else W).clone().requires_grad_(True)
                k = torch.tensor(K[bi, h, t])
                v = torch.tensor(V[bi, h, t])
                loss = 0.5 * ((k @ Wg - v) ** 2).sum()
                (g,) = torch.autograd.grad(loss, Wg)
                M = beta[h] * M + g
                W = W - eta[h] * M
                Y[bi, h, t] = (torch.tensor(Q[bi, h, t]) @ W).numpy()
            Wo[bi, h] = W.numpy()
            Mo[bi, h] = M.numpy()
    return Y, Wo, Mo


@pytest.mark.parametrize("grad_mode,b", [(0, 1), (0, 6), (1, 6), (1, 1)])
def test_momentum_matches_autograd(oracle, grad_mode, b):
    rng = np.random.default_rng(6)
    Q, K, V, W0, M0, eta, beta = _case(rng, B=1, H=3, T=23, d=4)
    got = oracle.linear_momentum(Q, K, V, W0, eta, beta, b, M0, grad_mode)
    ref = _autograd_reference(Q, K, V, W0, M0, eta, beta, b, grad_mode)
    for a, r in zip(got, ref):
        assert _rel(a, r) < 1e-13


# --------------------------------------------------------------------------
# 5. the chunked closed form (oracle/dual.py): the triangular solve for exact
# token steps, the geometric momentum sums for chunk-start gradients.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("grad_mode", [0, 1])
@pytest.mark.parametrize("b", [1, 7, 16])
def test_momentum_matches_chunk_closed_form(oracle, grad_mode, b):
    rng = np.random.default_rng(7)
    Q, K, V, W0, M0, eta, beta = _case(rng, T=45)
    got = oracle.linear_momentum(Q, K, V, W0, eta, beta, b, M0, grad_mode)
    ref = dual.linear_momentum_dual(Q, K, V, W0, eta, beta, b, M0, grad_mode)
    for a, r in zip(got, ref):
        assert _rel(a, r) < 1e-12


# --------------------------------------------------------------------------
# 6. invariants: a call resumed from (W_out, M_out) continues the sequence;
# exact token steps do not depend on b.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("grad_mode", [0, 1])
def test_momentum_chaining(oracle, grad_mode):
    rng = np.random.default_rng(8)
    Q, K, V, W0, M0, eta, beta = _case(rng, T=48)
    b, cut = 8, 24            # the cut falls on a chunk boundary
    Y, W, M = oracle.linear_momentum(Q, K, V, W0, eta, beta, b, M0, grad_mode)
    Y1, W1, M1 = oracle.linear_momentum(Q[:, :, :cut], K[:, :, :cut], V[:, :, :cut], W0, eta,
                                        beta, b, M0, grad_mode)
    Y2, W2, M2 = oracle.linear_momentum(Q[:, :, cut:], K[:, :, cut:], V[:, :, cut:], W1, eta,
                                        beta, b, M1, grad_mode)
    assert _rel(np.concatenate([Y1, Y2], axis=2), Y) < 1e-13
    assert _rel(W2, W) < 1e-13 and _rel(M2, M) < 1e-13


def test_exact_steps_do_not_depend_on_b(oracle):
    rng = np.random.default_rng(9)
    Q, K, V, W0, M0, eta, beta = _case(rng)
    ref = oracle.linear_momentum(Q, K, V, W0, eta, beta, 1, M0, 0)
    for b in (3, 16, 64):
        got = oracle.linear_momentum(Q, K, V, W0, eta, beta, b, M0, 0)
        for a, r in zip(got, ref):
            np.testing.assert_array_equal(a, r)


def test_momentum_rejects_bad_arguments(oracle):
    rng = np.random.default_rng(10)
    Q, K, V, W0, M0, eta, beta = _case(rng, T=4)
    with pytest.raises(RuntimeError):
        oracle.linear_momentum(Q, K, V, W0, eta, beta, 0, M0, 0)
    with pytest.raises(RuntimeError):
        oracle.linear_momentum(Q, K, V, W0, eta, beta, 4, M0, 2)
