"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's own loops: each compares it with
something else -- hand-derived exact values, a library routine (numpy matmul,
torch autograd, torch's SiLU), a closed form, finite differences, or the
chunked dual form.  Together they are meant to catch a dropped term, a wrong
sign or index, or a transposed operand anywhere in the oracle.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import dual

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


def _linear_case(rng, B=2, H=3, T=37, d=8, per_batch=False, eta=None):
    Q = _rand(rng, B, H, T, d, scale=d ** -0.5)
    K = _rand(rng, B, H, T, d, scale=d ** -0.5)
    V = _rand(rng, B, H, T, d, scale=d ** -0.5)
    W0 = _rand(rng, *((B, H) if per_batch else (H,)), d, d, scale=0.1)
    if eta is None:
        eta = rng.uniform(0.05, 0.5, size=H)
    return Q, K, V, W0, np.asarray(eta, np.float64)


# --------------------------------------------------------------------------
# 1. hand-derived exact examples (tests/golden/linear_d2_worked.json)
# --------------------------------------------------------------------------
def _frac(x):
    return float(Fraction(x))


def test_worked_examples_exact(oracle):
    g = json.load(open(os.path.join(GOLDEN, "linear_d2_worked.json")))
    eta = _frac(g["eta"])
    k = np.array(g["k"], np.float64)
    v = np.array(g["v"], np.float64)
    q = np.array(g["q"], np.float64)
    for case in g["cases"]:
        T, b = case["T"], case["b"]
        W0 = np.zeros((1, 2, 2)) if case["W0"] == "0" else np.eye(2)[None]
        Y, W = oracle.linear_forward(q[None, None, :T], k[None, None, :T], v[None, None, :T],
                                     W0, np.array([eta]), b)
        Yx = np.array([[_frac(x) for x in r] for r in case["Y"]])
        Wx = np.array([[_frac(x) for x in r] for r in case["W"]])
        np.testing.assert_array_equal(Y[0, 0], Yx, err_msg=str(case))
        np.testing.assert_array_equal(W[0, 0], Wx, err_msg=str(case))


# --------------------------------------------------------------------------
# 2. eta = 0: the state never moves, Y = Q W0 (numpy matmul)
# --------------------------------------------------------------------------
def test_eta_zero_linear(oracle):
    rng = np.random.default_rng(1)
    Q, K, V, W0, _ = _linear_case(rng)
    Y, W = oracle.linear_forward(Q, K, V, W0, np.zeros(W0.shape[0]), 16)
    np.testing.assert_array_equal(W, np.broadcast_to(W0, W.shape))
    assert _rel(Y, Q @ W0[None]) < 1e-14


# --------------------------------------------------------------------------
# 3. mini-batch GD with the gradient from torch autograd
# --------------------------------------------------------------------------
def _autograd_linear_chain(q, k, v, w0, eta, b):
    q, k, v = (torch.tensor(a, dtype=torch.float64) for a in (q, k, v))
    W = torch.tensor(w0, dtype=torch.float64)
    T = q.shape[0]
    Y = torch.zeros_like(q)
    for s in range(0, T, b):
        e = min(s + b, T)
        Wc = W.clone().requires_grad_(True)
        for t in range(s, e):
            # summed half squared reconstruction error of tokens s..t at the chunk-start W
            loss = 0.5 * ((k[s:t + 1] @ Wc - v[s:t + 1]) ** 2).sum()
            (g,) = torch.autograd.grad(loss, Wc)
            Wt = Wc.detach() - eta * g
            Y[t] = q[t] @ Wt
        W = Wt
    return Y.numpy(), W.numpy()


@pytest.mark.parametrize("b", [1, 3, 4, 16, 64])
def test_autograd_minibatch_linear(oracle, b):
    rng = np.random.default_rng(2 + b)
    Q, K, V, W0, eta = _linear_case(rng, B=1, H=2, T=21, d=6)
    Y, W = oracle.linear_forward(Q, K, V, W0, eta, b)
    for h in range(2):
        Ya, Wa = _autograd_linear_chain(Q[0, h], K[0, h], V[0, h], W0[h], eta[h], b)
        assert _rel(Y[0, h], Ya) < 1e-12
        assert _rel(W[0, h], Wa) < 1e-12


# --------------------------------------------------------------------------
# 4. b = 1 is online GD in the pages' column form: predict v with W_col k,
#    error = prediction - v, gradient = error (outer) k, W_col -= lr * grad,
#    output = W_col q with the updated W_col.  W_row = W_col^T.
# --------------------------------------------------------------------------
def test_b1_is_online_gd_column_form(oracle):
    rng = np.random.default_rng(4)
    Q, K, V, W0, eta = _linear_case(rng, B=1, H=1, T=30, d=5)
    Wcol = W0[0].T.copy()
    ys = []
    for t in range(30):
        err = Wcol @ K[0, 0, t] - V[0, 0, t]
        Wcol = Wcol - eta[0] * np.outer(err, K[0, 0, t])
        ys.append(Wcol @ Q[0, 0, t])
    Y, W = oracle.linear_forward(Q, K, V, W0, eta, 1)
    assert _rel(Y[0, 0], np.array(ys)) < 1e-13
    assert _rel(W[0, 0], Wcol.T) < 1e-13


# --------------------------------------------------------------------------
# 5. W0 = 0 and one chunk: eta * causal linear attention (closed form)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,b", [(16, 16), (11, 16), (40, 16)])
def test_zero_init_is_causal_linear_attention(oracle, T, b):
    rng = np.random.default_rng(5)
    Q, K, V, _, eta = _linear_case(rng, B=1, H=2, T=T, d=7)
    W0 = np.zeros((2, 7, 7))
    Y, _ = oracle.linear_forward(Q, K, V, W0, eta, b)
    n = min(T, b)  # the first chunk starts from W = 0
    for h in range(2):
        q, k, v = Q[0, h, :n], K[0, h, :n], V[0, h, :n]
        # y_t = eta * sum_{i <= t} (q_t . k_i) v_i
        ref = np.zeros((n, 7))
        for t in range(n):
            for i in range(t + 1):
                ref[t] += eta[h] * np.dot(q[t], k[i]) * v[i]
        assert _rel(Y[0, h, :n], ref) < 1e-13


# --------------------------------------------------------------------------
# 6. one chunk is an affine map of W: W' = (I - eta K^T K) W + eta K^T V
# --------------------------------------------------------------------------
def test_chunk_is_affine_map(oracle):
    rng = np.random.default_rng(6)
    Q, K, V, W0, eta = _linear_case(rng, B=1, H=1, T=16, d=9)
    _, W = oracle.linear_forward(Q, K, V, W0, eta, 16)
    k, v = K[0, 0], V[0, 0]
    ref = (np.eye(9) - eta[0] * k.T @ k) @ W0[0] + eta[0] * k.T @ v
    assert _rel(W[0, 0], ref) < 1e-13


# --------------------------------------------------------------------------
# 7. primal (oracle) == chunked dual form, including a ragged last chunk
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,b", [(64, 16), (37, 16), (5, 16), (50, 8), (33, 1)])
def test_primal_equals_dual_linear(oracle, T, b):
    rng = np.random.default_rng(7 + T + b)
    Q, K, V, W0, eta = _linear_case(rng, B=2, H=2, T=T, d=8)
    Y, W = oracle.linear_forward(Q, K, V, W0, eta, b)
    Yd, Wd = dual.linear_dual(Q, K, V, W0, eta, b)
    assert _rel(Y, Yd) < 1e-12
    assert _rel(W, Wd) < 1e-12


# --------------------------------------------------------------------------
# 8. chaining: forward(T) == forward(T1) then forward(T2) from the final W
# --------------------------------------------------------------------------
def test_chaining_is_exact(oracle):
    rng = np.random.default_rng(8)
    Q, K, V, W0, eta = _linear_case(rng, B=2, H=2, T=48, d=8)
    Y, W = oracle.linear_forward(Q, K, V, W0, eta, 16)
    Y1, W1 = oracle.linear_forward(Q[:, :, :32], K[:, :, :32], V[:, :, :32], W0, eta, 16)
    Y2, W2 = oracle.linear_forward(Q[:, :, 32:], K[:, :, 32:], V[:, :, 32:], W1, eta, 16)
    np.testing.assert_array_equal(Y, np.concatenate([Y1, Y2], axis=2))
    np.testing.assert_array_equal(W, W2)


def test_per_batch_state_and_empty(oracle):
    rng = np.random.default_rng(9)
    Q, K, V, W0, eta = _linear_case(rng, B=3, H=2, T=20, d=4)
    Y, W = oracle.linear_forward(Q, K, V, W0, eta, 16)
    Yb, Wb = oracle.linear_forward(Q, K, V, np.broadcast_to(W0, (3, 2, 4, 4)), eta, 16)
    np.testing.assert_array_equal(Y, Yb)
    np.testing.assert_array_equal(W, Wb)
    # T = 0: the final state is the initial one
    Y0, W0o = oracle.linear_forward(Q[:, :, :0], K[:, :, :0], V[:, :, :0], W0, eta, 16)
    assert Y0.shape == (3, 2, 0, 4)
    np.testing.assert_array_equal(W0o, np.broadcast_to(W0, (3, 2, 4, 4)))


# --------------------------------------------------------------------------
# TTT-MLP
# --------------------------------------------------------------------------
def _mlp_case(rng, B=1, H=2, T=20, d=6, m=24, scale=0.3):
    Q = _rand(rng, B, H, T, d, scale=d ** -0.5)
    K = _rand(rng, B, H, T, d, scale=d ** -0.5)
    V = _rand(rng, B, H, T, d, scale=d ** -0.5)
    W1 = _rand(rng, H, d, m, scale=scale)
    W2 = _rand(rng, H, m, d, scale=scale)
    eta = rng.uniform(0.05, 0.5, size=H)
    return Q, K, V, W1, W2, eta


def _silu_np(x):
    return torch.nn.functional.silu(torch.tensor(x)).numpy()


def test_eta_zero_mlp(oracle):
    rng = np.random.default_rng(10)
    Q, K, V, W1, W2, _ = _mlp_case(rng)
    Y, W1o, W2o = oracle.mlp_forward(Q, K, V, W1, W2, np.zeros(2), 4)
    np.testing.assert_array_equal(W1o[0], W1)
    np.testing.assert_array_equal(W2o[0], W2)
    ref = _silu_np(Q @ W1[None]) @ W2[None]
    assert _rel(Y, ref) < 1e-14


def test_mlp_zero_second_layer_is_kernel_linear_attention(oracle):
    """W2_0 = 0: the first chunk reads out eta * sum_{i<=t} (a(q_t).a(k_i)) v_i
    with a(z) = SiLU(z W1_0), since the first layer gets no gradient."""
    rng = np.random.default_rng(11)
    Q, K, V, W1, W2, eta = _mlp_case(rng, T=16)
    W2 = np.zeros_like(W2)
    Y, W1o, _ = oracle.mlp_forward(Q, K, V, W1, W2, eta, 16)
    for h in range(2):
        aq = _silu_np(Q[0, h] @ W1[h])
        ak = _silu_np(K[0, h] @ W1[h])
        ref = eta[h] * np.tril(aq @ ak.T) @ V[0, h]
        assert _rel(Y[0, h], ref) < 1e-13
        np.testing.assert_array_equal(W1o[0, h], W1[h])


def _autograd_mlp_chain(q, k, v, w1, w2, eta, b):
    q, k, v = (torch.tensor(a, dtype=torch.float64) for a in (q, k, v))
    A1 = torch.tensor(w1, dtype=torch.float64)
    A2 = torch.tensor(w2, dtype=torch.float64)
    T = q.shape[0]
    Y = torch.zeros_like(q)
    F = torch.nn.functional
    for s in range(0, T, b):
        e = min(s + b, T)
        c1 = A1.clone().requires_grad_(True)
        c2 = A2.clone().requires_grad_(True)
        for t in range(s, e):
            loss = 0.5 * ((F.silu(k[s:t + 1] @ c1) @ c2 - v[s:t + 1]) ** 2).sum()
            g1, g2 = torch.autograd.grad(loss, (c1, c2))
            n1 = c1.detach() - eta * g1
            n2 = c2.detach() - eta * g2
            Y[t] = F.silu(q[t] @ n1) @ n2
        A1, A2 = n1, n2
    return Y.numpy(), A1.numpy(), A2.numpy()


@pytest.mark.parametrize("b", [1, 4, 16])
def test_autograd_minibatch_mlp(oracle, b):
    rng = np.random.default_rng(12 + b)
    Q, K, V, W1, W2, eta = _mlp_case(rng, T=19)
    Y, W1o, W2o = oracle.mlp_forward(Q, K, V, W1, W2, eta, b)
    for h in range(2):
        Ya, A1, A2 = _autograd_mlp_chain(Q[0, h], K[0, h], V[0, h], W1[h], W2[h], eta[h], b)
        assert _rel(Y[0, h], Ya) < 1e-12
        assert _rel(W1o[0, h], A1) < 1e-12
        assert _rel(W2o[0, h], A2) < 1e-12


def test_mlp_gradient_matches_finite_differences(oracle):
    """One token, b = 1: W_out = W - eta * grad, so grad = (W - W_out) / eta;
    compare with central differences of 1/2 ||SiLU(k W1) W2 - v||^2."""
    rng = np.random.default_rng(14)
    Q, K, V, W1, W2, _ = _mlp_case(rng, H=1, T=1, d=4, m=8, scale=0.7)
    eta = np.array([0.25])
    _, W1o, W2o = oracle.mlp_forward(Q, K, V, W1, W2, eta, 1)
    g1 = (W1[0] - W1o[0, 0]) / eta[0]
    g2 = (W2[0] - W2o[0, 0]) / eta[0]
    k, v = K[0, 0, 0], V[0, 0, 0]

    def loss(a1, a2):
        z = a1.T @ k
        a = z / (1.0 + np.exp(-z))
        return 0.5 * np.sum((a @ a2 - v) ** 2)

    h = 1e-6
    fd1 = np.zeros_like(g1)
    for i in range(4):
        for p in range(8):
            dp = np.zeros_like(W1[0]); dp[i, p] = h
            fd1[i, p] = (loss(W1[0] + dp, W2[0]) - loss(W1[0] - dp, W2[0])) / (2 * h)
    fd2 = np.zeros_like(g2)
    for p in range(8):
        for j in range(4):
            dp = np.zeros_like(W2[0]); dp[p, j] = h
            fd2[p, j] = (loss(W1[0], W2[0] + dp) - loss(W1[0], W2[0] - dp)) / (2 * h)
    assert _rel(g1, fd1) < 1e-7
    assert _rel(g2, fd2) < 1e-7


@pytest.mark.parametrize("T,b", [(32, 16), (21, 16), (12, 4)])
def test_primal_equals_dual_mlp(oracle, T, b):
    rng = np.random.default_rng(15 + T)
    Q, K, V, W1, W2, eta = _mlp_case(rng, B=2, T=T)
    Y, W1o, W2o = oracle.mlp_forward(Q, K, V, W1, W2, eta, b)
    Yd, W1d, W2d = dual.mlp_dual(Q, K, V, W1, W2, eta, b)
    assert _rel(Y, Yd) < 1e-12
    assert _rel(W1o, W1d) < 1e-12
    assert _rel(W2o, W2d) < 1e-12


# --------------------------------------------------------------------------
# decode: n single-token steps == the scan with b = 1 from the same state
# --------------------------------------------------------------------------
def test_decode_steps_equal_b1_scan(oracle):
    rng = np.random.default_rng(16)
    Q, K, V, Wb, eta = _linear_case(rng, B=2, H=3, T=9, d=6, per_batch=True)
    Y, W = oracle.linear_forward(Q, K, V, Wb, eta, 1)
    Wcur = Wb.copy()
    for t in range(9):
        y, Wcur = oracle.linear_decode(Q[:, :, t], K[:, :, t], V[:, :, t], Wcur, eta)
        np.testing.assert_array_equal(y, Y[:, :, t])
    np.testing.assert_array_equal(Wcur, W)


def test_decode_worked_example(oracle):
    """Token 2 of the hand-derived d=2 example, as one decode step from W1."""
    W1 = np.array([[[[0.5, 1.0], [0.0, 0.0]]]])
    y, W2 = oracle.linear_decode(np.array([[[1.0, 0.0]]]), np.array([[[1.0, 1.0]]]),
                                 np.array([[[3.0, -1.0]]]), W1, np.array([0.5]))
    np.testing.assert_array_equal(y[0, 0], [1.75, 0.0])
    np.testing.assert_array_equal(W2[0, 0], [[1.75, 0.0], [1.25, -1.0]])
