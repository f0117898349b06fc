"""Pins of the oracle's TTT-Linear backward (the vector-Jacobian product of the
forward scan) against things other than itself.

The backward is the gradient of L = <dY, Y> + <dW_out, W_out> with respect to
Q, K, V, W0 and eta, where (Y, W_out) is the forward scan of mini-batch
gradient descent.  Pins:
  1. central finite differences of the oracle's forward, every coordinate, on
     tiny inputs (shared and per-batch W0, a ragged last mini-batch);
  2. torch autograd through a forward whose inner gradient is itself taken by
     autograd (double backward): no hand-written derivative anywhere;
  3. the closed form of every gradient at eta = 0 (W never moves; the
     derivative in eta is -tril(Q K^T) (K W0 - V) over the whole sequence,
     whatever b is);
  4. the gradients of eta * causal linear attention (W0 = 0, one mini-batch);
  5. the chain rule across two calls (the second resumes from W_out);
  6. T = 0.
"""
import numpy as np
import pytest
import torch


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


def _case(rng, B, H, T, d, per_batch=False, w0_scale=0.3):
    Q = rng.standard_normal((B, H, T, d)) * d ** -0.5
    K = rng.standard_normal((B, H, T, d)) * d ** -0.5
    V = rng.standard_normal((B, H, T, d)) * d ** -0.5
    W0 = rng.standard_normal(((B, H) if per_batch else (H,)) + (d, d)) * w0_scale
    eta = rng.uniform(0.1, 0.6, size=H)
    dY = rng.standard_normal((B, H, T, d))
    dWo = rng.standard_normal((B, H, d, d))
    return Q, K, V, W0, eta, dY, dWo


def _loss(oracle, Q, K, V, W0, eta, b, dY, dWo):
    Y, Wo = oracle.linear_forward(Q, K, V, W0, eta, b)
    return float((Y * dY).sum() + (Wo * dWo).sum())


# --------------------------------------------------------------------------
# 1. finite differences, every coordinate
# --------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,T,d,b,per_batch", [(2, 2, 7, 3, 3, False), (2, 1, 5, 2, 2, True),
                                                  (1, 2, 6, 3, 1, False)])
def test_backward_matches_finite_differences(oracle, B, H, T, d, b, per_batch):
    rng = np.random.default_rng(100 + T + d + b)
    Q, K, V, W0, eta, dY, dWo = _case(rng, B, H, T, d, per_batch)
    grads = oracle.linear_backward(Q, K, V, W0, eta, b, dY, dWo)
    args = [Q, K, V, W0, eta]
    eps = 1e-6
    for ai, a in enumerate(args):
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            plus = [x.copy() for x in args]
            minus = [x.copy() for x in args]
            plus[ai][idx] += eps
            minus[ai][idx] -= eps
            fd[idx] = (_loss(oracle, *plus, b, dY, dWo) - _loss(oracle, *minus, b, dY, dWo)) / (2 * eps)
        assert grads[ai].shape == a.shape
        assert np.abs(fd - grads[ai]).max() < 1e-7 * (1.0 + np.abs(fd).max()), f"argument {ai}"


# --------------------------------------------------------------------------
# 2. torch autograd through a forward whose inner step is autograd's too
# --------------------------------------------------------------------------
def _autograd_outer(q, k, v, w0, eta, b, dy, dwo):
    q, k, v, w0, dy, dwo = (torch.tensor(a, dtype=torch.float64) for a in (q, k, v, w0, dy, dwo))
    q.requires_grad_(True)
    k.requires_grad_(True)
    v.requires_grad_(True)
    w0.requires_grad_(True)
    et = torch.tensor(float(eta), dtype=torch.float64, requires_grad=True)
    T = q.shape[0]
    W = w0
    ys = []
    for s in range(0, T, b):
        e = min(s + b, T)
        Wc = W
        for t in range(s, e):
            # gradient at the chunk-start W of the summed half squared error of tokens s..t
            loss = 0.5 * ((k[s:t + 1] @ Wc - v[s:t + 1]) ** 2).sum()
            (g,) = torch.autograd.grad(loss, Wc, create_graph=True)
            Wt = Wc - et * g
            ys.append(q[t] @ Wt)
        W = Wt
    L = (torch.stack(ys) * dy).sum() + (W * dwo).sum()
    gq, gk, gv, gw, ge = torch.autograd.grad(L, (q, k, v, w0, et))
    return [x.detach().numpy() for x in (gq, gk, gv, gw, ge)]


@pytest.mark.parametrize("b", [1, 4, 16])
def test_backward_matches_double_autograd(oracle, b):
    rng = np.random.default_rng(200 + b)
    Q, K, V, W0, eta, dY, dWo = _case(rng, 1, 2, 21, 6, per_batch=True)
    dQ, dK, dV, dW0, deta = oracle.linear_backward(Q, K, V, W0, eta, b, dY, dWo)
    for h in range(2):
        ref = _autograd_outer(Q[0, h], K[0, h], V[0, h], W0[0, h], eta[h], b, dY[0, h], dWo[0, h])
        assert _rel(dQ[0, h], ref[0]) < 1e-12
        assert _rel(dK[0, h], ref[1]) < 1e-12
        assert _rel(dV[0, h], ref[2]) < 1e-12
        assert _rel(dW0[0, h], ref[3]) < 1e-12
        assert abs(deta[h] - ref[4]) < 1e-12 * (1 + abs(ref[4]))


# --------------------------------------------------------------------------
# 3. eta = 0: closed form of every gradient, independent of b
# --------------------------------------------------------------------------
@pytest.mark.parametrize("b", [1, 4, 16, 64])
def test_backward_eta_zero_closed_form(oracle, b):
    rng = np.random.default_rng(300 + b)
    B, H, T, d = 2, 2, 37, 8
    Q, K, V, W0, _, dY, dWo = _case(rng, B, H, T, d)
    eta = np.zeros(H)
    dQ, dK, dV, dW0, deta = oracle.linear_backward(Q, K, V, W0, eta, b, dY, dWo)
    assert _rel(dQ, dY @ np.swapaxes(W0, -1, -2)[None]) < 1e-13
    np.testing.assert_array_equal(dK, 0.0)
    np.testing.assert_array_equal(dV, 0.0)
    ref_w = (np.swapaxes(Q, -1, -2) @ dY + dWo).sum(axis=0)
    assert _rel(dW0, ref_w) < 1e-13
    R = K @ W0[None] - V
    A = np.tril(Q @ np.swapaxes(K, -1, -2))
    ref_e = -(dY * (A @ R)).sum(axis=(0, 2, 3)) - (dWo * (np.swapaxes(K, -1, -2) @ R)).sum(axis=(0, 2, 3))
    assert _rel(deta, ref_e) < 1e-12


# --------------------------------------------------------------------------
# 4. W0 = 0, one mini-batch: Y = eta tril(Q K^T) V, W_out = eta K^T V
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,b", [(16, 16), (11, 16), (9, 9)])
def test_backward_linear_attention(oracle, T, b):
    rng = np.random.default_rng(400 + T)
    Q, K, V, _, eta, dY, dWo = _case(rng, 1, 2, T, 5)
    W0 = np.zeros((2, 5, 5))
    dQ, dK, dV, dW0, deta = oracle.linear_backward(Q, K, V, W0, eta, b, dY, dWo)
    for h in range(2):
        q, k, v, g, G, e = Q[0, h], K[0, h], V[0, h], dY[0, h], dWo[0, h], eta[h]
        A = np.tril(q @ k.T)
        M = np.tril(g @ v.T)
        assert _rel(dQ[0, h], e * M @ k) < 1e-13
        assert _rel(dK[0, h], e * M.T @ q + e * v @ G.T) < 1e-13
        assert _rel(dV[0, h], e * A.T @ g + e * k @ G) < 1e-13
        assert abs(deta[h] - ((g * (A @ v)).sum() + (G * (k.T @ v)).sum())) < 1e-12
        ref_w = q.T @ g - e * k.T @ A.T @ g + G - e * k.T @ k @ G
        assert _rel(dW0[h], ref_w) < 1e-13


# --------------------------------------------------------------------------
# 5. chain rule across two calls: the second call resumes from W_out
# --------------------------------------------------------------------------
def test_backward_chain_rule_across_calls(oracle):
    rng = np.random.default_rng(500)
    B, H, T1, T2, d, b = 2, 2, 16, 13, 6, 4
    Q, K, V, W0, eta, dY, dWo = _case(rng, B, H, T1 + T2, d, per_batch=True)
    full = oracle.linear_backward(Q, K, V, W0, eta, b, dY, dWo)
    s1, s2 = slice(0, T1), slice(T1, T1 + T2)
    _, Wmid = oracle.linear_forward(Q[:, :, s1], K[:, :, s1], V[:, :, s1], W0, eta, b)
    g2 = oracle.linear_backward(Q[:, :, s2], K[:, :, s2], V[:, :, s2], Wmid, eta, b, dY[:, :, s2], dWo)
    g1 = oracle.linear_backward(Q[:, :, s1], K[:, :, s1], V[:, :, s1], W0, eta, b, dY[:, :, s1], g2[3])
    for i in range(3):
        assert _rel(full[i], np.concatenate([g1[i], g2[i]], axis=2)) < 1e-12
    assert _rel(full[3], g1[3]) < 1e-12
    assert _rel(full[4], g1[4] + g2[4]) < 1e-12


def test_backward_empty_sequence(oracle):
    rng = np.random.default_rng(600)
    Q, K, V, W0, eta, dY, dWo = _case(rng, 3, 2, 0, 4)
    dQ, dK, dV, dW0, deta = oracle.linear_backward(Q, K, V, W0, eta, 16, dY, dWo)
    assert dQ.shape == (3, 2, 0, 4)
    np.testing.assert_array_equal(dW0, dWo.sum(axis=0))
    np.testing.assert_array_equal(deta, 0.0)
