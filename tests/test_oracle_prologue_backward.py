"""Pins of the oracle's backward through the input prologue: a step size per
token, the chunk-start read, and LayerNorm of q and k.

The forward is the one the prologue pins fix (LayerNorm of the projected keys
and queries in the TTT-Linear listing of "Test-Time Training Layers: How
Inner-Loop Gradient Descent Replaces the Transformer KV Cache ...", section
"Hardware Parallelization"; the per-token inner learning rate of the uTTT
write-up on thelatestinai.com, Table D3, and its read-before-update of Figure
2(a)).  The backward is the gradient of L = <dY, Y> + <dW_out, W_out>.  Pins:
  1. with the prologue off it is the pinned linear_backward;
  2. central finite differences of linear_forward_ex in every coordinate
     (q, k, v, W0, per-token eta, gamma and beta of both LayerNorms), with and
     without the chunk-start read;
  3. torch autograd through torch's layer_norm and an inner step taken by
     autograd (no hand-written derivative);
  4. the per-token eta gradients of a chain sum to the head-eta gradient when
     every token carries the head's step size;
  5. T = 0.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


def _case(rng, B, H, T, d, per_batch=False):
    Q = rng.standard_normal((B, H, T, d)) * 0.8 + 0.3
    K = rng.standard_normal((B, H, T, d)) * 0.6 - 0.2
    V = rng.standard_normal((B, H, T, d)) * d ** -0.5
    W0 = rng.standard_normal(((B, H) if per_batch else (H,)) + (d, d)) * 0.3
    eta = rng.uniform(0.1, 0.5, size=H)
    et = rng.uniform(0.0, 0.4, size=(B, H, T))
    lq = np.stack([rng.uniform(0.6, 1.4, size=(H, d)), rng.standard_normal((H, d)) * 0.2], axis=1)
    lk = np.stack([rng.uniform(0.6, 1.4, size=(H, d)), rng.standard_normal((H, d)) * 0.2], axis=1)
    dY = rng.standard_normal((B, H, T, d))
    dWo = rng.standard_normal((B, H, d, d))
    return Q, K, V, W0, eta, et, lq, lk, dY, dWo


@pytest.mark.parametrize("B,H,T,b,per_batch", [(2, 3, 37, 16, False), (2, 2, 20, 1, True),
                                                (1, 2, 0, 4, False)])
def test_prologue_off_is_linear_backward(oracle, B, H, T, b, per_batch):
    rng = np.random.default_rng(900 + T + b)
    Q, K, V, W0, eta, _, _, _, dY, dWo = _case(rng, B, H, T, 5, per_batch)
    g = oracle.linear_backward_ex(Q, K, V, W0, eta, b, dY, dWo)
    ref = oracle.linear_backward(Q, K, V, W0, eta, b, dY, dWo)
    for n, r in zip(("dQ", "dK", "dV", "dW0", "deta"), ref):
        assert g[n].shape == r.shape
        assert _rel(g[n], r) < 1e-13, n


# --------------------------------------------------------------------------
# 2. finite differences, every coordinate
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,d,b,read_start,per_batch", [(7, 3, 3, False, False),
                                                         (7, 3, 3, True, True),
                                                         (5, 4, 1, True, False),
                                                         (6, 3, 6, False, True)])
def test_matches_finite_differences(oracle, T, d, b, read_start, per_batch):
    B, H = 2, 2
    rng = np.random.default_rng(910 + T + d + b + read_start)
    Q, K, V, W0, eta, et, lq, lk, dY, dWo = _case(rng, B, H, T, d, per_batch)
    g = oracle.linear_backward_ex(Q, K, V, W0, eta, b, dY, dWo, eta_tok=et, ln_q=lq, ln_k=lk,
                                  ln_eps=1e-3, read_chunk_start=read_start)
    args = {"Q": Q, "K": K, "V": V, "W0": W0, "eta_tok": et, "ln_q": lq, "ln_k": lk}

    def loss(a):
        Y, Wo = oracle.linear_forward_ex(a["Q"], a["K"], a["V"], a["W0"], eta, b,
                                         eta_tok=a["eta_tok"], ln_q=a["ln_q"], ln_k=a["ln_k"],
                                         ln_eps=1e-3, read_chunk_start=read_start)
        return float((Y * dY).sum() + (Wo * dWo).sum())

    grad_name = {"Q": "dQ", "K": "dK", "V": "dV", "W0": "dW0", "eta_tok": "deta_tok",
                 "ln_q": "dln_q", "ln_k": "dln_k"}
    eps = 1e-6
    for name, a in args.items():
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            p = {k: v.copy() for k, v in args.items()}
            m = {k: v.copy() for k, v in args.items()}
            p[name][idx] += eps
            m[name][idx] -= eps
            fd[idx] = (loss(p) - loss(m)) / (2 * eps)
        got = g[grad_name[name]]
        assert got.shape == a.shape, name
        assert np.abs(fd - got).max() < 1e-6 * (1.0 + np.abs(fd).max()), name
    assert np.array_equal(g["deta"], np.zeros(H))


# --------------------------------------------------------------------------
# 3. torch autograd: layer_norm from torch, inner gradient from autograd
# --------------------------------------------------------------------------
def _torch_chain(q, k, v, w0, et, lq, lk, eps, b, read_start):
    qn = F.layer_norm(q, (q.shape[-1],), lq[0], lq[1], eps)
    kn = F.layer_norm(k, (k.shape[-1],), lk[0], lk[1], eps)
    T = q.shape[0]
    W = w0
    ys = []
    for s in range(0, T, b):
        e = min(s + b, T)
        Wc = W
        for t in range(s, e):
            inner = (0.5 * et[s:t + 1] * ((kn[s:t + 1] @ Wc - v[s:t + 1]) ** 2).sum(-1)).sum()
            (gW,) = torch.autograd.grad(inner, Wc, create_graph=True)
            Wt = Wc - gW
            ys.append(qn[t] @ (Wc if read_start else Wt))
        W = Wt
    return torch.stack(ys), W


@pytest.mark.parametrize("b,read_start", [(4, False), (4, True), (16, False)])
def test_matches_torch_autograd(oracle, b, read_start):
    B, H, T, d = 1, 2, 23, 6
    rng = np.random.default_rng(930 + b + read_start)
    Q, K, V, W0, eta, et, lq, lk, dY, dWo = _case(rng, B, H, T, d)
    g = oracle.linear_backward_ex(Q, K, V, W0, eta, b, dY, dWo, eta_tok=et, ln_q=lq, ln_k=lk,
                                  ln_eps=1e-5, read_chunk_start=read_start)
    dlq = np.zeros_like(lq)
    dlk = np.zeros_like(lk)
    dW0 = np.zeros_like(W0)
    for h in range(H):
        t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True)
             for n, a in (("q", Q[0, h]), ("k", K[0, h]), ("v", V[0, h]), ("w0", W0[h]),
                          ("et", et[0, h]), ("lq", lq[h]), ("lk", lk[h]))}
        Y, Wo = _torch_chain(t["q"], t["k"], t["v"], t["w0"], t["et"], t["lq"], t["lk"], 1e-5, b,
                             read_start)
        L = (Y * torch.tensor(dY[0, h])).sum() + (Wo * torch.tensor(dWo[0, h])).sum()
        L.backward()
        assert _rel(g["dQ"][0, h], t["q"].grad.numpy()) < 1e-11
        assert _rel(g["dK"][0, h], t["k"].grad.numpy()) < 1e-11
        assert _rel(g["dV"][0, h], t["v"].grad.numpy()) < 1e-11
        assert _rel(g["deta_tok"][0, h], t["et"].grad.numpy()) < 1e-11
        dW0[h] = t["w0"].grad.numpy()
        dlq[h] = t["lq"].grad.numpy()
        dlk[h] = t["lk"].grad.numpy()
    assert _rel(g["dW0"], dW0) < 1e-11
    assert _rel(g["dln_q"], dlq) < 1e-11
    assert _rel(g["dln_k"], dlk) < 1e-11


# --------------------------------------------------------------------------
# 4. per-token gradients sum to the head's
# --------------------------------------------------------------------------
@pytest.mark.parametrize("read_start", [False, True])
def test_token_eta_gradients_sum_to_head_gradient(oracle, read_start):
    rng = np.random.default_rng(950 + read_start)
    Q, K, V, W0, eta, _, _, _, dY, dWo = _case(rng, 2, 3, 45, 5)
    et = np.ascontiguousarray(np.broadcast_to(eta[None, :, None], (2, 3, 45)))
    g = oracle.linear_backward_ex(Q, K, V, W0, eta, 16, dY, dWo, eta_tok=et,
                                  read_chunk_start=read_start)
    # the head-eta gradient by central differences of the forward
    eps = 1e-6
    for h in range(3):
        ep, em = eta.copy(), eta.copy()
        ep[h] += eps
        em[h] -= eps
        lp = sum(float((a * w).sum()) for a, w in zip(
            oracle.linear_forward_ex(Q, K, V, W0, ep, 16, read_chunk_start=read_start), (dY, dWo)))
        lm = sum(float((a * w).sum()) for a, w in zip(
            oracle.linear_forward_ex(Q, K, V, W0, em, 16, read_chunk_start=read_start), (dY, dWo)))
        fd = (lp - lm) / (2 * eps)
        assert abs(g["deta_tok"][:, h].sum() - fd) < 1e-6 * (1 + abs(fd))


def test_empty_sequence(oracle):
    rng = np.random.default_rng(960)
    Q, K, V, W0, eta, et, lq, lk, dY, dWo = _case(rng, 2, 3, 0, 4)
    g = oracle.linear_backward_ex(Q, K, V, W0, eta, 16, dY, dWo, eta_tok=et, ln_q=lq, ln_k=lk)
    assert g["dQ"].shape == (2, 3, 0, 4) and g["deta_tok"].shape == (2, 3, 0)
    assert np.array_equal(g["dW0"], dWo.sum(0))
    assert np.array_equal(g["dln_q"], np.zeros_like(lq))
