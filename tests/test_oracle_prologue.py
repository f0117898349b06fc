"""Pins of the oracle's input prologue: LayerNorm of q and k, and a step size
per token.

The pages' layer listing LayerNorms the projected keys and queries before the
inner loop ("Test-Time Training Layers: How Inner-Loop Gradient Descent
Replaces the Transformer KV Cache ...", the TTT-Linear listing of section
"Hardware Parallelization"); the uTTT write-up on thelatestinai.com (Table
D3) gives the inner learning rate per token.  Pins: LayerNorm equals torch's
layer_norm; a per-token step size equal to the head's gives linear_forward;
mini-batch GD with per-token weights from torch autograd; tokens with a zero
step size leave the weights alone.
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


def _case(rng, B=2, H=3, T=37, d=8, per_batch=False):
    Q = rng.standard_normal((B, H, T, d)) * 0.7 + 0.2
    K = rng.standard_normal((B, H, T, d)) * 0.5 - 0.1
    V = rng.standard_normal((B, H, T, d)) * d ** -0.5
    W0 = rng.standard_normal(((B, H) if per_batch else (H,)) + (d, d)) * 0.1
    eta = rng.uniform(0.05, 0.3, size=H)
    ln = np.stack([rng.uniform(0.5, 1.5, size=(H, d)), rng.standard_normal((H, d)) * 0.1], axis=1)
    return Q, K, V, W0, eta, ln


def _torch_ln(X, ln, eps):
    X = torch.tensor(X, dtype=torch.float64)
    out = torch.empty_like(X)
    for h in range(X.shape[1]):
        out[:, h] = F.layer_norm(X[:, h], (X.shape[-1],), torch.tensor(ln[h, 0]),
                                 torch.tensor(ln[h, 1]), eps)
    return out.numpy()


@pytest.mark.parametrize("eps", [1e-5, 1e-2])
def test_layernorm_matches_torch(oracle, eps):
    rng = np.random.default_rng(800)
    Q, _, _, _, _, ln = _case(rng, B=2, H=3, T=11, d=16)
    Q[0, 1, 3] = 5.0                    # a constant row: variance 0, eps decides
    got = oracle.layernorm(Q, ln, eps)
    assert _rel(got, _torch_ln(Q, ln, eps)) < 1e-14


def test_prologue_is_layernorm_then_scan(oracle):
    rng = np.random.default_rng(801)
    Q, K, V, W0, eta, ln = _case(rng)
    ln_k = ln[:, ::-1].copy()
    Y, W = oracle.linear_forward_ex(Q, K, V, W0, eta, 16, ln_q=ln, ln_k=ln_k, ln_eps=1e-5)
    Yr, Wr = oracle.linear_forward(_torch_ln(Q, ln, 1e-5), _torch_ln(K, ln_k, 1e-5), V, W0, eta, 16)
    assert _rel(Y, Yr) < 1e-13 and _rel(W, Wr) < 1e-13


@pytest.mark.parametrize("b", [1, 4, 16])
def test_constant_token_eta_is_head_eta(oracle, b):
    rng = np.random.default_rng(802 + b)
    Q, K, V, W0, eta, _ = _case(rng, per_batch=True)
    et = np.broadcast_to(eta[None, :, None], Q.shape[:3]).copy()
    Y, W = oracle.linear_forward_ex(Q, K, V, W0, eta, b, eta_tok=et)
    Yr, Wr = oracle.linear_forward(Q, K, V, W0, eta, b)
    assert _rel(Y, Yr) < 1e-13 and _rel(W, Wr) < 1e-13


def _autograd_tok_chain(q, k, v, w0, et, b):
    q, k, v, et = (torch.tensor(a, dtype=torch.float64) for a in (q, k, v, et))
    W = torch.tensor(w0, dtype=torch.float64)
    T = q.shape[0]
    Y = torch.zeros_like(q)
    for s in range(0, T, b):
        e = min(s + b, T)
        Wc = W.clone().requires_grad_(True)
        for t in range(s, e):
            # per-token weighted half squared errors of tokens s..t at the chunk-start W
            loss = (0.5 * et[s:t + 1] * ((k[s:t + 1] @ Wc - v[s:t + 1]) ** 2).sum(-1)).sum()
            (g,) = torch.autograd.grad(loss, Wc)
            Wt = Wc.detach() - g
            Y[t] = q[t] @ Wt
        W = Wt
    return Y.numpy(), W.numpy()


@pytest.mark.parametrize("b", [1, 3, 16])
def test_token_eta_matches_autograd(oracle, b):
    rng = np.random.default_rng(803 + b)
    Q, K, V, W0, eta, _ = _case(rng, B=1, H=2, T=21, d=6)
    et = rng.uniform(0.0, 0.5, size=(1, 2, 21))
    Y, W = oracle.linear_forward_ex(Q, K, V, W0, eta, b, eta_tok=et)
    for h in range(2):
        Ya, Wa = _autograd_tok_chain(Q[0, h], K[0, h], V[0, h], W0[h], et[0, h], b)
        assert _rel(Y[0, h], Ya) < 1e-12
        assert _rel(W[0, h], Wa) < 1e-12


def test_zero_token_eta_freezes_the_state(oracle):
    rng = np.random.default_rng(804)
    Q, K, V, W0, eta, _ = _case(rng, B=2, H=2, T=40, d=5)
    et = rng.uniform(0.05, 0.3, size=(2, 2, 40))
    et[:, :, 16:] = 0.0                 # chunks 1 and 2 take no step
    Y, W = oracle.linear_forward_ex(Q, K, V, W0, eta, 16, eta_tok=et)
    Y1, W1 = oracle.linear_forward_ex(Q[:, :, :16], K[:, :, :16], V[:, :, :16], W0, eta, 16,
                                      eta_tok=et[:, :, :16])
    assert _rel(W, W1) < 1e-15
    assert _rel(Y[:, :, 16:], Q[:, :, 16:] @ W1) < 1e-13


# --------------------------------------------------------------------------
# chunk-start read (the uTTT write-up, Figure 2(a))
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,b", [(32, 16), (13, 8), (16, 16)])
def test_chunk_start_read_is_block_causal_linear_attention(oracle, T, b):
    # from W0 = 0 the weights of mini-batch 1 are eta K_0^T V_0 exactly, so
    # the first two mini-batches read block-causal linear attention
    rng = np.random.default_rng(810 + T + b)
    Q, K, V, _, eta, _ = _case(rng, B=1, H=2, T=T, d=6)
    W0 = np.zeros((2, 6, 6))
    Y, _ = oracle.linear_forward_ex(Q, K, V, W0, eta, b, read_chunk_start=True)
    for h in range(2):
        ref = np.zeros((T, 6))
        for t in range(T):
            for s in range(t - t % b):          # tokens of earlier mini-batches only
                ref[t] += eta[h] * np.dot(Q[0, h, t], K[0, h, s]) * V[0, h, s]
        assert _rel(Y[0, h], ref) < 1e-13


def test_chunk_start_read_b1_is_online_gd_read_before_update(oracle):
    rng = np.random.default_rng(820)
    Q, K, V, W0, eta, _ = _case(rng, B=1, H=1, T=25, d=5)
    Wcol = W0[0].T.copy()
    ys = []
    for t in range(25):
        ys.append(Wcol @ Q[0, 0, t])            # read with the weights before this token
        err = Wcol @ K[0, 0, t] - V[0, 0, t]
        Wcol = Wcol - eta[0] * np.outer(err, K[0, 0, t])
    Y, W = oracle.linear_forward_ex(Q, K, V, W0, eta, 1, read_chunk_start=True)
    assert _rel(Y[0, 0], np.array(ys)) < 1e-13
    assert _rel(W[0, 0], Wcol.T) < 1e-13


def test_chunk_start_read_keeps_the_state_recurrence(oracle):
    rng = np.random.default_rng(830)
    Q, K, V, W0, eta, _ = _case(rng, B=2, H=2, T=45, d=7)
    et = rng.uniform(0.05, 0.3, size=(2, 2, 45))
    _, W1 = oracle.linear_forward_ex(Q, K, V, W0, eta, 16, eta_tok=et, read_chunk_start=True)
    _, W2 = oracle.linear_forward_ex(Q, K, V, W0, eta, 16, eta_tok=et)
    np.testing.assert_array_equal(W1, W2)
