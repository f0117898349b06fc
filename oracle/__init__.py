"""fp64 CPU oracle for the TTT forward scan -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never loads it and the
two share no code.

The arithmetic lives in ``ttt_oracle.c`` (plain loops, fp64, OpenMP over the
independent (batch, head) chains); this module only compiles it with gcc and
marshals numpy arrays.  ``dual.py`` holds a second, independent formulation
(the chunked matrix "dual form") used by the oracle's own tests.

Parity status of each function (how it is pinned, see tests/test_oracle.py):
  linear_forward  -- pinned: hand-derived exact d=2 examples, eta=0, autograd
                     mini-batch GD, causal linear attention (W0=0), affine
                     chunk map, dual form, chaining, column separability.
  mlp_forward     -- pinned: eta=0, kernelised linear attention (W2_0=0),
                     autograd mini-batch GD, finite differences, dual form.
                     No exact worked example exists (SiLU is transcendental).
  linear_decode   -- pinned: n steps equal linear_forward with b=1.
  linear_forward_ex -- pinned: per-token eta equal to the head's eta gives
                     linear_forward; autograd mini-batch GD with per-token
                     step sizes; a zero step size drops a token from the
                     update; LayerNorm equals torch's layer_norm; the
                     chunk-start read is block-causal linear attention for
                     W0 = 0, online GD read before the update for b = 1, and
                     leaves W_out unchanged.
  linear_backward_ex -- pinned: equals linear_backward with the prologue off;
                     finite differences of linear_forward_ex in every
                     coordinate (q, k, v, W0, per-token eta, gamma, beta),
                     with and without the chunk-start read; torch autograd
                     of layer_norm for the LayerNorm part.
  linear_momentum -- pinned: a hand-worked d=2 example (tests/golden), the
                     heavy-ball closed form of the scalar recursion, beta=0
                     equal to linear_forward (b=1 for exact token steps, b for
                     chunk-start gradients), torch autograd gradients with
                     momentum steps, the chunk closed form of the momentum
                     sums (chunk-start gradients), and the triangular-solve
                     chunk form in dual.py (exact token steps).
  linear_backward -- pinned: central finite differences of linear_forward in
                     every coordinate (tiny sizes), the closed form of every
                     gradient at eta=0 (independent of b), the gradients of
                     causal linear attention (W0=0, one mini-batch), and the
                     chain rule across two calls (resume from W_out).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ttt_oracle.c")
_LIB = os.path.join(_HERE, "libttt_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ttt_oracle.c into libttt_oracle.so (gcc, -O2, OpenMP)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    L = ctypes.c_long
    I = ctypes.c_int
    lib.ttt_oracle_linear_forward.argtypes = [P, P, P, P, I, P, L, L, L, L, L, P, P, I]
    lib.ttt_oracle_linear_forward.restype = I
    lib.ttt_oracle_mlp_forward.argtypes = [P, P, P, P, P, I, P, L, L, L, L, L, L, P, P, P, I]
    lib.ttt_oracle_mlp_forward.restype = I
    lib.ttt_oracle_linear_decode.argtypes = [P, P, P, P, P, L, L, L, P]
    lib.ttt_oracle_linear_decode.restype = I
    lib.ttt_oracle_linear_backward.argtypes = [P, P, P, P, I, P, L, L, L, L, L, P, P,
                                               P, P, P, P, P, I]
    lib.ttt_oracle_linear_backward.restype = I
    lib.ttt_oracle_linear_forward_tok.argtypes = [P, P, P, P, I, P, I, L, L, L, L, L, P, P, I]
    lib.ttt_oracle_linear_forward_tok.restype = I
    lib.ttt_oracle_layernorm_rows.argtypes = [P, L, L, L, L, P, P, ctypes.c_double]
    lib.ttt_oracle_layernorm_rows.restype = I
    lib.ttt_oracle_linear_backward_tok.argtypes = [P, P, P, P, I, P, I, L, L, L, L, L, P, P,
                                                   P, P, P, P, P, I]
    lib.ttt_oracle_linear_backward_tok.restype = I
    lib.ttt_oracle_layernorm_rows_backward.argtypes = [P, P, L, L, L, L, P, ctypes.c_double, P]
    lib.ttt_oracle_layernorm_rows_backward.restype = I
    lib.ttt_oracle_linear_momentum.argtypes = [P, P, P, P, I, P, P, P, I, L, L, L, L, L,
                                               P, P, P, I]
    lib.ttt_oracle_linear_momentum.restype = I
    lib.ttt_oracle_max_threads.argtypes = []
    lib.ttt_oracle_max_threads.restype = I
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    """Exact upcast of an fp32/bf16/fp64 array (numpy or torch CPU) to fp64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().ttt_oracle_max_threads())


def linear_forward(Q, K, V, W0, eta, b: int, nthreads: int = 0):
    """Primal mini-batch GD, TTT-Linear.  Q,K,V [B,H,T,d]; W0 [H,d,d] or
    [B,H,d,d]; eta [H].  Returns (Y [B,H,T,d], W_out [B,H,d,d]) in fp64."""
    Q, K, V, W0, eta = map(_f64, (Q, K, V, W0, eta))
    B, H, T, d = Q.shape
    assert K.shape == Q.shape and V.shape == Q.shape
    per_batch = 1 if W0.ndim == 4 else 0
    assert W0.shape == ((B, H, d, d) if per_batch else (H, d, d))
    assert eta.shape == (H,)
    Y = np.zeros((B, H, T, d))
    W_out = np.zeros((B, H, d, d))
    rc = _load().ttt_oracle_linear_forward(_ptr(Q), _ptr(K), _ptr(V), _ptr(W0), per_batch,
                                           _ptr(eta), B, H, T, d, int(b), _ptr(Y),
                                           _ptr(W_out), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle linear_forward failed ({rc})")
    return Y, W_out


def layernorm(X, ln, eps: float):
    """LayerNorm of every d-vector of X [B,H,T,d] with the head's gamma, beta
    (ln [H,2,d]: gamma then beta), biased variance; fp64."""
    X = _f64(X).copy()
    ln = _f64(ln)
    B, H, T, d = X.shape
    assert ln.shape == (H, 2, d)
    gamma = np.ascontiguousarray(ln[:, 0])
    beta = np.ascontiguousarray(ln[:, 1])
    if X.size:
        rc = _load().ttt_oracle_layernorm_rows(_ptr(X), B * H * T, T, H, d, _ptr(gamma),
                                               _ptr(beta), float(eps))
        if rc != 0:
            raise RuntimeError(f"oracle layernorm failed ({rc})")
    return X


def linear_forward_ex(Q, K, V, W0, eta, b: int, eta_tok=None, ln_q=None, ln_k=None,
                      ln_eps: float = 1e-5, read_chunk_start: bool = False, nthreads: int = 0):
    """TTT-Linear with the input prologue: Q and K each LayerNorm'd over the
    head dim when ln_q / ln_k ([H,2,d], gamma then beta) are given, and a step
    size per token eta_tok [B,H,T] (else the head's eta).  read_chunk_start:
    every token reads out with its mini-batch's start weights.  Returns
    (Y, W_out) in fp64."""
    Q, K, V, W0, eta = map(_f64, (Q, K, V, W0, eta))
    B, H, T, d = Q.shape
    if ln_q is not None:
        Q = layernorm(Q, ln_q, ln_eps)
    if ln_k is not None:
        K = layernorm(K, ln_k, ln_eps)
    if eta_tok is None and not read_chunk_start:
        return linear_forward(Q, K, V, W0, eta, b, nthreads)
    et = _f64(eta_tok) if eta_tok is not None else np.broadcast_to(eta[None, :, None], (B, H, T)).copy()
    assert et.shape == (B, H, T)
    per_batch = 1 if W0.ndim == 4 else 0
    assert W0.shape == ((B, H, d, d) if per_batch else (H, d, d))
    Y = np.zeros((B, H, T, d))
    W_out = np.zeros((B, H, d, d))
    rc = _load().ttt_oracle_linear_forward_tok(_ptr(Q), _ptr(K), _ptr(V), _ptr(W0), per_batch,
                                               _ptr(et), int(bool(read_chunk_start)), B, H, T, d,
                                               int(b), _ptr(Y),
                                               _ptr(W_out), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle linear_forward_tok failed ({rc})")
    return Y, W_out


def linear_backward(Q, K, V, W0, eta, b: int, dY, dW_out, nthreads: int = 0):
    """Vector-Jacobian product of linear_forward: the gradients of
    <dY, Y> + <dW_out, W_out> with respect to Q, K, V, W0 and eta.
    dY [B,H,T,d]; dW_out [B,H,d,d].  Returns (dQ, dK, dV, dW0, deta) in fp64,
    dW0 shaped like W0 (summed over the batch when W0 is [H,d,d]) and deta [H]
    (summed over the batch)."""
    Q, K, V, W0, eta, dY, dW_out = map(_f64, (Q, K, V, W0, eta, dY, dW_out))
    B, H, T, d = Q.shape
    assert K.shape == Q.shape and V.shape == Q.shape and dY.shape == Q.shape
    per_batch = 1 if W0.ndim == 4 else 0
    assert W0.shape == ((B, H, d, d) if per_batch else (H, d, d))
    assert eta.shape == (H,) and dW_out.shape == (B, H, d, d)
    dQ = np.zeros((B, H, T, d))
    dK = np.zeros((B, H, T, d))
    dV = np.zeros((B, H, T, d))
    dW0c = np.zeros((B, H, d, d))
    detac = np.zeros((B, H))
    rc = _load().ttt_oracle_linear_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(W0), per_batch,
                                            _ptr(eta), B, H, T, d, int(b), _ptr(dY),
                                            _ptr(dW_out), _ptr(dQ), _ptr(dK), _ptr(dV),
                                            _ptr(dW0c), _ptr(detac), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle linear_backward failed ({rc})")
    dW0 = dW0c if per_batch else dW0c.sum(axis=0)
    return dQ, dK, dV, dW0, detac.sum(axis=0)


def linear_backward_ex(Q, K, V, W0, eta, b: int, dY, dW_out, eta_tok=None, ln_q=None,
                       ln_k=None, ln_eps: float = 1e-5, read_chunk_start: bool = False,
                       nthreads: int = 0):
    """Vector-Jacobian product of linear_forward_ex.  Returns a dict with dQ,
    dK, dV (of the raw inputs), dW0 (shaped like W0, summed over the batch
    when shared), deta [H] (head step sizes; zero when eta_tok is given),
    deta_tok [B,H,T] (when eta_tok is given), dln_q / dln_k [H,2,d] (when
    given)."""
    Q, K, V, W0, eta, dY, dW_out = map(_f64, (Q, K, V, W0, eta, dY, dW_out))
    B, H, T, d = Q.shape
    per_batch = 1 if W0.ndim == 4 else 0
    Qn = layernorm(Q, ln_q, ln_eps) if ln_q is not None else Q
    Kn = layernorm(K, ln_k, ln_eps) if ln_k is not None else K
    et = (_f64(eta_tok) if eta_tok is not None
          else np.ascontiguousarray(np.broadcast_to(eta[None, :, None], (B, H, T))))
    dQ = np.zeros((B, H, T, d))
    dK = np.zeros((B, H, T, d))
    dV = np.zeros((B, H, T, d))
    dW0c = np.zeros((B, H, d, d))
    detat = np.zeros((B, H, T))
    rc = _load().ttt_oracle_linear_backward_tok(_ptr(Qn), _ptr(Kn), _ptr(V), _ptr(W0), per_batch,
                                                _ptr(et), int(bool(read_chunk_start)), B, H, T,
                                                d, int(b), _ptr(dY), _ptr(dW_out), _ptr(dQ),
                                                _ptr(dK), _ptr(dV), _ptr(dW0c), _ptr(detat),
                                                int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle linear_backward_tok failed ({rc})")
    out = {"dV": dV, "dW0": dW0c if per_batch else dW0c.sum(axis=0)}
    for name, X, dX, ln in (("Q", Q, dQ, ln_q), ("K", K, dK, ln_k)):
        if ln is not None:
            ln = _f64(ln)
            dgb = np.zeros((H, 2, d))
            if X.size:
                rc = _load().ttt_oracle_layernorm_rows_backward(
                    _ptr(X), _ptr(dX), B * H * T, T, H, d, _ptr(np.ascontiguousarray(ln[:, 0])),
                    float(ln_eps), _ptr(dgb))
                if rc != 0:
                    raise RuntimeError(f"oracle layernorm backward failed ({rc})")
            out["dln_" + name.lower()] = dgb
        out["d" + name] = dX
    if eta_tok is None:
        out["deta"] = detat.sum(axis=(0, 2))
    else:
        out["deta"] = np.zeros(H)
        out["deta_tok"] = detat
    return out


def linear_momentum(Q, K, V, W0, eta, beta, b: int = 1, M0=None, grad_mode: int = 0,
                    nthreads: int = 0):
    """Momentum GD on TTT-Linear, token by token (E2-TTT write-up, "E2-TTT's
    Breakthrough").  grad_mode 0: exact token-level gradients at W_{t-1};
    1: gradients at the start of each chunk of b tokens.  W0 [H,d,d] or
    [B,H,d,d]; M0 None (zero) or [B,H,d,d]; eta, beta [H].
    Returns (Y [B,H,T,d], W_out, M_out [B,H,d,d]) in fp64."""
    Q, K, V, W0, eta, beta = map(_f64, (Q, K, V, W0, eta, beta))
    B, H, T, d = Q.shape
    assert K.shape == Q.shape and V.shape == Q.shape
    per_batch = 1 if W0.ndim == 4 else 0
    assert W0.shape == ((B, H, d, d) if per_batch else (H, d, d))
    assert eta.shape == (H,) and beta.shape == (H,)
    if M0 is not None:
        M0 = _f64(M0)
        assert M0.shape == (B, H, d, d)
    Y = np.zeros((B, H, T, d))
    W_out = np.zeros((B, H, d, d))
    M_out = np.zeros((B, H, d, d))
    rc = _load().ttt_oracle_linear_momentum(_ptr(Q), _ptr(K), _ptr(V), _ptr(W0), per_batch,
                                            None if M0 is None else _ptr(M0), _ptr(eta),
                                            _ptr(beta), int(grad_mode), B, H, T, d, int(b),
                                            _ptr(Y), _ptr(W_out), _ptr(M_out), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle linear_momentum failed ({rc})")
    return Y, W_out, M_out


def mlp_forward(Q, K, V, W1, W2, eta, b: int, nthreads: int = 0):
    """Primal mini-batch GD, TTT-MLP f(z)=SiLU(z W1) W2.  W1 [H,d,m] or
    [B,H,d,m]; W2 [H,m,d] or [B,H,m,d].  Returns (Y, W1_out, W2_out), fp64."""
    Q, K, V, W1, W2, eta = map(_f64, (Q, K, V, W1, W2, eta))
    B, H, T, d = Q.shape
    m = W1.shape[-1]
    per_batch = 1 if W1.ndim == 4 else 0
    lead = (B, H) if per_batch else (H,)
    assert W1.shape == lead + (d, m) and W2.shape == lead + (m, d)
    assert eta.shape == (H,)
    Y = np.zeros((B, H, T, d))
    W1o = np.zeros((B, H, d, m))
    W2o = np.zeros((B, H, m, d))
    rc = _load().ttt_oracle_mlp_forward(_ptr(Q), _ptr(K), _ptr(V), _ptr(W1), _ptr(W2),
                                        per_batch, _ptr(eta), B, H, T, d, m, int(b),
                                        _ptr(Y), _ptr(W1o), _ptr(W2o), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle mlp_forward failed ({rc})")
    return Y, W1o, W2o


def linear_decode(q, k, v, W, eta):
    """One online-GD token step for every (batch, head).  q,k,v [B,H,d];
    W [B,H,d,d].  Returns (y [B,H,d], W_new [B,H,d,d]); W is not modified."""
    q, k, v, eta = map(_f64, (q, k, v, eta))
    Wn = _f64(W).copy()
    B, H, d = q.shape
    assert Wn.shape == (B, H, d, d) and eta.shape == (H,)
    y = np.zeros((B, H, d))
    rc = _load().ttt_oracle_linear_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(Wn), _ptr(eta),
                                          B, H, d, _ptr(y))
    if rc != 0:
        raise RuntimeError(f"oracle linear_decode failed ({rc})")
    return y, Wn
