"""Seeded synthetic inputs for the TTT forward scan.

This module holds no arithmetic of the method: it only draws random numbers
with the shapes and distributions of the workloads and casts them.  Both the
HIP path and the fp64 oracle consume what it returns (the oracle upcasts the
already-cast values exactly), so the two sides see identical inputs.

Workloads (shapes follow the 124M/760M model shapes of the uTTT write-up on
thelatestinai.com, Table D1 -- head dim 64, 12 or 24 heads; mini-batch 16 as in
the dual-form section of "Test-Time Training Layers: How Inner-Loop Gradient
Descent Replaces the Transformer KV Cache ..."):

  1  TTT-Linear  B1  H1  d16 T64    b16 fp32  Q,K,V ~ N(0, 1/d)  W0 = 0          eta = 0.1
  2  TTT-Linear  B1  H4  d64 T2048  b16 fp32  Q,K,V ~ N(0, 1/d)  W0 ~ N(0, .02^2) eta = 1/d
  3  TTT-Linear  B8  H12 d64 T2048  b16 bf16  Q,K,V ~ N(0, 1/d)  W0 ~ N(0, .02^2) eta_h ~ U[.01, .1]
  4  TTT-Linear  B2  H24 d64 T32768 b16 bf16  as 3, plus 256 single-token decode steps
  5  TTT-MLP     B4  H12 d64 m256 T8192 b16 bf16  W1, W2 ~ N(0, .02^2)          eta = 0.05

Readings: N(0, 1/d) is a variance (std d^-1/2, so |k|^2 is about 1);
N(0, 0.02) is read as a standard deviation of 0.02.  Real workloads are
LayerNorm'd projections of language-model activations; iid Gaussians with
unit-norm keys stand in for them.

Backward cotangents (make_cotangents): dY ~ N(0, 1/d) in the input dtype and
dW_out ~ N(0, 1/d) fp32, from their own seed -- a stand-in for the gradient an
outer loss sends back into the layer.

Input prologue (make_prologue): LayerNorm gamma ~ U[0.8, 1.2] and beta ~
N(0, 0.1^2) per head for q and for k, and per-token step sizes
eta_t ~ U[0.1/d, 0.6/d] (LayerNorm'd keys have |k|^2 about d, so eta_t |k|^2
stays below 1 and each step contracts).

Momentum (make_momentum): a momentum coefficient per head beta_h ~ U[0, 0.9]
(the E2-TTT write-up names the coefficient but gives no value; 0.9 is the
largest, with 1/(1 - beta) = 10 the largest step amplification), optionally
a start momentum M0 ~ N(0, 0.02^2) per chain.

Generator: numpy.random.default_rng(seed), float32 standard normals scaled in
float32, then cast to the input dtype (bf16 by round-to-nearest-even through
torch).  Draw order: Q, K, V, initial state (W0, or W1 then W2), eta, then the
decode q, k, v.  Seed = 1000 + config number unless given.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    kind: str                 # "linear" or "mlp"
    B: int
    H: int
    T: int
    d: int
    b: int
    dtype: str                # "fp32" or "bf16" (Q/K/V/Y); state is always fp32
    w0: tuple = ("normal", 0.02)   # ("zero",) | ("normal", std) | ("eye",)
    eta: tuple = ("const", 0.1)    # ("const", v) | ("uniform", lo, hi)
    m: int = 0                # MLP hidden width
    decode_steps: int = 0
    name: str = ""
    extra: dict = field(default_factory=dict)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


WORKLOADS = {
    1: Workload("linear", B=1, H=1, T=64, d=16, b=16, dtype="fp32", w0=("zero",),
                eta=("const", 0.1), name="ttt_linear_B1_H1_d16_T64_b16_fp32"),
    2: Workload("linear", B=1, H=4, T=2048, d=64, b=16, dtype="fp32", w0=("normal", 0.02),
                eta=("const", 1.0 / 64), name="ttt_linear_B1_H4_d64_T2048_b16_fp32"),
    3: Workload("linear", B=8, H=12, T=2048, d=64, b=16, dtype="bf16", w0=("normal", 0.02),
                eta=("uniform", 0.01, 0.1), name="ttt_linear_B8_H12_d64_T2048_b16_bf16"),
    4: Workload("linear", B=2, H=24, T=32768, d=64, b=16, dtype="bf16", w0=("normal", 0.02),
                eta=("uniform", 0.01, 0.1), decode_steps=256,
                name="ttt_linear_B2_H24_d64_T32768_b16_bf16"),
    5: Workload("mlp", B=4, H=12, T=8192, d=64, m=256, b=16, dtype="bf16", w0=("normal", 0.02),
                eta=("const", 0.05), name="ttt_mlp_B4_H12_d64_m256_T8192_b16_bf16"),
}


def _normal(rng, shape, std):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(std)
    return x


def _state(rng, spec, shape):
    if spec[0] == "zero":
        return np.zeros(shape, np.float32)
    if spec[0] == "eye":
        out = np.zeros(shape, np.float32)
        n = min(shape[-2], shape[-1])
        out[..., np.arange(n), np.arange(n)] = 1.0
        return out
    if spec[0] == "normal":
        return _normal(rng, shape, spec[1])
    raise ValueError(f"unknown state spec {spec}")


def _eta(rng, spec, H):
    if spec[0] == "const":
        return np.full((H,), spec[1], np.float32)
    if spec[0] == "uniform":
        return rng.uniform(spec[1], spec[2], size=(H,)).astype(np.float32)
    raise ValueError(f"unknown eta spec {spec}")


def make_inputs(w: Workload, seed: int, device="cpu", w0_per_batch: bool = False) -> dict:
    """Draw one batch of inputs for workload ``w``.

    Returns a dict of torch tensors on ``device``: Q, K, V [B,H,T,d] in the
    input dtype; eta [H] fp32; for linear W0 [H,d,d] (or [B,H,d,d] with
    ``w0_per_batch``) fp32; for MLP W1 [H,d,m] and W2 [H,m,d] fp32; and, when
    ``w.decode_steps`` > 0, dq, dk, dv [steps,B,H,d] in the input dtype.
    """
    rng = np.random.default_rng(seed)
    std = 1.0 / math.sqrt(w.d)
    shp = (w.B, w.H, w.T, w.d)
    out = {}
    for name in ("Q", "K", "V"):
        out[name] = torch.from_numpy(_normal(rng, shp, std)).to(w.torch_dtype)
    lead = (w.B, w.H) if w0_per_batch else (w.H,)
    if w.kind == "linear":
        out["W0"] = torch.from_numpy(_state(rng, w.w0, lead + (w.d, w.d)))
    else:
        out["W1"] = torch.from_numpy(_state(rng, w.w0, lead + (w.d, w.m)))
        out["W2"] = torch.from_numpy(_state(rng, w.w0, lead + (w.m, w.d)))
    out["eta"] = torch.from_numpy(_eta(rng, w.eta, w.H))
    if w.decode_steps:
        dshp = (w.decode_steps, w.B, w.H, w.d)
        for name in ("dq", "dk", "dv"):
            out[name] = torch.from_numpy(_normal(rng, dshp, std)).to(w.torch_dtype)
    return {k: v.to(device) for k, v in out.items()}


def make_cotangents(w: Workload, seed: int, device="cpu", zero_state: bool = False) -> dict:
    """Seeded cotangents for the backward of a TTT-Linear workload: dY
    [B,H,T,d] in the input dtype and dW_out [B,H,d,d] fp32 (zeros with
    ``zero_state``, the case of a layer whose final state is not used)."""
    rng = np.random.default_rng(seed)
    std = 1.0 / math.sqrt(w.d)
    dY = torch.from_numpy(_normal(rng, (w.B, w.H, w.T, w.d), std)).to(w.torch_dtype)
    if zero_state:
        dWo = torch.zeros((w.B, w.H, w.d, w.d), dtype=torch.float32)
    else:
        dWo = torch.from_numpy(_normal(rng, (w.B, w.H, w.d, w.d), std))
    return {"dY": dY.to(device), "dW_out": dWo.to(device)}


def make_prologue(w: Workload, seed: int, device="cpu") -> dict:
    """Seeded prologue parameters for a TTT-Linear workload: ln_q, ln_k
    [H,2,d] fp32 (gamma row, beta row), eta_tok [B,H,T] fp32 and a head eta
    [H] on the same scale."""
    rng = np.random.default_rng(seed)
    out = {}
    for name in ("ln_q", "ln_k"):
        gamma = rng.uniform(0.8, 1.2, size=(w.H, w.d)).astype(np.float32)
        beta = _normal(rng, (w.H, w.d), 0.1)
        out[name] = torch.from_numpy(np.stack([gamma, beta], axis=1))
    lo, hi = 0.1 / w.d, 0.6 / w.d
    out["eta_tok"] = torch.from_numpy(rng.uniform(lo, hi, size=(w.B, w.H, w.T)).astype(np.float32))
    out["eta"] = torch.from_numpy(rng.uniform(lo, hi, size=(w.H,)).astype(np.float32))
    return {k: v.to(device) for k, v in out.items()}


def make_momentum(w: Workload, seed: int, device="cpu", m0: bool = False) -> dict:
    """Seeded momentum parameters for a TTT-Linear workload: beta [H] fp32
    and, with ``m0``, a start momentum M0 [B,H,d,d] fp32 (else None)."""
    rng = np.random.default_rng(seed)
    out = {"beta": torch.from_numpy(rng.uniform(0.0, 0.9, size=(w.H,)).astype(np.float32))}
    out["M0"] = torch.from_numpy(_normal(rng, (w.B, w.H, w.d, w.d), 0.02)) if m0 else None
    return {k: (v.to(device) if v is not None else None) for k, v in out.items()}


def default_seed(config: int) -> int:
    return 1000 + int(config)
