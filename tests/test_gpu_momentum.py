"""GPU parity of ttt_linear_momentum_forward against the fp64 oracle
(oracle.linear_momentum: momentum gradient descent token by token).

Relative-L2 comparison of Y, W_out and M_out on the same seeded inputs:
within 1e-4 for fp32 Q/K/V and 2e-2 for bf16 Q/K/V (fp32 state), for both
gradient points (exact token steps, chunk-start gradients).  Small cases span
several chunks and a ragged tail on both kernels (MFMA: bf16, d = 64, b = 16;
plain fp32 kernel: every other shape); the 96-chain and the 32768-token
workloads run at full size, every chain, in the launch configuration the
benchmark times.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import test_sequence_layers_linear_amd as ttt
from parity_util import (TOL, WORKLOADS, announce, cached_inputs, default_seed, make_inputs,
                         rel_l2, to_gpu)
from test_sequence_layers_linear_amd.inputs import make_momentum

pytestmark = pytest.mark.gpu


def _run(inp, mom, b, grad_mode, dtype, tol=None):
    tol = TOL[dtype] if tol is None else tol
    g = to_gpu(inp)
    M0 = None if mom["M0"] is None else mom["M0"].cuda()
    Y, W, M = ttt.ttt_linear_momentum_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"],
                                              mom["beta"].cuda(), b, M0, grad_mode)
    torch.cuda.synchronize()
    Yr, Wr, Mr = oracle.linear_momentum(inp["Q"], inp["K"], inp["V"], inp["W0"], inp["eta"],
                                        mom["beta"], b, mom["M0"], grad_mode)
    ey, ew, em = rel_l2(Y, Yr), rel_l2(W, Wr), rel_l2(M, Mr)
    print(f"  rel-L2 Y {ey:.3e}  W {ew:.3e}  M {em:.3e}", flush=True)
    assert ey <= tol and ew <= tol and em <= tol, (ey, ew, em)
    return Y, W, M


@pytest.mark.parametrize("grad_mode", [0, 1])
def test_momentum_config3_full(grad_mode):
    """B8 H12 T2048 bf16, d = 64, b = 16: all 96 chains, whole tensors."""
    w = WORKLOADS[3]
    announce("momentum config 3, all chains, grad_mode", grad_mode)
    inp = make_inputs(w, default_seed(3))
    _run(inp, make_momentum(w, 31), w.b, grad_mode, "bf16")


@pytest.mark.parametrize("grad_mode", [0, 1])
def test_momentum_config4_full(grad_mode):
    """B2 H24 T32768 bf16 in the launch configuration the benchmark times:
    all 48 chains, relative L2 over the whole Y, W_out and M_out tensors."""
    w = WORKLOADS[4]
    announce("momentum config 4, all chains, grad_mode", grad_mode)
    inp = cached_inputs(4, default_seed(4))
    _run(inp, make_momentum(w, 31), w.b, grad_mode, "bf16")


@pytest.mark.parametrize("grad_mode", [0, 1])
def test_momentum_config2_fp32(grad_mode):
    """B1 H4 T2048 fp32 on the plain fp32 kernel, within 1e-4."""
    w = WORKLOADS[2]
    announce("momentum config 2 fp32, grad_mode", grad_mode)
    _run(make_inputs(w, default_seed(2)), make_momentum(w, 32, m0=True), w.b, grad_mode, "fp32")


@pytest.mark.parametrize("grad_mode", [0, 1])
@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (1, 1, 5), (1, 1, 16), (1, 1, 17), (2, 3, 48),
                                   (1, 7, 257), (2, 2, 1000)])
def test_momentum_mfma_shapes(B, H, T, grad_mode):
    w = WORKLOADS[3].with_(B=B, H=H, T=T)
    announce("momentum mfma", B, H, T, grad_mode)
    _run(make_inputs(w, 40 + T), make_momentum(w, 41 + T, m0=T % 2 == 1), 16, grad_mode, "bf16")


@pytest.mark.parametrize("grad_mode", [0, 1])
@pytest.mark.parametrize("d,b,dtype", [(16, 16, "fp32"), (32, 7, "fp32"), (64, 16, "fp32"),
                                       (128, 16, "fp32"), (64, 1, "fp32"), (32, 64, "fp32"),
                                       (16, 16, "bf16"), (128, 16, "bf16"), (64, 8, "bf16"),
                                       (64, 32, "bf16")])
def test_momentum_generic_shapes(d, b, dtype, grad_mode):
    w = WORKLOADS[2].with_(B=2, H=3, T=3 * b + 5, d=d, b=b, dtype=dtype,
                           eta=("uniform", 0.01, 0.1))
    announce("momentum generic", d, b, dtype, grad_mode)
    _run(make_inputs(w, 200 + d + b), make_momentum(w, 201 + d, m0=True), b, grad_mode, dtype)


@pytest.mark.parametrize("cfg", [2, 3])
def test_beta_zero_chunk_start_matches_linear_forward(cfg):
    """beta = 0 with chunk-start gradients is the mini-batch scan of
    ttt_linear_forward: the two entry points agree within the tolerance."""
    w = WORKLOADS[cfg].with_(B=2, H=3, T=300)
    announce("momentum beta=0 vs linear forward", cfg)
    g = to_gpu(make_inputs(w, 50 + cfg))
    beta = torch.zeros(w.H, device="cuda")
    Y, W, _ = ttt.ttt_linear_momentum_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], beta,
                                              16, None, 1)
    Yl, Wl = ttt.ttt_linear_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], 16)
    torch.cuda.synchronize()
    tol = TOL[w.dtype]
    assert rel_l2(Y, Yl.double().cpu().numpy()) <= tol
    assert rel_l2(W, Wl.double().cpu().numpy()) <= tol


def test_momentum_empty_sequence_copies_state():
    w = WORKLOADS[3].with_(B=2, H=3, T=0)
    g = to_gpu(make_inputs(w, 5))
    mom = make_momentum(w, 6, m0=True)
    Y, W, M = ttt.ttt_linear_momentum_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"],
                                              mom["beta"].cuda(), 16, mom["M0"].cuda(), 0)
    torch.cuda.synchronize()
    assert Y.shape == (2, 3, 0, 64)
    assert torch.equal(W, g["W0"][None].expand(2, 3, 64, 64))
    assert torch.equal(M.cpu(), mom["M0"])
    _, _, Mz = ttt.ttt_linear_momentum_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"],
                                               mom["beta"].cuda(), 16, None, 0)
    torch.cuda.synchronize()
    assert not Mz.any()


@pytest.mark.parametrize("cfg,grad_mode", [(3, 0), (3, 1), (2, 0)])
def test_momentum_chaining_in_place(cfg, grad_mode):
    """Two calls that resume from (W_out, M_out), updated in place, continue
    the sequence: they match one call over all the tokens."""
    w = WORKLOADS[cfg].with_(B=2, H=3, T=320)
    announce("momentum chaining", cfg, grad_mode)
    inp = make_inputs(w, 60 + cfg, w0_per_batch=True)
    g = to_gpu(inp)
    beta = make_momentum(w, 61)["beta"].cuda()
    Y, W, M = ttt.ttt_linear_momentum_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], beta,
                                              16, None, grad_mode)
    Ws = g["W0"].clone()
    Ms = torch.zeros_like(Ws)
    Ys = []
    for lo, hi in ((0, 160), (160, 320)):
        sl = [x[:, :, lo:hi].contiguous() for x in (g["Q"], g["K"], g["V"])]
        Yp, _, _ = ttt.ttt_linear_momentum_forward(*sl, Ws, g["eta"], beta, 16, Ms, grad_mode,
                                                   W_out=Ws, M_out=Ms)
        Ys.append(Yp)
    torch.cuda.synchronize()
    tol = TOL[w.dtype]
    assert rel_l2(torch.cat(Ys, dim=2), Y.double().cpu().numpy()) <= tol
    assert rel_l2(Ws, W.double().cpu().numpy()) <= tol
    assert rel_l2(Ms, M.double().cpu().numpy()) <= tol


@pytest.mark.parametrize("path", ["generic_fp32", "mfma_bf16"])
def test_momentum_worked_examples_bit_exact(path):
    """The hand-worked d = 2 examples embedded by zero padding; every value
    is dyadic with few bits, so both kernels reproduce them exactly."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "momentum_d2_worked.json")))
    eta = torch.tensor([float(Fraction(g["eta"]))]).cuda()
    beta = torch.tensor([float(Fraction(g["beta"]))]).cuda()
    fr = lambda rows: torch.tensor([[float(Fraction(x)) for x in r] for r in rows])
    for case in g["cases"]:
        if path == "mfma_bf16":
            if case["grad_mode"] == 1 and case["b"] < 2:
                continue      # b = 16 covers both tokens in one chunk: only b >= T matches
            d, b, dtype = 64, 16, torch.bfloat16
        else:
            d, b, dtype = 16, case["b"], torch.float32

        def pad(rows):
            x = torch.zeros(1, 1, 2, d)
            x[0, 0, :, :2] = torch.tensor(rows, dtype=torch.float32)
            return x.to(dtype).cuda()
        M0 = torch.zeros(1, 1, d, d)
        M0[0, 0, :2, :2] = fr(case["M0"])
        Y, W, M = ttt.ttt_linear_momentum_forward(pad(g["q"]), pad(g["k"]), pad(g["v"]),
                                                  torch.zeros(1, d, d).cuda(), eta, beta, b,
                                                  M0.cuda(), case["grad_mode"])
        torch.cuda.synchronize()
        assert torch.equal(Y[0, 0, :, :2].float().cpu(), fr(case["Y"])), case
        assert torch.equal(W[0, 0, :2, :2].cpu(), fr(case["W"])), case
        assert torch.equal(M[0, 0, :2, :2].cpu(), fr(case["M"])), case
        assert not Y[0, 0, :, 2:].float().any() and not W[0, 0, 2:].any()


@pytest.mark.parametrize("S", [None, 5])
def test_momentum_graph_capture(S, monkeypatch):
    """Exact momentum steps (the inverse launch, then the scan; with S = 5
    forced segments also the maps and their composition) captured in a HIP
    graph with the caller's workspace: every replay equals the eager call bit
    for bit, with other eager work through the same workspace between the
    replays."""
    if S is not None:
        monkeypatch.setenv("TTT_MOMENTUM_SEGMENTS", str(S))
    w = WORKLOADS[3].with_(B=2, H=6, T=1000)
    announce("momentum graph capture, segments", S)
    if S is not None:
        assert ttt.ttt_linear_momentum_segments(w.B, w.H, w.T, 64, 16, torch.bfloat16, 0) == S
    g = to_gpu(make_inputs(w, 70))
    beta = make_momentum(w, 71)["beta"].cuda()
    nbytes = ttt.ttt_linear_momentum_workspace_bytes(w.B, w.H, w.T, 64, 16, torch.bfloat16, 0)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    Y_e, W_e, M_e = ttt.ttt_linear_momentum_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"],
                                                    beta, 16, None, 0, workspace=ws)
    torch.cuda.synchronize()
    Y, W, M = torch.empty_like(Y_e), torch.empty_like(W_e), torch.empty_like(M_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the launch path off the capture
        ttt.ttt_linear_momentum_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], beta, 16,
                                        None, 0, Y=Y, W_out=W, M_out=M, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ttt.ttt_linear_momentum_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], beta, 16,
                                        None, 0, Y=Y, W_out=W, M_out=M, workspace=ws)
    og = to_gpu(make_inputs(w.with_(B=1, H=4, T=700), 72))
    obeta = make_momentum(w.with_(H=4), 73)["beta"].cuda()
    for rep in range(3):
        Y.zero_()
        W.zero_()
        M.zero_()
        ws.fill_(0xff)
        ttt.ttt_linear_momentum_forward(og["Q"], og["K"], og["V"], og["W0"], og["eta"], obeta,
                                        16, None, 0, workspace=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_e) and torch.equal(W, W_e) and torch.equal(M, M_e), rep


@pytest.mark.parametrize("grad_mode", [0, 1])
@pytest.mark.parametrize("S,T", [(2, 33), (2, 48), (2, 64), (2, 1000), (3, 333), (5, 1000),
                                 (12, 1000)])
def test_momentum_forced_segments(S, T, grad_mode, monkeypatch):
    """Sequence segments of the MFMA scan (maps of [W; M], their composition,
    segment scans) against the oracle, forced to S segments of whole stages of
    32 tokens, with a ragged last segment (down to one token, T = 33, or one
    chunk, T = 48), a start momentum and one head with beta = 0 (whose scan
    does not carry M)."""
    monkeypatch.setenv("TTT_MOMENTUM_SEGMENTS", str(S))
    w = WORKLOADS[3].with_(B=2, H=3, T=T)
    announce("momentum segments", S, T, grad_mode)
    stages = -(-T // 32)
    want = -(-stages // -(-stages // S))       # segments of ceil(stages / S) stages
    assert ttt.ttt_linear_momentum_segments(w.B, w.H, w.T, w.d, w.b, torch.bfloat16,
                                            grad_mode) == want
    mom = make_momentum(w, 50 + S, m0=True)
    mom["beta"][1] = 0.0
    _run(make_inputs(w, 51 + T), mom, 16, grad_mode, "bf16")


@pytest.mark.parametrize("grad_mode", [0, 1])
def test_momentum_segments_in_place_chaining(grad_mode, monkeypatch):
    """Segmented calls with per-batch W0 updated in place (W_out = W0,
    M_out = M0): two calls over halves of a sequence equal one call over the
    whole (both segmented), up to rounding."""
    monkeypatch.setenv("TTT_MOMENTUM_SEGMENTS", "3")
    w = WORKLOADS[3].with_(B=1, H=2, T=512)
    announce("momentum segments in place", grad_mode)
    inp = make_inputs(w, 61, w0_per_batch=True)
    mom = make_momentum(w, 62, m0=True)
    g = to_gpu(inp)
    beta = mom["beta"].cuda()
    Y1, W1, M1 = ttt.ttt_linear_momentum_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], beta,
                                                 16, mom["M0"].cuda(), grad_mode)
    W = g["W0"].clone()
    M = mom["M0"].cuda().clone()
    half = w.T // 2
    ys = []
    for sl in (slice(0, half), slice(half, w.T)):
        q, k, v = (g[n][:, :, sl].contiguous() for n in ("Q", "K", "V"))
        y, _, _ = ttt.ttt_linear_momentum_forward(q, k, v, W, g["eta"], beta, 16, M, grad_mode,
                                                  W_out=W, M_out=M)
        ys.append(y)
    torch.cuda.synchronize()
    Y2 = torch.cat(ys, dim=2)
    for a, b in ((Y1, Y2), (W1, W), (M1, M)):
        r = float((a.float() - b.float()).norm() / b.float().norm())
        assert r <= 1e-2, r
