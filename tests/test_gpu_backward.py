"""GPU parity of ttt_linear_backward against the fp64 oracle's backward.

The same seeded inputs and cotangents go to both sides; every gradient (dQ,
dK, dV, dW0, deta) is compared element by element in relative L2: within 1e-4
for fp32 Q/K/V and 2e-2 for bf16 Q/K/V (whose dQ, dK, dV are rounded to
bf16).  Small cases span several chunks and a ragged tail; the benchmark
workloads run at full size with every chain (the 32768-token one with W0
given per batch, so dW0 is per chain).
"""
import numpy as np
import pytest
import torch

import oracle
import test_sequence_layers_linear_amd as ttt
from parity_util import WORKLOADS, TOL, announce, default_seed, make_inputs, rel_l2, to_gpu
from test_sequence_layers_linear_amd.inputs import make_cotangents

pytestmark = pytest.mark.gpu

NAMES = ("dQ", "dK", "dV", "dW0", "deta")


def _gpu(inp, cot, b):
    g = to_gpu(inp)
    c = to_gpu(cot)
    out = ttt.ttt_linear_backward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], b, c["dY"], c["dW_out"])
    torch.cuda.synchronize()
    return out


def _oracle(inp, cot, b):
    return oracle.linear_backward(inp["Q"], inp["K"], inp["V"], inp["W0"], inp["eta"], b,
                                  cot["dY"], cot["dW_out"])


def _compare(got, ref, tol, skip=()):
    errs = {}
    for n, x, r in zip(NAMES, got, ref):
        if n in skip:
            continue
        errs[n] = rel_l2(x, r)
    print("  rel-L2 " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,H,T,per_batch,zero_state", [
    (1, 2, 16, False, False),     # one chunk
    (2, 3, 37, False, False),     # ragged tail, W0 shared (dW0 summed over the batch)
    (2, 2, 200, True, False),     # many chunks, per-batch W0
    (1, 1, 1, False, False),      # a single token
    (3, 2, 96, False, True),      # final state unused (dW_out = 0)
])
def test_backward_small(dtype, B, H, T, per_batch, zero_state):
    w = WORKLOADS[3].with_(B=B, H=H, T=T, dtype=dtype, eta=("uniform", 0.1, 0.6))
    seed = 7000 + B * 100 + H * 10 + T
    announce("backward", dtype, B, H, T, "per_batch" if per_batch else "shared", seed)
    inp = make_inputs(w, seed, w0_per_batch=per_batch)
    cot = make_cotangents(w, seed + 1, zero_state=zero_state)
    _compare(_gpu(inp, cot, 16), _oracle(inp, cot, 16), TOL[dtype])


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,H,T,S,per_batch", [
    (1, 2, 100, 2, False),        # 7 chunks: segments of 4 and 3, ragged last chunk
    (2, 3, 333, 3, True),
    (1, 4, 1000, 7, False),
    (2, 1, 480, 30, False),       # 30 one-chunk segments
    (2, 2, 48, 3, True),          # 3 chunks, one per segment
])
def test_backward_segmented(dtype, B, H, T, S, per_batch, monkeypatch):
    monkeypatch.setenv("TTT_LINEAR_BWD_SEGMENTS", str(S))
    got_s = ttt.ttt_linear_backward_segments(B, H, T, 64, 16,
                                             torch.float32 if dtype == "fp32" else torch.bfloat16)
    assert got_s == S
    w = WORKLOADS[3].with_(B=B, H=H, T=T, dtype=dtype, eta=("uniform", 0.1, 0.6))
    seed = 7300 + B * 100 + H * 10 + S
    announce("backward segmented", dtype, B, H, T, "segments", S, seed)
    inp = make_inputs(w, seed, w0_per_batch=per_batch)
    cot = make_cotangents(w, seed + 1)
    _compare(_gpu(inp, cot, 16), _oracle(inp, cot, 16), TOL[dtype])


def test_backward_bf16_long_walk(monkeypatch):
    """bf16, one segment of 2048 chunks: sweep 2 walks the chunk-start states
    back from the last chunk through all of them (W_c = W_{c+1} - K_c^T E'_c),
    so any drift of that walk would show most here; whole tensors against the
    oracle."""
    monkeypatch.setenv("TTT_LINEAR_BWD_SEGMENTS", "1")
    w = WORKLOADS[4].with_(B=1, H=2)
    assert ttt.ttt_linear_backward_segments(w.B, w.H, w.T, w.d, w.b, w.torch_dtype) == 1
    seed = 7700
    announce("backward bf16 one long segment", w.name, seed)
    inp = make_inputs(w, seed, w0_per_batch=True)
    cot = make_cotangents(w, seed + 1)
    _compare(_gpu(inp, cot, w.b), _oracle(inp, cot, w.b), TOL["bf16"])


def test_backward_segmented_close_to_single_segment(monkeypatch):
    """fp32: a segmented backward is the same arithmetic in another rounding
    order of the state and the cotangent."""
    w = WORKLOADS[2]
    announce("backward segments vs one segment", w.name)
    inp = make_inputs(w, default_seed(2))
    cot = make_cotangents(w, default_seed(2) + 500)
    seg = _gpu(inp, cot, w.b)
    monkeypatch.setenv("TTT_LINEAR_BWD_SEGMENTS", "1")
    one = _gpu(inp, cot, w.b)
    for n, x, y in zip(NAMES, seg, one):
        e = rel_l2(x, y.detach().to("cpu", torch.float64).numpy())
        print(f"  {n} rel-L2 {e:.2e}", flush=True)
        assert e <= 2e-6, n


def test_backward_empty_sequence():
    w = WORKLOADS[3].with_(B=2, H=3, T=0)
    announce("backward T=0")
    inp = make_inputs(w, 7100)
    cot = make_cotangents(w, 7101)
    dQ, dK, dV, dW0, deta = _gpu(inp, cot, 16)
    assert dQ.shape == (2, 3, 0, 64)
    assert torch.equal(dW0.cpu(), cot["dW_out"].sum(0))
    assert torch.equal(deta.cpu(), torch.zeros(3))


def test_backward_deterministic():
    w = WORKLOADS[3].with_(B=2, H=4, T=300)
    announce("backward determinism")
    inp = to_gpu(make_inputs(w, 7200))
    cot = to_gpu(make_cotangents(w, 7201))
    a = ttt.ttt_linear_backward(inp["Q"], inp["K"], inp["V"], inp["W0"], inp["eta"], 16,
                                cot["dY"], cot["dW_out"])
    b = ttt.ttt_linear_backward(inp["Q"], inp["K"], inp["V"], inp["W0"], inp["eta"], 16,
                                cot["dY"], cot["dW_out"])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("cfg", [2, 3])
def test_backward_config_full(cfg):
    w = WORKLOADS[cfg]
    announce("backward config", cfg, w.name, "segments",
             ttt.ttt_linear_backward_segments(w.B, w.H, w.T, w.d, w.b, w.torch_dtype))
    inp = make_inputs(w, default_seed(cfg))
    cot = make_cotangents(w, default_seed(cfg) + 500)
    _compare(_gpu(inp, cot, w.b), _oracle(inp, cot, w.b), TOL[w.dtype])


def test_backward_config4_full():
    """The 32768-token workload's backward in its planned segments, W0 given
    per batch (dW0 per chain), every chain and every gradient (deta summed over
    the batch on both sides), relative L2 over the whole tensors."""
    w = WORKLOADS[4]
    announce("backward config 4, all chains", w.name, "segments",
             ttt.ttt_linear_backward_segments(w.B, w.H, w.T, w.d, w.b, w.torch_dtype))
    inp = make_inputs(w, default_seed(4), w0_per_batch=True)
    cot = make_cotangents(w, default_seed(4) + 500)
    got = _gpu(inp, cot, w.b)
    ref = _oracle(inp, cot, w.b)
    _compare(got, ref, TOL["bf16"])
