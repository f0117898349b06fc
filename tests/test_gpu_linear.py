"""GPU parity of ttt_linear_forward against the fp64 oracle.

Element-by-element relative-L2 comparison on the same seeded inputs: within
1e-4 for fp32 Q/K/V and 2e-2 for bf16 Q/K/V (fp32 state), for Y and for the
final W.  Small cases span several chunks and a ragged tail; the benchmark
workloads run at full size, every chain, with the relative L2 taken over the
whole tensor.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import test_sequence_layers_linear_amd as ttt
from parity_util import (WORKLOADS, TOL, announce, cached_inputs, default_seed, linear_gpu,
                         linear_oracle, make_inputs, per_chain_rel_l2, rel_l2, to_gpu)

pytestmark = pytest.mark.gpu


def _check(inp, b, dtype, tol=None):
    tol = TOL[dtype] if tol is None else tol
    Y, W = linear_gpu(to_gpu(inp), b)
    Yr, Wr = linear_oracle(inp, b)
    ey, ew = rel_l2(Y, Yr), rel_l2(W, Wr)
    print(f"  rel-L2 Y {ey:.3e}  W {ew:.3e}", flush=True)
    assert ey <= tol and ew <= tol, (ey, ew)
    return Y, W


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_config_full(cfg):
    w = WORKLOADS[cfg]
    announce("linear config", cfg, w.name)
    inp = make_inputs(w, default_seed(cfg))
    _check(inp, w.b, w.dtype)


def test_config4_full():
    """The 32768-token workload in the launch configuration the benchmark
    times (the planned segments: maps, composition, segment scans), all 48
    chains against the oracle, relative L2 over the whole Y and W tensors."""
    w = WORKLOADS[4]
    announce("linear config 4, all chains", w.name, "segments",
             ttt.ttt_linear_segments(w.B, w.H, w.T, w.d, w.b, torch.bfloat16))
    inp = cached_inputs(4, default_seed(4))
    Y, W = linear_gpu(to_gpu(inp), w.b)
    Yr, Wr = linear_oracle(inp, w.b)
    ey, ew = rel_l2(Y, Yr), rel_l2(W, Wr)
    cy, cw = per_chain_rel_l2(Y, Yr), per_chain_rel_l2(W, Wr)
    print(f"  rel-L2 Y {ey:.3e}  W {ew:.3e}  (worst chain: Y {cy.max():.3e}, W {cw.max():.3e})",
          flush=True)
    assert ey <= TOL["bf16"] and ew <= TOL["bf16"]


# ---------------------------------------------------------------------------
# edge cases on the MFMA path (bf16, d = 64, b = 16) and the generic path
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (1, 1, 5), (1, 1, 16), (1, 1, 17), (1, 3, 31),
                                   (2, 3, 48), (3, 1, 100), (1, 7, 257), (2, 2, 1000)])
def test_mfma_shapes(B, H, T):
    w = WORKLOADS[3].with_(B=B, H=H, T=T)
    announce("linear mfma", B, H, T)
    _check(make_inputs(w, 7 + T), 16, "bf16")


@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (1, 1, 17), (2, 3, 48), (1, 7, 257), (2, 2, 1000)])
def test_mfma_fp32_shapes(B, H, T):
    w = WORKLOADS[2].with_(B=B, H=H, T=T, eta=("uniform", 0.01, 0.1))
    announce("linear mfma fp32", B, H, T)
    _check(make_inputs(w, 9 + T), 16, "fp32")


@pytest.mark.parametrize("d,b,dtype", [(16, 16, "fp32"), (32, 16, "fp32"), (64, 16, "fp32"),
                                       (128, 16, "fp32"), (64, 1, "fp32"), (16, 8, "fp32"),
                                       (32, 64, "fp32"), (128, 32, "fp32"), (16, 16, "bf16"),
                                       (32, 16, "bf16"), (128, 16, "bf16"), (64, 8, "bf16"),
                                       (64, 32, "bf16"), (64, 1, "bf16")])
def test_generic_shapes(d, b, dtype):
    w = WORKLOADS[2].with_(B=2, H=3, T=3 * b + 5, d=d, b=b, dtype=dtype, eta=("uniform", 0.01, 0.1))
    announce("linear generic", d, b, dtype)
    _check(make_inputs(w, 100 + d + b), b, dtype)


def test_empty_sequence_copies_state():
    w = WORKLOADS[3].with_(B=2, H=3, T=0)
    inp = to_gpu(make_inputs(w, 5))
    Y, W = linear_gpu(inp, 16)
    assert Y.shape == (2, 3, 0, 64)
    assert torch.equal(W, inp["W0"][None].expand(2, 3, 64, 64))


@pytest.mark.parametrize("cfg", [2, 3])
def test_eta_zero(cfg):
    w = WORKLOADS[cfg].with_(B=2, H=2, T=100, eta=("const", 0.0))
    inp = make_inputs(w, 11)
    g = to_gpu(inp)
    Y, W = linear_gpu(g, 16)
    assert torch.equal(W, g["W0"][None].expand_as(W))       # the state never moves
    ref = torch.matmul(inp["Q"].double(), inp["W0"].double()[None])
    assert rel_l2(Y, ref.numpy()) <= TOL[w.dtype]


# ---------------------------------------------------------------------------
# hand-derived exact examples (d = 2, eta = 1/2) embedded by zero padding:
# every value is dyadic, so both paths must reproduce them bit for bit.
# ---------------------------------------------------------------------------
def _worked_cases():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "linear_d2_worked.json")))
    return g, g["cases"]


def _embed(g, case, d, dtype):
    T = case["T"]
    def pad(rows):
        x = torch.zeros(1, 1, T, d)
        x[0, 0, :, :2] = torch.tensor(rows[:T], dtype=torch.float32)
        return x.to(dtype).cuda()
    W0 = torch.zeros(1, d, d)
    if case["W0"] == "I":
        W0[0, :2, :2] = torch.eye(2)
    return pad(g["q"]), pad(g["k"]), pad(g["v"]), W0.cuda()


@pytest.mark.parametrize("path", ["generic_fp32", "mfma_bf16", "mfma_fp32"])
def test_worked_examples_bit_exact(path):
    g, cases = _worked_cases()
    eta = torch.tensor([float(Fraction(g["eta"]))]).cuda()
    for case in cases:
        if path.startswith("mfma"):
            # when b >= T one chunk covers the sequence, so b equals b = 16 there
            if case["b"] < case["T"]:
                continue
            d, b = 64, 16
            dtype = torch.bfloat16 if path == "mfma_bf16" else torch.float32
        else:
            d, dtype, b = 16, torch.float32, case["b"]
        q, k, v, W0 = _embed(g, case, d, dtype)
        Y, W = ttt.ttt_linear_forward(q, k, v, W0, eta, b)
        torch.cuda.synchronize()
        Yx = torch.tensor([[float(Fraction(x)) for x in r] for r in case["Y"]])
        Wx = torch.tensor([[float(Fraction(x)) for x in r] for r in case["W"]])
        assert torch.equal(Y[0, 0, :, :2].float().cpu(), Yx), case
        assert torch.equal(W[0, 0, :2, :2].cpu(), Wx), case
        assert torch.count_nonzero(Y[0, 0, :, 2:]).item() == 0
        assert torch.count_nonzero(W[0, 0, 2:, :]).item() == 0


# ---------------------------------------------------------------------------
# invariants of the implementation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [2, 3])
def test_deterministic(cfg):
    w = WORKLOADS[cfg].with_(B=2, H=3, T=512)
    g = to_gpu(make_inputs(w, 21))
    Y1, W1 = linear_gpu(g, 16)
    Y2, W2 = linear_gpu(g, 16)
    assert torch.equal(Y1, Y2) and torch.equal(W1, W2)


@pytest.mark.parametrize("cfg", [2, 3])
def test_chaining_through_state_is_exact(cfg, monkeypatch):
    """forward(T) == forward(T1) then forward(T2) from W_out (T1 mod b == 0):
    the fp32 state is stored and reloaded exactly (one segment per chain: a
    segmented scan composes the same updates in another order)."""
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "1")
    w = WORKLOADS[cfg].with_(B=2, H=3, T=160)
    g = to_gpu(make_inputs(w, 31))
    Y, W = linear_gpu(g, 16)
    first = {k: (v[:, :, :64].contiguous() if k in "QKV" else v) for k, v in g.items()}
    second = {k: (v[:, :, 64:].contiguous() if k in "QKV" else v) for k, v in g.items()}
    Y1, W1 = linear_gpu(first, 16)
    second["W0"] = W1
    Y2, W2 = linear_gpu(second, 16)
    assert torch.equal(torch.cat([Y1, Y2], dim=2), Y)
    assert torch.equal(W2, W)


@pytest.mark.parametrize("cfg", [2, 3])
def test_in_place_state_update(cfg):
    w = WORKLOADS[cfg].with_(B=2, H=3, T=80)
    inp = make_inputs(w, 41, w0_per_batch=True)
    g = to_gpu(inp)
    Y_ref, W_ref = linear_gpu(g, 16)
    state = g["W0"].clone()
    Y, W = ttt.ttt_linear_forward(g["Q"], g["K"], g["V"], state, g["eta"], 16, W_out=state)
    torch.cuda.synchronize()
    assert W.data_ptr() == state.data_ptr()
    assert torch.equal(Y, Y_ref) and torch.equal(state, W_ref)


@pytest.mark.parametrize("cfg", [2, 3])
def test_guard_bands_untouched(cfg):
    w = WORKLOADS[cfg].with_(B=2, H=3, T=37)
    g = to_gpu(make_inputs(w, 51))
    G = 4096
    dt = g["Q"].dtype
    ny, nw = g["Q"].numel(), 2 * 3 * 64 * 64
    ybuf = torch.full((ny + 2 * G,), 7.0, dtype=dt, device="cuda")
    wbuf = torch.full((nw + 2 * G,), 7.0, dtype=torch.float32, device="cuda")
    Y = ybuf[G:G + ny].view(g["Q"].shape)
    W = wbuf[G:G + nw].view(2, 3, 64, 64)
    ttt.ttt_linear_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], 16, Y=Y, W_out=W)
    torch.cuda.synchronize()
    for buf, n in ((ybuf, ny), (wbuf, nw)):
        assert (buf[:G] == 7.0).all() and (buf[G + n:] == 7.0).all()
    Yr, Wr = linear_gpu(g, 16)
    assert torch.equal(Y, Yr) and torch.equal(W, Wr)


def test_nan_propagates():
    w = WORKLOADS[3].with_(B=1, H=2, T=64)
    inp = make_inputs(w, 61)
    inp["V"][0, 1, 20, 3] = float("nan")
    Y, W = linear_gpu(to_gpu(inp), 16)
    assert torch.isfinite(Y[0, 0].float()).all() and torch.isfinite(W[0, 0]).all()
    assert torch.isnan(W[0, 1]).any()


# ---------------------------------------------------------------------------
# sequence-segment scan: each segment maps its start state affinely, so the
# chain is cut into segments whose maps are composed (forced segment counts;
# the benchmark workloads above use the library's own choice)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fused", ["1", "0"])
@pytest.mark.parametrize("cfg", [2, 3])
@pytest.mark.parametrize("T,S,per_batch", [(100, 2, False), (333, 3, True), (1000, 7, False),
                                           (100, 50, True), (512, 4, False), (48, 3, False)])
def test_segmented_scan(cfg, T, S, per_batch, fused, monkeypatch):
    """Forced segment counts against the oracle; bf16 runs S >= 3 in the
    fused layout (segment 0 scanned beside the maps) unless
    TTT_LINEAR_FUSED=0."""
    if cfg == 2 and fused == "0":
        pytest.skip("fp32 has no fused layout")
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", str(S))
    monkeypatch.setenv("TTT_LINEAR_FUSED", fused)
    w = WORKLOADS[cfg].with_(B=2, H=3, T=T, w0=("normal", 0.3), eta=("uniform", 0.01, 0.1))
    announce("linear segmented", cfg, T, S, per_batch, "fused" if fused == "1" else "unfused")
    is_fused = ttt.ttt_linear_fused(w.B, w.H, w.T, w.d, w.b, w.torch_dtype)
    if cfg == 2 or fused == "0":
        assert not is_fused
    elif (T, S) == (1000, 7):                    # room for a shorter segment 0
        assert is_fused
    _check(make_inputs(w, 400 + T + S, w0_per_batch=per_batch), 16, w.dtype)


@pytest.mark.parametrize("fused", ["1", "0"])
@pytest.mark.parametrize("cfg", [2, 3])
def test_segmented_in_place_and_deterministic(cfg, fused, monkeypatch):
    """W_out == W0 with several segments: the later segments still start from
    the original W0 (in the unfused layout segment 0 reads the composition's
    copy of it, since the last segment writes W_out in the same launch);
    repeated calls agree bit for bit."""
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "4")
    monkeypatch.setenv("TTT_LINEAR_FUSED", fused)
    w = WORKLOADS[cfg].with_(B=2, H=3, T=300)
    g = to_gpu(make_inputs(w, 71, w0_per_batch=True))
    Y_ref, W_ref = linear_gpu(g, 16)
    Y_again, W_again = linear_gpu(g, 16)
    assert torch.equal(Y_ref, Y_again) and torch.equal(W_ref, W_again)
    state = g["W0"].clone()
    Y, W = ttt.ttt_linear_forward(g["Q"], g["K"], g["V"], state, g["eta"], 16, W_out=state)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_ref) and torch.equal(state, W_ref)


def test_segmented_close_to_single_segment(monkeypatch):
    """fp32: the composed maps change only the rounding order."""
    w = WORKLOADS[2].with_(B=1, H=4, T=1024, w0=("normal", 0.3))
    g = to_gpu(make_inputs(w, 81))
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "1")
    Y1, W1 = linear_gpu(g, 16)
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "16")
    Y16, W16 = linear_gpu(g, 16)
    assert rel_l2(Y16, Y1.double().cpu().numpy()) <= 2e-6
    assert rel_l2(W16, W1.double().cpu().numpy()) <= 2e-6


# ---------------------------------------------------------------------------
# fp32 scans with few chains split each chain's columns over 4 workgroups;
# the one-workgroup kernel still runs with many chains, with the prologue and
# for the backward's start states (TTT_LINEAR_F32_COLS=0 selects it here)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,S,per_batch", [(16, 1, False), (515, 1, True), (1000, 7, False),
                                           (2048, 16, False), (333, 3, True)])
def test_f32_one_workgroup_kernel(T, S, per_batch, monkeypatch):
    monkeypatch.setenv("TTT_LINEAR_F32_COLS", "0")
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", str(S))
    w = WORKLOADS[2].with_(B=2, H=3, T=T, w0=("normal", 0.3), eta=("uniform", 0.01, 0.1))
    announce("linear fp32 one workgroup per chain", T, S, per_batch)
    _check(make_inputs(w, 500 + T + S, w0_per_batch=per_batch), 16, "fp32")


@pytest.mark.parametrize("S", ["1", "5", "16"])
def test_f32_column_split_close_to_one_workgroup(S, monkeypatch):
    """The column split changes only the order of the sums over the 64 input
    rows (four partial products added in LDS)."""
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", S)
    w = WORKLOADS[2].with_(B=1, H=4, T=1100, w0=("normal", 0.3))
    announce("fp32 column split vs one workgroup", S)
    g = to_gpu(make_inputs(w, 91))
    Y1, W1 = linear_gpu(g, 16)
    monkeypatch.setenv("TTT_LINEAR_F32_COLS", "0")
    Y0, W0 = linear_gpu(g, 16)
    ey = rel_l2(Y1, Y0.double().cpu().numpy())
    ew = rel_l2(W1, W0.double().cpu().numpy())
    print(f"  rel-L2 Y {ey:.2e}  W {ew:.2e}", flush=True)
    assert ey <= 2e-6 and ew <= 2e-6


@pytest.mark.parametrize("B,H,T", [(1, 2, 1000), (2, 2, 3001), (1, 4, 2048)])
def test_f32_planned_segments(B, H, T):
    """The library's own segment plan for few fp32 chains (column split, the
    segments composing their own start states)."""
    w = WORKLOADS[2].with_(B=B, H=H, T=T, w0=("normal", 0.3), eta=("uniform", 0.01, 0.1))
    n = ttt.ttt_linear_segments(B, H, T, 64, 16, torch.float32)
    announce("fp32 planned segments", B, H, T, "segments", n)
    assert n > 1
    _check(make_inputs(w, 600 + T), 16, "fp32")


# ---------------------------------------------------------------------------
# the caller's workspace: the segment maps live there; a smaller one gives
# fewer segments (none without a workspace); the call can be captured
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [2, 3])
def test_workspace_limits_segments(cfg, monkeypatch):
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "8")
    w = WORKLOADS[cfg].with_(B=2, H=3, T=1000, w0=("normal", 0.3), eta=("uniform", 0.01, 0.1))
    announce("workspace limits the segment count", cfg)
    inp = make_inputs(w, 800 + cfg)
    g = to_gpu(inp)
    full = ttt.ttt_linear_workspace_bytes(w.B, w.H, w.T, 64, 16, w.torch_dtype)
    assert full == w.B * w.H * (3 * 8 - 2) * 64 * 64 * 4
    Yr, Wr = linear_oracle(inp, 16)

    def run(nbytes):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        Y, W = ttt.ttt_linear_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], 16, workspace=ws)
        torch.cuda.synchronize()
        return Y, W

    def forced(S):
        monkeypatch.setenv("TTT_LINEAR_SEGMENTS", str(S))
        out = run(ttt.ttt_linear_workspace_bytes(w.B, w.H, w.T, 64, 16, w.torch_dtype))
        monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "8")
        return out

    for nbytes, S in ((0, 1), (full - 1, 7), (w.B * w.H * (3 * 4 - 2) * 64 * 64 * 4, 4), (full, 8)):
        Y, W = run(nbytes)
        Ys, Ws = forced(S)
        assert torch.equal(Y, Ys) and torch.equal(W, Ws), (nbytes, S)
        ey, ew = rel_l2(Y, Yr), rel_l2(W, Wr)
        print(f"  {nbytes} bytes -> {S} segments: rel-L2 Y {ey:.2e}  W {ew:.2e}", flush=True)
        assert ey <= TOL[w.dtype] and ew <= TOL[w.dtype]


def test_graph_capture_config4_shape():
    """A segmented forward of the 32768-token workload's shape captured in a
    HIP graph: every replay equals the eager call bit for bit, with other
    eager work on the stream between the replays."""
    w = WORKLOADS[4]
    assert ttt.ttt_linear_segments(w.B, w.H, w.T, 64, 16, torch.bfloat16) > 1
    announce("graph capture, config 4 shape")
    g = to_gpu(cached_inputs(4, default_seed(4)))
    Y_e, W_e = linear_gpu(g, 16)
    Y = torch.empty_like(Y_e)
    W = torch.empty_like(W_e)
    ws = torch.empty(ttt.ttt_linear_workspace_bytes(w.B, w.H, w.T, 64, 16, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the launch path off the capture
        ttt.ttt_linear_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], 16, Y=Y, W_out=W,
                               workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ttt.ttt_linear_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], 16, Y=Y, W_out=W,
                               workspace=ws)
    other = make_inputs(w.with_(B=1, H=4, T=3000), 4242)
    og = to_gpu(other)
    for rep in range(3):
        Y.zero_()
        W.zero_()
        ws.fill_(0xff)
        # eager work between the replays, also through the workspace
        ttt.ttt_linear_forward(og["Q"], og["K"], og["V"], og["W0"], og["eta"], 16, workspace=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_e) and torch.equal(W, W_e), rep
