"""GPU parity of ttt_linear_backward_ex (the backward through LayerNorm of q
and k, per-token step sizes and the chunk-start read) against the fp64
oracle's linear_backward_ex.

Every gradient -- dQ, dK (of the raw rows), dV, dW0, deta, deta_tok, dln_q,
dln_k -- is compared in relative L2 on the same seeded inputs and cotangents:
within 1e-4 for fp32 Q/K/V and 2e-2 for bf16 Q/K/V (normalised rows and
gradients rounded to bf16).  Cases: each part of the prologue alone and
together, the chunk-start read, ragged tails, forced segment counts, and three
benchmark workloads at full size (every chain).
"""
import pytest
import torch

import oracle
import test_sequence_layers_linear_amd as ttt
from parity_util import WORKLOADS, TOL, announce, default_seed, make_inputs, rel_l2, to_gpu
from test_sequence_layers_linear_amd.inputs import make_cotangents, make_prologue

pytestmark = pytest.mark.gpu

PARTS = {"ln": ("ln_q", "ln_k"), "ln_q": ("ln_q",), "tok": ("eta_tok",),
         "all": ("ln_q", "ln_k", "eta_tok")}


def _case(w, seed, parts, per_batch=False, zero_state=False):
    inp = make_inputs(w, seed, w0_per_batch=per_batch)
    pro = make_prologue(w, seed + 3)
    inp["eta"] = pro["eta"]
    kw = {k: pro[k] for k in parts}
    cot = make_cotangents(w, seed + 1, zero_state=zero_state)
    return inp, kw, cot


def _gpu(inp, kw, cot, b, read_start):
    g, gk, gc = to_gpu(inp), to_gpu(kw), to_gpu(cot)
    out = ttt.ttt_linear_backward_ex(g["Q"], g["K"], g["V"], g["W0"], g["eta"], b, gc["dY"],
                                     gc["dW_out"], read_chunk_start=read_start, **gk)
    torch.cuda.synchronize()
    return out


def _oracle(inp, kw, cot, b, read_start):
    return oracle.linear_backward_ex(inp["Q"], inp["K"], inp["V"], inp["W0"], inp["eta"], b,
                                     cot["dY"], cot["dW_out"], read_chunk_start=read_start, **kw)


def _compare(got, ref, tol, names=None):
    names = names or sorted(ref)
    errs = {n: rel_l2(got[n], ref[n]) for n in names}
    print("  rel-L2 " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("part", sorted(PARTS))
@pytest.mark.parametrize("read_start", [False, True])
@pytest.mark.parametrize("B,H,T,per_batch", [(1, 2, 16, False), (2, 3, 77, True), (1, 2, 300, False)])
def test_backward_prologue_small(dtype, part, read_start, B, H, T, per_batch, monkeypatch):
    monkeypatch.setenv("TTT_LINEAR_BWD_SEGMENTS", "1")
    w = WORKLOADS[3].with_(B=B, H=H, T=T, dtype=dtype)
    seed = 9500 + B * 100 + H * 10 + T
    announce("backward prologue", dtype, part, "start-read" if read_start else "", B, H, T, seed)
    inp, kw, cot = _case(w, seed, PARTS[part], per_batch)
    got = _gpu(inp, kw, cot, w.b, read_start)
    ref = _oracle(inp, kw, cot, w.b, read_start)
    assert sorted(got) == sorted(ref)
    _compare(got, ref, TOL[dtype])
    if "eta_tok" in kw:
        assert torch.count_nonzero(got["deta"]).item() == 0


def test_backward_read_start_alone():
    # only the chunk-start read: no LayerNorm, the head's step size
    w = WORKLOADS[3].with_(B=2, H=2, T=90, dtype="fp32")
    announce("backward chunk-start read only")
    inp, _, cot = _case(w, 9601, ())
    _compare(_gpu(inp, {}, cot, 16, True), _oracle(inp, {}, cot, 16, True), TOL["fp32"])


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T,S,per_batch", [(100, 2, False), (333, 3, True), (480, 30, False)])
def test_backward_prologue_segmented(dtype, T, S, per_batch, monkeypatch):
    monkeypatch.setenv("TTT_LINEAR_BWD_SEGMENTS", str(S))
    w = WORKLOADS[3].with_(B=2, H=2, T=T, dtype=dtype)
    assert ttt.ttt_linear_backward_segments(w.B, w.H, w.T, w.d, w.b, w.torch_dtype) == S
    seed = 9700 + T + S
    announce("backward prologue segmented", dtype, T, S, seed)
    inp, kw, cot = _case(w, seed, PARTS["all"], per_batch)
    _compare(_gpu(inp, kw, cot, w.b, False), _oracle(inp, kw, cot, w.b, False), TOL[dtype])


def test_backward_prologue_empty_sequence():
    w = WORKLOADS[3].with_(B=2, H=3, T=0)
    announce("backward prologue T=0")
    inp, kw, cot = _case(w, 9800, PARTS["all"])
    got = _gpu(inp, kw, cot, 16, False)
    assert got["dQ"].shape == (2, 3, 0, 64) and got["deta_tok"].shape == (2, 3, 0)
    assert torch.equal(got["dW0"].cpu(), cot["dW_out"].sum(0))
    assert torch.count_nonzero(got["dln_q"]).item() == 0
    assert torch.count_nonzero(got["deta"]).item() == 0


def test_backward_prologue_deterministic():
    w = WORKLOADS[3].with_(B=2, H=4, T=300)
    announce("backward prologue determinism")
    inp, kw, cot = _case(w, 9810, PARTS["all"])
    a = _gpu(inp, kw, cot, 16, False)
    b = _gpu(inp, kw, cot, 16, False)
    for n in a:
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("cfg", [2, 3])
def test_backward_prologue_config_full(cfg):
    w = WORKLOADS[cfg]
    announce("backward prologue config", cfg, w.name, "segments",
             ttt.ttt_linear_backward_segments(w.B, w.H, w.T, w.d, w.b, w.torch_dtype))
    inp, kw, cot = _case(w, default_seed(cfg) + 700, PARTS["all"])
    _compare(_gpu(inp, kw, cot, w.b, False), _oracle(inp, kw, cot, w.b, False), TOL[w.dtype])


def test_backward_prologue_config4_full():
    """The 32768-token workload's backward through the whole prologue, W0
    given per batch, every chain and every gradient (the LayerNorm and head-eta
    gradients summed over the batch on both sides), relative L2 over the whole
    tensors."""
    w = WORKLOADS[4]
    announce("backward prologue config 4, all chains", w.name)
    inp, kw, cot = _case(w, default_seed(4) + 700, PARTS["all"], per_batch=True)
    _compare(_gpu(inp, kw, cot, w.b, False), _oracle(inp, kw, cot, w.b, False), TOL["bf16"])
