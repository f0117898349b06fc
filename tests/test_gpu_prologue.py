"""GPU parity of ttt_linear_forward_ex (LayerNorm of q and k, step size per
token) against the fp64 oracle's linear_forward_ex.

Relative L2 of Y and W_out within 1e-4 for fp32 inputs and 2e-2 for bf16
inputs (whose normalised rows are rounded to bf16 before the products, while
the oracle keeps them exact).  Cases: each part of the prologue alone and
together, ragged tails, segmented scans (forced segment counts) and three
benchmark workloads at full size (every chain).
"""
import pytest
import torch

import oracle
import test_sequence_layers_linear_amd as ttt
from parity_util import (WORKLOADS, TOL, announce, default_seed, make_inputs, per_chain_rel_l2,
                         rel_l2, to_gpu)
from test_sequence_layers_linear_amd.inputs import make_prologue

pytestmark = pytest.mark.gpu

PARTS = {"ln": ("ln_q", "ln_k"), "ln_k": ("ln_k",), "tok": ("eta_tok",),
         "all": ("ln_q", "ln_k", "eta_tok")}


def _run(w, seed, parts, per_batch=False, eps=1e-5):
    inp = make_inputs(w, seed, w0_per_batch=per_batch)
    pro = make_prologue(w, seed + 3)
    inp["eta"] = pro["eta"]
    kw = {k: pro[k] for k in parts}
    g = to_gpu(inp)
    gk = to_gpu(kw)
    Y, W = ttt.ttt_linear_forward_ex(g["Q"], g["K"], g["V"], g["W0"], g["eta"], w.b, ln_eps=eps, **gk)
    torch.cuda.synchronize()
    Yr, Wr = oracle.linear_forward_ex(inp["Q"], inp["K"], inp["V"], inp["W0"], inp["eta"], w.b,
                                      ln_eps=eps, **kw)
    ey, ew = rel_l2(Y, Yr), rel_l2(W, Wr)
    print(f"  rel-L2 Y {ey:.3e}  W {ew:.3e}", flush=True)
    return ey, ew


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("part", sorted(PARTS))
@pytest.mark.parametrize("B,H,T,per_batch", [(1, 2, 16, False), (2, 3, 77, True), (1, 2, 300, False)])
def test_prologue_small(dtype, part, B, H, T, per_batch, monkeypatch):
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "1")
    w = WORKLOADS[3].with_(B=B, H=H, T=T, dtype=dtype)
    seed = 9000 + B * 100 + H * 10 + T
    announce("prologue", dtype, part, B, H, T, seed)
    ey, ew = _run(w, seed, PARTS[part], per_batch)
    assert ey <= TOL[dtype] and ew <= TOL[dtype]


@pytest.mark.parametrize("part", ["all", "tok"])
@pytest.mark.parametrize("T,S", [(77, 1), (333, 3)])
def test_prologue_f32_one_workgroup_kernel(part, T, S, monkeypatch):
    """fp32 with one workgroup per chain (the kernel for many chains; few
    chains split W by columns unless TTT_LINEAR_F32_COLS=0)."""
    monkeypatch.setenv("TTT_LINEAR_F32_COLS", "0")
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", str(S))
    w = WORKLOADS[3].with_(B=2, H=3, T=T, dtype="fp32")
    seed = 9200 + T + S
    announce("prologue fp32 one workgroup per chain", part, T, S, seed)
    ey, ew = _run(w, seed, PARTS[part])
    assert ey <= TOL["fp32"] and ew <= TOL["fp32"]


@pytest.mark.parametrize("dtype,layout", [("fp32", "unfused"), ("bf16", "unfused"), ("bf16", "fused")])
@pytest.mark.parametrize("T,S", [(100, 2), (333, 3), (480, 30)])
def test_prologue_segmented(dtype, layout, T, S, monkeypatch):
    """bf16 runs both segment layouts: maps then scans, and segment 0's scan
    beside the other segments' maps (from 3 segments on)."""
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", str(S))
    monkeypatch.setenv("TTT_LINEAR_FUSED", "1" if layout == "fused" else "0")
    w = WORKLOADS[3].with_(B=1, H=3, T=T, dtype=dtype)
    seed = 9100 + T + S
    announce("prologue segmented", dtype, layout, T, S, seed)
    ey, ew = _run(w, seed, PARTS["all"])
    assert ey <= TOL[dtype] and ew <= TOL[dtype]


def test_prologue_eps_matters_for_flat_rows():
    """A constant key row normalises to beta alone; eps only scales the zero."""
    w = WORKLOADS[3].with_(B=1, H=2, T=40, dtype="fp32")
    announce("prologue flat rows")
    inp = make_inputs(w, 9200)
    inp["K"][0, 1, 5] = 0.25
    pro = make_prologue(w, 9203)
    inp["eta"] = pro["eta"]
    g = to_gpu(inp)
    Y, W = ttt.ttt_linear_forward_ex(g["Q"], g["K"], g["V"], g["W0"], g["eta"], 16,
                                     ln_k=pro["ln_k"].cuda(), ln_eps=1e-3)
    torch.cuda.synchronize()
    Yr, Wr = oracle.linear_forward_ex(inp["Q"], inp["K"], inp["V"], inp["W0"], inp["eta"], 16,
                                      ln_k=pro["ln_k"], ln_eps=1e-3)
    assert rel_l2(Y, Yr) <= 1e-4 and rel_l2(W, Wr) <= 1e-4


def test_prologue_off_is_plain_forward():
    w = WORKLOADS[3].with_(B=2, H=2, T=200)
    announce("prologue off")
    g = to_gpu(make_inputs(w, 9300))
    Y0, W0 = ttt.ttt_linear_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], 16)
    Y1, W1 = ttt.ttt_linear_forward_ex(g["Q"], g["K"], g["V"], g["W0"], g["eta"], 16)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1) and torch.equal(W0, W1)


@pytest.mark.parametrize("cfg", [2, 3])
def test_prologue_config_full(cfg):
    w = WORKLOADS[cfg]
    announce("prologue config", cfg, w.name)
    ey, ew = _run(w, default_seed(cfg) + 900, PARTS["all"])
    assert ey <= TOL[w.dtype] and ew <= TOL[w.dtype]


def test_prologue_config4_full():
    """The 32768-token workload with the whole prologue, in the launch
    configuration the benchmark times (planned segments: maps, combine and the
    staging-wave scans), all 48 chains, relative L2 over the whole tensors."""
    w = WORKLOADS[4]
    announce("prologue config 4, all chains", w.name)
    inp = dict(make_inputs(w, default_seed(4) + 900))
    pro = make_prologue(w, default_seed(4) + 903)
    inp["eta"] = pro["eta"]
    g = to_gpu(inp)
    Y, W = ttt.ttt_linear_forward_ex(g["Q"], g["K"], g["V"], g["W0"], g["eta"], w.b,
                                     **to_gpu({k: pro[k] for k in PARTS["all"]}))
    torch.cuda.synchronize()
    Yr, Wr = oracle.linear_forward_ex(inp["Q"], inp["K"], inp["V"], inp["W0"], inp["eta"], w.b,
                                      **{k: pro[k] for k in PARTS["all"]})
    ey, ew = rel_l2(Y, Yr), rel_l2(W, Wr)
    print(f"  rel-L2 Y {ey:.3e}  W {ew:.3e}  (worst chain Y {per_chain_rel_l2(Y, Yr).max():.3e})",
          flush=True)
    assert ey <= TOL["bf16"] and ew <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp32-one-workgroup"])
@pytest.mark.parametrize("T,S,parts", [(77, 1, ()), (300, 1, ("eta_tok",)), (333, 3, ("ln_q", "ln_k", "eta_tok"))])
def test_chunk_start_read(dtype, T, S, parts, monkeypatch):
    """Tokens read out with their mini-batch's start weights (read_mode 1)."""
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", str(S))
    if dtype == "fp32-one-workgroup":
        monkeypatch.setenv("TTT_LINEAR_F32_COLS", "0")
        dtype = "fp32"
    w = WORKLOADS[3].with_(B=2, H=3, T=T, dtype=dtype)
    seed = 9400 + T + S
    announce("chunk-start read", dtype, T, S, parts, seed)
    inp = make_inputs(w, seed)
    pro = make_prologue(w, seed + 3)
    inp["eta"] = pro["eta"]
    kw = {k: pro[k] for k in parts}
    g = to_gpu(inp)
    Y, W = ttt.ttt_linear_forward_ex(g["Q"], g["K"], g["V"], g["W0"], g["eta"], 16,
                                     read_chunk_start=True, **to_gpu(kw))
    torch.cuda.synchronize()
    Yr, Wr = oracle.linear_forward_ex(inp["Q"], inp["K"], inp["V"], inp["W0"], inp["eta"], 16,
                                      read_chunk_start=True, **kw)
    ey, ew = rel_l2(Y, Yr), rel_l2(W, Wr)
    print(f"  rel-L2 Y {ey:.3e}  W {ew:.3e}", flush=True)
    assert ey <= TOL[dtype] and ew <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("parts,read_start", [(("ln_q", "ln_k", "eta_tok"), False),
                                              (("ln_k",), True), ((), True)])
def test_decode_step_ex(dtype, d, parts, read_start):
    """Three prologue decode steps from a random state against the oracle's
    one-token forward (b = 1) with per-batch W0 = the state."""
    w = WORKLOADS[3].with_(B=2, H=3, T=3, d=d, dtype=dtype)
    seed = 9500 + d + len(parts) + int(read_start)
    announce("decode_ex", dtype, d, parts, read_start, seed)
    inp = make_inputs(w, seed, w0_per_batch=True)
    pro = make_prologue(w, seed + 3)
    inp["eta"] = pro["eta"]
    W = inp["W0"].clone().cuda()
    Wref = inp["W0"]
    for t in range(3):
        kw = {k: pro[k] for k in parts if k != "eta_tok"}
        if "eta_tok" in parts:
            kw["eta_tok"] = pro["eta_tok"][:, :, t].contiguous()
        y = ttt.ttt_linear_decode_step_ex(inp["Q"][:, :, t].contiguous().cuda(),
                                          inp["K"][:, :, t].contiguous().cuda(),
                                          inp["V"][:, :, t].contiguous().cuda(), W,
                                          inp["eta"].cuda(), read_chunk_start=read_start,
                                          **to_gpu(kw))
        torch.cuda.synchronize()
        okw = {k: pro[k] for k in parts if k != "eta_tok"}
        if "eta_tok" in parts:
            okw["eta_tok"] = pro["eta_tok"][:, :, t:t + 1]
        yr, Wref = oracle.linear_forward_ex(inp["Q"][:, :, t:t + 1], inp["K"][:, :, t:t + 1],
                                            inp["V"][:, :, t:t + 1], Wref, inp["eta"], 1,
                                            read_chunk_start=read_start, **okw)
        ey, ew = rel_l2(y, yr[:, :, 0]), rel_l2(W, Wref)
        print(f"  step {t} rel-L2 y {ey:.3e}  W {ew:.3e}", flush=True)
        assert ey <= TOL[dtype] and ew <= TOL[dtype]
