"""The forward entry point that allocates nothing (ttt_linear_forward_noalloc:
the segment maps and start states live in the library's static device
scratch) against ttt_linear_forward with a caller workspace.  Both run the
same plan on the same kernels, so they must agree bit for bit; the scratch
keeps the previous call's contents, so the calls run back to back, each
smaller than the one before, and an unsegmented call needs no scratch."""
import pytest
import torch

import test_sequence_layers_linear_amd as ttt
from parity_util import WORKLOADS, TOL, announce, default_seed, linear_oracle, make_inputs, rel_l2, to_gpu

pytestmark = pytest.mark.gpu

# (workload, overrides, seed): the 32768-token workload (5 planned segments),
# then smaller ones: few bf16 chains (many segments), few fp32 chains (the
# column-split scan), many chains (one segment, no scratch)
CASES = [
    (4, {}, default_seed(4)),
    (3, dict(B=1, H=4, T=2048), 1301),
    (2, dict(B=1, H=2, T=1000), 1302),
    (3, dict(B=8, H=12, T=300), 1303),
]


def _case(cfg, over, seed):
    w = WORKLOADS[cfg].with_(**over) if over else WORKLOADS[cfg]
    return w, make_inputs(w, seed)


def test_noalloc_matches_workspace_entry_point():
    assert ttt.load_library().ttt_linear_noalloc_max_workspace_bytes() == 16 << 20
    for i, (cfg, over, seed) in enumerate(CASES):
        w, inp = _case(cfg, over, seed)
        nseg = ttt.ttt_linear_segments(w.B, w.H, w.T, w.d, w.b, w.torch_dtype)
        need = ttt.ttt_linear_workspace_bytes(w.B, w.H, w.T, w.d, w.b, w.torch_dtype)
        announce("noalloc call", i, w.name, "segments", nseg, "scratch bytes", need)
        assert need <= 16 << 20
        g = to_gpu(inp)
        Y_ref, W_ref = ttt.ttt_linear_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], w.b)
        Y = torch.full_like(Y_ref, float("nan"))
        W = torch.full_like(W_ref, float("nan"))
        torch.cuda.synchronize()
        ttt.ttt_linear_forward_noalloc(g["Q"], g["K"], g["V"], g["W0"], g["eta"], w.b, Y, W)
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_ref) and torch.equal(W, W_ref), i
        if w.B * w.H * w.T <= 48 * 32768:
            Yr, Wr = linear_oracle(inp, w.b)
            ey, ew = rel_l2(Y, Yr), rel_l2(W, Wr)
            print(f"  rel-L2 Y {ey:.2e}  W {ew:.2e}", flush=True)
            assert ey <= TOL[w.dtype] and ew <= TOL[w.dtype]


def test_noalloc_repeated_calls_agree():
    """Two calls in a row on one input give the same result (nothing in the
    scratch carries over)."""
    w, inp = _case(3, dict(B=2, H=3, T=1000), 1304)
    g = to_gpu(inp)
    outs = []
    for _ in range(2):
        Y = torch.empty_like(g["Q"])
        W = torch.empty((w.B, w.H, 64, 64), device="cuda")
        ttt.ttt_linear_forward_noalloc(g["Q"], g["K"], g["V"], g["W0"], g["eta"], w.b, Y, W)
        torch.cuda.synchronize()
        outs.append((Y, W))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
