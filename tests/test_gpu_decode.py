"""GPU parity of ttt_linear_decode_step against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import test_sequence_layers_linear_amd as ttt
from parity_util import (WORKLOADS, TOL, announce, cached_inputs, default_seed, linear_gpu,
                         make_inputs, per_chain_rel_l2, rel_l2, to_gpu)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_steps_match_online_gd(d, dtype):
    """n decode steps from a per-(batch, head) state == the oracle's b = 1 scan."""
    announce("decode", d, dtype)
    w = WORKLOADS[2].with_(B=2, H=3, T=9, d=d, dtype=dtype, eta=("uniform", 0.01, 0.1))
    inp = make_inputs(w, 70 + d, w0_per_batch=True)
    Yr, Wr = oracle.linear_forward(inp["Q"], inp["K"], inp["V"], inp["W0"], inp["eta"], 1)
    g = to_gpu(inp)
    W = g["W0"].clone()
    ys = []
    for t in range(w.T):
        ys.append(ttt.ttt_linear_decode_step(g["Q"][:, :, t].contiguous(),
                                             g["K"][:, :, t].contiguous(),
                                             g["V"][:, :, t].contiguous(), W, g["eta"]))
    torch.cuda.synchronize()
    Y = torch.stack(ys, dim=2)
    ey, ew = rel_l2(Y, Yr), rel_l2(W, Wr)
    print(f"  rel-L2 y {ey:.3e}  W {ew:.3e}", flush=True)
    assert ey <= TOL[dtype] and ew <= TOL[dtype]


def test_config4_prefill_then_256_decode_steps():
    """The long-context workload's tail: forward over T = 32768 tokens, then
    256 single-token steps from the final W, every chain, relative L2 over the
    whole tensor of the 256 outputs and of the final state."""
    w = WORKLOADS[4]
    announce("decode after config 4 prefill, all chains", w.name)
    inp = cached_inputs(4, default_seed(4))
    g = to_gpu(inp)
    _, W = linear_gpu(g, w.b)
    ys = []
    for s in range(w.decode_steps):
        ys.append(ttt.ttt_linear_decode_step(g["dq"][s], g["dk"][s], g["dv"][s], W, g["eta"]))
    torch.cuda.synchronize()
    y = torch.stack(ys)                           # [steps, B, H, d]
    _, Wr = oracle.linear_forward(inp["Q"], inp["K"], inp["V"], inp["W0"], inp["eta"], w.b)
    yr = []
    for s in range(w.decode_steps):
        ys_, Wr = oracle.linear_decode(inp["dq"][s], inp["dk"][s], inp["dv"][s], Wr, inp["eta"])
        yr.append(ys_)
    yr = np.stack(yr)
    ey, ew = rel_l2(y, yr), rel_l2(W, Wr)
    print(f"  rel-L2 y {ey:.3e}  W {ew:.3e}  (worst chain W {per_chain_rel_l2(W, Wr).max():.3e})",
          flush=True)
    assert ey <= TOL["bf16"] and ew <= TOL["bf16"]


def test_decode_worked_example_exact():
    """Token 2 of the hand-derived d = 2 example as one step, embedded in d = 16."""
    W = torch.zeros(1, 1, 16, 16)
    W[0, 0, 0, :2] = torch.tensor([0.5, 1.0])
    q = torch.zeros(1, 1, 16); q[0, 0, :2] = torch.tensor([1.0, 0.0])
    k = torch.zeros(1, 1, 16); k[0, 0, :2] = torch.tensor([1.0, 1.0])
    v = torch.zeros(1, 1, 16); v[0, 0, :2] = torch.tensor([3.0, -1.0])
    W = W.cuda()
    y = ttt.ttt_linear_decode_step(q.cuda(), k.cuda(), v.cuda(), W, torch.tensor([0.5]).cuda())
    torch.cuda.synchronize()
    assert torch.equal(y[0, 0, :2].cpu(), torch.tensor([1.75, 0.0]))
    assert torch.equal(W[0, 0, :2, :2].cpu(), torch.tensor([[1.75, 0.0], [1.25, -1.0]]))


def test_decode_steps_in_a_hip_graph_match_eager():
    """Decode steps captured once in a HIP graph and replayed several times
    (with eager work and synchronisation between the replays) give exactly
    the eager results each time."""
    w = WORKLOADS[4].with_(B=2, H=3, T=16, decode_steps=8)
    g = to_gpu(make_inputs(w, 91, w0_per_batch=True))
    W = g["W0"].clone()
    y = torch.empty_like(g["dq"][0])

    def steps():
        for s in range(w.decode_steps):
            ttt.ttt_linear_decode_step(g["dq"][s], g["dk"][s], g["dv"][s], W, g["eta"], y=y)

    steps()
    torch.cuda.synchronize()
    W_ref, y_ref = W.clone(), y.clone()
    W.copy_(g["W0"])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps()
    for _ in range(3):
        W.copy_(g["W0"])
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(W, W_ref) and torch.equal(y, y_ref)
