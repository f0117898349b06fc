"""GPU parity of ttt_mlp_forward against the fp64 oracle."""
import pytest
import torch

import test_sequence_layers_linear_amd as ttt
from parity_util import (WORKLOADS, TOL, announce, default_seed, make_inputs, mlp_gpu, mlp_oracle,
                         per_chain_rel_l2, rel_l2, to_gpu)

pytestmark = pytest.mark.gpu


def _check(inp, b, dtype):
    Y, W1, W2 = mlp_gpu(to_gpu(inp), b)
    Yr, W1r, W2r = mlp_oracle(inp, b)
    e = (rel_l2(Y, Yr), rel_l2(W1, W1r), rel_l2(W2, W2r))
    print("  rel-L2 Y %.3e  W1 %.3e  W2 %.3e" % e, flush=True)
    assert max(e) <= TOL[dtype], e


@pytest.mark.parametrize("d,m,b,T,dtype", [(64, 256, 16, 100, "bf16"), (64, 256, 16, 16, "bf16"),
                                           (64, 256, 16, 5, "bf16"), (64, 256, 16, 48, "bf16"),
                                           (64, 256, 16, 300, "fp32"),
                                           (16, 64, 4, 37, "fp32"), (32, 128, 16, 50, "fp32"),
                                           (32, 128, 8, 50, "bf16"), (64, 512, 16, 40, "bf16"),
                                           (16, 16, 1, 9, "fp32")])
def test_mlp_shapes(d, m, b, T, dtype):
    announce("mlp", d, m, b, T, dtype)
    w = WORKLOADS[5].with_(B=2, H=3, T=T, d=d, m=m, b=b, dtype=dtype)
    _check(make_inputs(w, 200 + d + m + T), b, dtype)


@pytest.mark.parametrize("T,std,eta,per_batch", [(32, 0.3, 0.3, False), (100, 0.2, 0.1, True),
                                                  (160, 0.2, 0.1, False), (257, 0.1, 0.05, True)])
def test_mlp_strong_state(T, std, eta, per_batch):
    """d64 m256 b16 bf16 with a state large enough that every term of the
    update and the readout moves the result well above the tolerance (the
    updates change Y by 70-100 % in rel-L2 here; larger eta at T = 100 makes
    the inner descent itself diverge)."""
    announce("mlp strong state", T, std, eta, per_batch)
    w = WORKLOADS[5].with_(B=2, H=3, T=T, w0=("normal", std), eta=("const", eta))
    _check(make_inputs(w, 300 + T, w0_per_batch=per_batch), 16, "bf16")


def test_config5_full():
    """The TTT-MLP workload at full size, all 48 chains, relative L2 over the
    whole Y, W1 and W2 tensors."""
    w = WORKLOADS[5]
    announce("mlp config 5, all chains", w.name)
    inp = make_inputs(w, default_seed(5))
    Y, W1, W2 = mlp_gpu(to_gpu(inp), w.b)
    Yr, W1r, W2r = mlp_oracle(inp, w.b)
    e = (rel_l2(Y, Yr), rel_l2(W1, W1r), rel_l2(W2, W2r))
    print("  rel-L2 Y %.3e  W1 %.3e  W2 %.3e" % e
          + f"  (worst chain Y {per_chain_rel_l2(Y, Yr).max():.3e})", flush=True)
    assert max(e) <= TOL["bf16"]


def test_mlp_eta_zero_keeps_state():
    w = WORKLOADS[5].with_(B=1, H=2, T=64, eta=("const", 0.0))
    g = to_gpu(make_inputs(w, 9))
    Y, W1, W2 = mlp_gpu(g, 16)
    assert torch.equal(W1, g["W1"][None].expand_as(W1))
    assert torch.equal(W2, g["W2"][None].expand_as(W2))


def test_mlp_deterministic_and_empty():
    w = WORKLOADS[5].with_(B=2, H=2, T=80)
    g = to_gpu(make_inputs(w, 19))
    a = mlp_gpu(g, 16)
    b = mlp_gpu(g, 16)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    e = to_gpu(make_inputs(w.with_(T=0), 19))
    Y, W1, W2 = mlp_gpu(e, 16)
    assert torch.equal(W1, e["W1"][None].expand_as(W1)) and torch.equal(W2, e["W2"][None].expand_as(W2))
