"""The roof kernels of include/ttt_roofs.h on the GPU: the copy moves every
byte, the MFMA loop reports the flops it was asked for and keeps its products,
and the empty launch runs in a HIP graph."""
import ctypes

import pytest
import torch

import test_sequence_layers_linear_amd as ttt
from parity_util import announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    lib = ttt.load_library()
    lib.ttt_roof_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.ttt_roof_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    lib.ttt_roof_launch.argtypes = [ctypes.c_int64, ctypes.c_void_p]
    return lib


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 3 << 20])
def test_copy_is_exact(lib, nbytes):
    """Every byte arrives, including a ragged tail past the unrolled loop; the
    bytes after the copied range stay untouched."""
    announce("roof copy", nbytes)
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.full((nbytes + 64,), 7, dtype=torch.uint8, device="cuda")
    ttt._check(lib.ttt_roof_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream()))
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 7).all())


@pytest.mark.parametrize("dtype,per", [(1, 2 * 16 * 16 * 32), (0, 2 * 16 * 16 * 4)])
def test_mfma_loop_counts_and_keeps_products(lib, dtype, per):
    """The flop count is waves x iters x 8 chains x one MFMA; every thread
    writes a finite, non-zero sum (the products are not folded away)."""
    announce("roof mfma", dtype)
    waves, iters = 8, 50
    out = torch.full((waves * 64,), float("nan"), device="cuda")
    fl = ctypes.c_double(0.0)
    ttt._check(lib.ttt_roof_mfma(out.data_ptr(), dtype, waves, iters, ctypes.byref(fl), stream()))
    torch.cuda.synchronize()
    assert fl.value == waves * iters * 8 * per
    assert bool(torch.isfinite(out).all())
    assert bool((out != 0).any())


def test_empty_launch_in_a_graph(lib):
    """The launch floor's kernel captures and replays in a HIP graph (as the
    decode measurement uses it) and leaves the stream usable."""
    announce("roof launch")

    def launches():
        for _ in range(16):
            ttt._check(lib.ttt_roof_launch(96, stream()))

    launches()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launches()
    for _ in range(3):
        graph.replay()
    x = torch.ones(4, device="cuda")
    torch.cuda.synchronize()
    assert float((x * 2).sum()) == 8.0
