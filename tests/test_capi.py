"""The C ABI of libttt.so, checked without a GPU.

The library must load and export every function include/ttt.h declares, and
every argument error must come back as its status code before any HIP call
is made (so these run on a machine with no GPU).  Fake, never-dereferenced
addresses stand in for device buffers.
"""
import ctypes
import glob
import os
import re

import pytest

import test_sequence_layers_linear_amd as ttt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, INVALID, UNSUPPORTED = ttt.TTT_OK, ttt.TTT_ERR_INVALID_ARG, ttt.TTT_ERR_UNSUPPORTED

# fake device addresses, far apart so only deliberate overlaps overlap
QA, KA, VA, W0A, ETA, YA, WOA = (0x10_0000_0000 * (i + 1) for i in range(7))
W1A, W2A, W1O, W2O = (0x90_0000_0000 + 0x10_0000_0000 * i for i in range(4))


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ttt_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return ttt.load_library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) >= {"ttt_linear_forward", "ttt_mlp_forward", "ttt_linear_decode_step",
                          "ttt_linear_backward", "ttt_linear_forward_ex", "ttt_linear_segments",
                          "ttt_linear_backward_segments", "ttt_linear_decode_step_ex",
                          "ttt_linear_workspace_bytes", "ttt_linear_backward_workspace_bytes",
                          "ttt_status_string", "ttt_roof_copy", "ttt_roof_mfma", "ttt_roof_launch",
                          "ttt_linear_forward_noalloc", "ttt_linear_noalloc_max_workspace_bytes",
                          "ttt_linear_momentum_segments", "ttt_linear_fused",
                          "ttt_abi_version"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ttt.h but not exported"


def test_status_strings_and_version(lib):
    for s in (OK, INVALID, UNSUPPORTED, ttt.TTT_ERR_HIP, 12345):
        assert isinstance(ttt.status_string(s), str) and ttt.status_string(s)
    assert lib.ttt_abi_version() >> 16 == 2


# a fake workspace address apart from every other one
WSA = 0x300_0000_0000


def lin(lib, Q=QA, K=KA, V=VA, dt=1, W0=W0A, pb=0, eta=ETA, B=2, H=3, T=64, d=64, b=16,
        Y=YA, Wo=WOA, ws=None, wsb=0):
    return lib.ttt_linear_forward(Q, K, V, dt, W0, pb, eta, B, H, T, d, b, Y, Wo, ws, wsb, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), INVALID), (dict(H=-2), INVALID), (dict(T=-5), INVALID),
    (dict(b=0), INVALID), (dict(pb=2), INVALID),
    (dict(Q=None), INVALID), (dict(K=None), INVALID), (dict(V=None), INVALID),
    (dict(Y=None), INVALID), (dict(W0=None), INVALID), (dict(eta=None), INVALID),
    (dict(Wo=None), INVALID),
    (dict(d=48), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(b=65), UNSUPPORTED),
    (dict(dt=7), UNSUPPORTED), (dict(d=128, b=64, dt=0), UNSUPPORTED),  # > 160 KB of LDS
    (dict(Y=QA), INVALID), (dict(Y=KA + 64), INVALID), (dict(Y=VA), INVALID),
    (dict(Y=WOA), INVALID), (dict(Wo=QA), INVALID), (dict(Wo=W0A), INVALID),
    (dict(Wo=W0A + 4, pb=1), INVALID),
    (dict(B=0), OK), (dict(H=0), OK),
    # the caller's workspace
    (dict(wsb=-1), INVALID), (dict(ws=None, wsb=4096), INVALID),
    (dict(ws=QA + 128, wsb=4096), INVALID), (dict(ws=WOA - 64, wsb=4096), INVALID),
    (dict(ws=YA, wsb=1), INVALID),
    # sequence length beyond the 32-bit token index; more chains than a grid holds
    (dict(T=2**31), UNSUPPORTED), (dict(B=2**20 + 1, H=1, T=1), UNSUPPORTED),
])
def test_linear_validation(lib, kw, expect):
    assert lin(lib, **kw) == expect


TOKA, LNQA, LNKA = (0xC0_0000_0000 + 0x10_0000_0000 * i for i in range(3))


def linx(lib, tok=TOKA, lnq=LNQA, lnk=LNKA, eps=1e-5, rm=0, d=64, b=16, Y=YA, Wo=WOA, T=64, dt=1,
         B=2):
    return lib.ttt_linear_forward_ex(QA, KA, VA, dt, W0A, 0, ETA, tok, lnq, lnk, eps, rm, B, 3, T,
                                     d, b, Y, Wo, None, 0, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(eps=0.0), INVALID), (dict(eps=-1.0), INVALID), (dict(eps=float("nan")), INVALID),
    (dict(d=32), UNSUPPORTED), (dict(b=8), UNSUPPORTED), (dict(d=32, tok=None), UNSUPPORTED),
    (dict(Y=TOKA), INVALID), (dict(Wo=LNKA + 64), INVALID), (dict(Y=LNQA), INVALID),
    (dict(rm=2), INVALID), (dict(rm=-1), INVALID),
    (dict(tok=None, lnq=None, lnk=None, rm=1, d=32), UNSUPPORTED),
    (dict(B=0), OK),
    # eps is not checked when no LayerNorm is asked for; every prologue pointer
    # NULL falls back to the plain forward's rules
    (dict(lnq=None, lnk=None, eps=0.0, B=0), OK),
    (dict(tok=None, lnq=None, lnk=None, d=48), UNSUPPORTED),
])
def test_linear_forward_ex_validation(lib, kw, expect):
    assert linx(lib, **kw) == expect


def test_linear_no_inputs_needed_when_empty(lib):
    # B*H == 0: a no-op, even with null pointers
    assert lib.ttt_linear_forward(None, None, None, 1, None, 0, None, 0, 4, 8, 64, 16,
                                  None, None, None, 0, None) == OK


def mlp(lib, dt=1, W1=W1A, W2=W2A, pb=0, B=2, H=3, T=64, d=64, m=256, b=16, Y=YA,
        W1o=W1O, W2o=W2O, Q=QA):
    return lib.ttt_mlp_forward(Q, KA, VA, dt, W1, W2, pb, ETA, B, H, T, d, m, b, Y, W1o, W2o,
                               None)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), INVALID), (dict(b=0), INVALID), (dict(m=0), INVALID),
    (dict(W1=None), INVALID), (dict(W2o=None), INVALID), (dict(Q=None), INVALID),
    (dict(d=128), UNSUPPORTED), (dict(m=100), UNSUPPORTED), (dict(m=1024), UNSUPPORTED),
    (dict(dt=3), UNSUPPORTED), (dict(b=80), UNSUPPORTED),
    (dict(Y=W1A), INVALID), (dict(W1o=W2O), INVALID), (dict(W1o=W1A), INVALID),
    (dict(B=0), OK), (dict(T=2**31), UNSUPPORTED),
])
def test_mlp_validation(lib, kw, expect):
    assert mlp(lib, **kw) == expect


def dec(lib, q=QA, W=W0A, y=YA, dt=1, B=2, H=24, d=64):
    return lib.ttt_linear_decode_step(q, KA, VA, dt, W, ETA, B, H, d, y, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), INVALID), (dict(q=None), INVALID), (dict(W=None), INVALID),
    (dict(y=None), INVALID), (dict(d=96), UNSUPPORTED), (dict(dt=9), UNSUPPORTED),
    (dict(y=QA), INVALID), (dict(y=W0A), INVALID), (dict(W=KA), INVALID),
    (dict(B=0), OK), (dict(B=2**20, H=2), UNSUPPORTED),
    # rows of q, k and W are read with 16-byte loads
    (dict(q=QA + 8), INVALID), (dict(W=W0A + 4), INVALID),
])
def test_decode_validation(lib, kw, expect):
    assert dec(lib, **kw) == expect


DYA, DWOA, DQA, DKA, DVA, DW0A, DETA = (0xA0_0000_0000 + 0x10_0000_0000 * i for i in range(7))


def bwd(lib, Q=QA, dt=1, W0=W0A, pb=0, eta=ETA, B=2, H=3, T=64, d=64, b=16, dY=DYA, dWo=DWOA,
        dQ=DQA, dK=DKA, dV=DVA, dW0=DW0A, deta=DETA, ws=WSA, wsb=1 << 30):
    return lib.ttt_linear_backward(Q, KA, VA, dt, W0, pb, eta, B, H, T, d, b, dY, dWo, dQ, dK, dV,
                                   dW0, deta, ws, wsb, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), INVALID), (dict(T=-1), INVALID), (dict(b=0), INVALID), (dict(pb=3), INVALID),
    (dict(Q=None), INVALID), (dict(dY=None), INVALID), (dict(dWo=None), INVALID),
    (dict(dQ=None), INVALID), (dict(dW0=None), INVALID), (dict(deta=None), INVALID),
    (dict(W0=None), INVALID), (dict(eta=None), INVALID),
    (dict(d=32), UNSUPPORTED), (dict(b=8), UNSUPPORTED), (dict(dt=5), UNSUPPORTED),
    (dict(dQ=QA), INVALID), (dict(dK=DQA + 8), INVALID), (dict(dV=DYA), INVALID),
    (dict(dW0=DWOA), INVALID), (dict(deta=ETA), INVALID), (dict(dW0=W0A), INVALID),
    (dict(deta=DW0A + 16), INVALID),
    (dict(H=0), OK),
    # the caller's workspace: required (the chunk-start states), never overlapping
    (dict(wsb=-8), INVALID), (dict(ws=None), INVALID), (dict(ws=None, wsb=0), INVALID),
    (dict(wsb=1000), INVALID), (dict(ws=DQA - 4096), INVALID), (dict(ws=QA), INVALID),
    # the kernels' 32-bit byte offsets bound a chain's length
    (dict(T=2**24), UNSUPPORTED), (dict(T=2**31), UNSUPPORTED),
])
def test_backward_validation(lib, kw, expect):
    assert bwd(lib, **kw) == expect


# prologue inputs and their gradients, apart from every address above
PTOKA, PLNQA, PLNKA, DTOKA, DLNQA, DLNKA = (0x200_0000_0000 + 0x10_0000_0000 * i for i in range(6))


def bwdx(lib, tok=PTOKA, lnq=PLNQA, lnk=PLNKA, eps=1e-5, rm=0, dtok=DTOKA, dlnq=DLNQA, dlnk=DLNKA,
         d=64, b=16, H=3, dQ=DQA, deta=DETA):
    return lib.ttt_linear_backward_ex(QA, KA, VA, 1, W0A, 0, ETA, tok, lnq, lnk, eps, rm, 2, H, 64,
                                      d, b, DYA, DWOA, dQ, DKA, DVA, DW0A, deta, dtok, dlnq, dlnk,
                                      WSA, 1 << 30, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(eps=0.0), INVALID), (dict(eps=float("inf")), INVALID), (dict(rm=2), INVALID),
    # every prologue input comes with its gradient output and the reverse
    (dict(dtok=None), INVALID), (dict(tok=None), INVALID), (dict(dlnq=None), INVALID),
    (dict(lnk=None), INVALID), (dict(tok=None, dtok=None, lnq=None, dlnq=None, d=32), UNSUPPORTED),
    (dict(d=32), UNSUPPORTED), (dict(b=8), UNSUPPORTED),
    (dict(dtok=PTOKA), INVALID), (dict(dlnq=PLNQA + 4), INVALID), (dict(dlnk=DLNQA + 8), INVALID),
    (dict(dtok=DQA + 64), INVALID), (dict(dQ=DLNKA), INVALID), (dict(deta=DTOKA + 4), INVALID),
    (dict(H=0), OK), (dict(lnq=None, dlnq=None, lnk=None, dlnk=None, eps=0.0, H=0), OK),
])
def test_backward_ex_validation(lib, kw, expect):
    assert bwdx(lib, **kw) == expect


def test_backward_ex_fixture_addresses_are_disjoint():
    # the valid default call of bwdx must not overlap itself, so that each
    # INVALID case above fails for its own reason
    spans = [(a, 0x10_0000_0000) for a in (QA, KA, VA, W0A, ETA, DYA, DWOA, DQA, DKA, DVA, DW0A,
                                           DETA, PTOKA, PLNQA, PLNKA, DTOKA, DLNQA, DLNKA, WSA)]
    spans.sort()
    for (a, n), (b, _) in zip(spans, spans[1:]):
        assert a + n <= b


def decx(lib, tok=TOKA, lnq=LNQA, lnk=LNKA, eps=1e-5, rm=0, d=64, y=YA, W=W0A, B=2):
    return lib.ttt_linear_decode_step_ex(QA, KA, VA, 1, W, ETA, tok, lnq, lnk, eps, rm, B, 24, d,
                                         y, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(eps=0.0), INVALID), (dict(rm=3), INVALID), (dict(d=96), UNSUPPORTED),
    (dict(y=TOKA), INVALID), (dict(W=LNQA), INVALID), (dict(y=LNKA + 100), INVALID),
    (dict(B=0), OK), (dict(lnq=None, lnk=None, eps=-1.0, B=0), OK),
])
def test_decode_ex_validation(lib, kw, expect):
    assert decx(lib, **kw) == expect


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 16, 16)
    with pytest.raises((ValueError, TypeError, RuntimeError)):
        ttt.ttt_linear_forward(x, x, x, torch.zeros(1, 16, 16), torch.zeros(1), 16,
                               Y=torch.zeros(1, 1, 16, 16), W_out=torch.zeros(1, 1, 16, 16),
                               stream=None)


def test_segment_query_validation_and_override(lib, monkeypatch):
    """The segment-count query validates like ttt_linear_forward; the
    TTT_LINEAR_SEGMENTS override is applied (clamped to 30, at least one
    mini-batch per segment) before any device query."""
    assert lib.ttt_linear_segments(-1, 3, 64, 64, 16, 1) == INVALID
    assert lib.ttt_linear_segments(1, 3, 64, 64, 0, 1) == INVALID
    assert lib.ttt_linear_segments(1, 3, 64, 48, 16, 1) == UNSUPPORTED
    assert lib.ttt_linear_segments(1, 3, 64, 64, 16, 7) == UNSUPPORTED
    assert lib.ttt_linear_segments(0, 3, 64, 64, 16, 1) == 1
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "4")
    assert lib.ttt_linear_segments(1, 4, 2048, 64, 16, 0) == 4
    assert lib.ttt_linear_segments(1, 4, 16, 64, 16, 0) == 1       # one mini-batch
    assert lib.ttt_linear_segments(1, 4, 40, 64, 16, 1) == 3       # 3 chunks, one each
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "50")
    # clamped to 30: 128 chunks in segments of ceil(128 / 30) = 5 -> 26 segments
    assert lib.ttt_linear_segments(1, 4, 2048, 64, 16, 0) == 26
    assert lib.ttt_linear_segments(1, 4, 30 * 16, 64, 16, 0) == 30
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "3")
    assert lib.ttt_linear_segments(1, 4, 2048, 32, 16, 0) == 1     # generic kernel: no split


def test_fused_layout_query(lib, monkeypatch):
    """ttt_linear_fused validates like ttt_linear_segments; with a forced
    segment count of 3 or more the bf16 d = 64, b = 16 forward takes the
    fused layout (same count, same workspace), unless TTT_LINEAR_FUSED=0;
    fp32, other shapes and two segments never do."""
    assert lib.ttt_linear_fused(-1, 3, 64, 64, 16, 1) == INVALID
    assert lib.ttt_linear_fused(1, 3, 64, 48, 16, 1) == UNSUPPORTED
    assert lib.ttt_linear_fused(0, 3, 64, 64, 16, 1) == 0
    monkeypatch.delenv("TTT_LINEAR_FUSED", raising=False)
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "6")
    assert lib.ttt_linear_fused(2, 24, 32768, 64, 16, 1) == 1
    assert lib.ttt_linear_segments(2, 24, 32768, 64, 16, 1) == 6
    assert lib.ttt_linear_workspace_bytes(2, 24, 32768, 64, 16, 1) == 48 * (3 * 6 - 2) * 64 * 64 * 4
    assert lib.ttt_linear_fused(2, 24, 32768, 64, 16, 0) == 0      # fp32
    assert lib.ttt_linear_fused(2, 24, 32768, 32, 16, 1) == 0      # generic kernel
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "2")
    assert lib.ttt_linear_fused(2, 24, 32768, 64, 16, 1) == 0
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "6")
    monkeypatch.setenv("TTT_LINEAR_FUSED", "0")
    assert lib.ttt_linear_fused(2, 24, 32768, 64, 16, 1) == 0
    assert lib.ttt_linear_segments(2, 24, 32768, 64, 16, 1) == 6


def test_backward_segment_query_validation_and_override(lib, monkeypatch):
    """Same contract for the backward's segment count (TTT_LINEAR_BWD_SEGMENTS)."""
    assert lib.ttt_linear_backward_segments(-1, 3, 64, 64, 16, 1) == INVALID
    assert lib.ttt_linear_backward_segments(1, 3, 64, 64, 0, 1) == INVALID
    assert lib.ttt_linear_backward_segments(1, 3, 64, 32, 16, 1) == UNSUPPORTED
    assert lib.ttt_linear_backward_segments(1, 3, 64, 64, 8, 1) == UNSUPPORTED
    assert lib.ttt_linear_backward_segments(1, 3, 64, 64, 16, 4) == UNSUPPORTED
    assert lib.ttt_linear_backward_segments(0, 3, 64, 64, 16, 1) == 1
    assert lib.ttt_linear_backward_segments(2, 3, 0, 64, 16, 1) == 1
    monkeypatch.setenv("TTT_LINEAR_BWD_SEGMENTS", "7")
    assert lib.ttt_linear_backward_segments(1, 4, 1000, 64, 16, 0) == 7   # 63 chunks, 9 each
    assert lib.ttt_linear_backward_segments(1, 4, 40, 64, 16, 1) == 3
    monkeypatch.setenv("TTT_LINEAR_BWD_SEGMENTS", "99")
    assert lib.ttt_linear_backward_segments(1, 4, 2048, 64, 16, 1) == 26


def test_workspace_queries(lib, monkeypatch):
    """Workspace sizes: the forward needs B*H*(3S - 2) d x d fp32 matrices for S
    segments (none unsegmented); the backward's figure covers the chunk-start
    states (bf16 W^T for bf16 inputs, fp32 W otherwise), a per-chain dW0 and
    the small per-segment sums, each piece padded to 256 bytes."""
    monkeypatch.delenv("TTT_LINEAR_SEGMENTS", raising=False)
    monkeypatch.delenv("TTT_LINEAR_BWD_SEGMENTS", raising=False)
    assert lib.ttt_linear_workspace_bytes(-1, 3, 64, 64, 16, 1) == INVALID
    assert lib.ttt_linear_workspace_bytes(1, 3, 64, 48, 16, 1) == UNSUPPORTED
    assert lib.ttt_linear_workspace_bytes(1, 3, 2**31, 64, 16, 1) == UNSUPPORTED
    assert lib.ttt_linear_workspace_bytes(0, 3, 64, 64, 16, 1) == 0
    assert lib.ttt_linear_workspace_bytes(1, 3, 64, 32, 16, 1) == 0        # generic kernel
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "4")
    assert lib.ttt_linear_workspace_bytes(1, 4, 2048, 64, 16, 0) == 4 * (3 * 4 - 2) * 64 * 64 * 4
    assert lib.ttt_linear_workspace_bytes(2, 3, 2048, 64, 16, 1) == 6 * (3 * 4 - 2) * 64 * 64 * 4
    assert lib.ttt_linear_workspace_bytes(1, 4, 16, 64, 16, 0) == 0        # one mini-batch

    assert lib.ttt_linear_backward_workspace_bytes(1, 3, 64, 32, 16, 1) == UNSUPPORTED
    monkeypatch.setenv("TTT_LINEAR_BWD_SEGMENTS", "1")
    st = 64 * 64 * 4
    units, chunks = 2, 4
    pad = lambda n: (n + 255) // 256 * 256
    small = pad(units * 4) + pad(units * 4 * 64 * 4)     # deta per segment, LayerNorm sums
    # per chunk: fp32 W (fp32 inputs); bf16 inputs keep the update operand E',
    # 256 threads x 8 bytes, from which the kernel walks the states back
    for dt, state in ((1, 256 * 8), (0, st)):
        want = pad(units * chunks * state) + pad(units * st) + small
        assert lib.ttt_linear_backward_workspace_bytes(1, 2, 64, 64, 16, dt) == want
    # the plain call with shared W0 needs the states, dW0 per chain and deta
    # (no LayerNorm sums); one byte short of that is rejected before any launch
    need = pad(units * chunks * 256 * 8) + pad(units * st) + pad(units * 4)
    assert bwd(lib, B=1, H=2, ws=WSA, wsb=need - 1) == INVALID


def test_roof_probe_validation(lib):
    """The roof kernels reject bad arguments before any launch."""
    lib.ttt_roof_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.ttt_roof_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_void_p, ctypes.c_void_p]
    assert lib.ttt_roof_copy(None, YA, 1024, None) == INVALID
    assert lib.ttt_roof_copy(QA, YA, 1000, None) == INVALID          # not a multiple of 16
    assert lib.ttt_roof_copy(QA + 4, YA, 1024, None) == INVALID      # unaligned
    assert lib.ttt_roof_copy(QA, QA + 512, 1024, None) == INVALID    # overlapping
    assert lib.ttt_roof_copy(QA, YA, 0, None) == OK
    assert lib.ttt_roof_mfma(None, 1, 1024, 10, None, None) == INVALID
    assert lib.ttt_roof_mfma(YA, 2, 1024, 10, None, None) == INVALID
    assert lib.ttt_roof_mfma(YA, 1, 1022, 10, None, None) == INVALID
    assert lib.ttt_roof_mfma(YA, 0, 1024, 0, None, None) == INVALID
    lib.ttt_roof_launch.argtypes = [ctypes.c_int64, ctypes.c_void_p]
    assert lib.ttt_roof_launch(0, None) == INVALID
    assert lib.ttt_roof_launch(1 << 31, None) == INVALID


def test_noalloc_validation_and_limit(lib, monkeypatch):
    """The entry point without allocation validates like ttt_linear_forward and
    rejects sizes whose plan needs more than its static scratch (16 MiB)
    before any HIP call."""
    f = lib.ttt_linear_forward_noalloc
    lib.ttt_linear_noalloc_max_workspace_bytes.restype = ctypes.c_int64
    assert lib.ttt_linear_noalloc_max_workspace_bytes() == 16 << 20

    def na(**kw):
        a = dict(Q=QA, K=KA, V=VA, dt=1, W0=W0A, pb=0, eta=ETA, B=2, H=24, T=32768, d=64, b=16,
                 Y=YA, Wo=WOA)
        a.update(kw)
        return f(a["Q"], a["K"], a["V"], a["dt"], a["W0"], a["pb"], a["eta"], a["B"], a["H"],
                 a["T"], a["d"], a["b"], a["Y"], a["Wo"], None)
    assert na(Q=None) == INVALID and na(Y=QA) == INVALID and na(d=48) == UNSUPPORTED
    assert na(B=0) == OK
    # 30 forced segments of 48 chains: 48 * 88 matrices of 16 KB = 69 MB > 16 MiB
    monkeypatch.setenv("TTT_LINEAR_SEGMENTS", "30")
    assert na() == UNSUPPORTED


MOA, M0A, BETA = (0xD0_0000_0000 + 0x10_0000_0000 * i for i in range(3))


def mom(lib, Q=QA, K=KA, V=VA, dt=1, W0=W0A, pb=0, M0=M0A, eta=ETA, beta=BETA, gm=0, B=2, H=3,
        T=64, d=64, b=16, Y=YA, Wo=WOA, Mo=MOA, ws=WSA, wsb=1 << 20):
    return lib.ttt_linear_momentum_forward(Q, K, V, dt, W0, pb, M0, eta, beta, gm, B, H, T, d, b,
                                           Y, Wo, Mo, ws, wsb, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), INVALID), (dict(T=-1), INVALID), (dict(b=0), INVALID), (dict(pb=2), INVALID),
    (dict(gm=2), INVALID), (dict(gm=-1), INVALID),
    (dict(Q=None), INVALID), (dict(Y=None), INVALID), (dict(W0=None), INVALID),
    (dict(eta=None), INVALID), (dict(beta=None), INVALID), (dict(Wo=None), INVALID),
    (dict(Mo=None), INVALID),
    (dict(d=48), UNSUPPORTED), (dict(b=65), UNSUPPORTED), (dict(dt=5), UNSUPPORTED),
    (dict(d=128, b=21, dt=0), UNSUPPORTED), (dict(T=2**31), UNSUPPORTED),
    # overlaps: outputs with inputs, the two outputs, the workspace
    (dict(Y=QA), INVALID), (dict(Mo=KA), INVALID), (dict(Mo=WOA + 64), INVALID),
    (dict(Wo=M0A), INVALID), (dict(Mo=BETA), INVALID), (dict(Wo=BETA - 4), INVALID),
    (dict(ws=VA), INVALID), (dict(ws=MOA - 64), INVALID), (dict(ws=M0A), INVALID),
    (dict(Mo=M0A + 4), INVALID), (dict(Wo=W0A), INVALID),
    (dict(wsb=-1), INVALID), (dict(ws=None, wsb=16), INVALID),
    # in place: W_out = W0 (per batch), M_out = M0; no start momentum
    (dict(Wo=W0A, pb=1, B=0), OK), (dict(M0=None, B=0), OK), (dict(B=0, Q=None), OK),
])
def test_momentum_validation(lib, kw, expect):
    assert mom(lib, **kw) == expect


def test_momentum_workspace_query(lib):
    q = lib.ttt_linear_momentum_workspace_bytes
    assert q(-1, 3, 64, 64, 16, 1, 0) == INVALID
    assert q(1, 3, 64, 64, 16, 1, 2) == INVALID
    assert q(1, 3, 64, 48, 16, 1, 0) == UNSUPPORTED
    assert q(1, 3, 64, 128, 32, 0, 0) == UNSUPPORTED
    for args in ((1, 3, 64, 64, 16, 1, 1), (1, 3, 64, 64, 16, 0, 0), (1, 3, 64, 32, 16, 1, 0),
                 (1, 3, 64, 64, 8, 1, 0)):
        assert q(*args) == 0          # chunk-start gradients, or the plain fp32 kernel
    # exact steps on the bf16 MFMA path: 512-byte inverses, one per chunk of 16
    # tokens, stored in pairs (T = 100: 7 chunks in 4 pairs)
    assert q(2, 3, 100, 64, 16, 1, 0) == 6 * 4 * 1024
    assert q(0, 3, 100, 64, 16, 1, 0) == 0
    # one byte short of that is rejected before any launch
    assert mom(lib, B=2, H=3, T=100, ws=WSA, wsb=6 * 4 * 1024 - 1) == INVALID


def test_momentum_segments_query_and_workspace(lib, monkeypatch):
    """Without a GPU the plan has one segment; a forced split of whole
    stages of 32 tokens adds the maps (6 d^2 floats each) and start states
    (2 d^2 floats each) to the documented workspace."""
    seg = lib.ttt_linear_momentum_segments
    q = lib.ttt_linear_momentum_workspace_bytes
    assert seg(2, 3, 1000, 64, 16, 1, 0) == 1
    assert seg(2, 3, 1000, 48, 16, 1, 0) == UNSUPPORTED
    assert seg(2, 3, 1000, 64, 16, 1, 5) == INVALID
    monkeypatch.setenv("TTT_MOMENTUM_SEGMENTS", "5")
    pad = lambda n: (n + 255) // 256 * 256
    units, d = 6, 64
    for gm in (0, 1):
        # T = 1000: 32 stages, 7 per segment, so 5 segments
        assert seg(2, 3, 1000, 64, 16, 1, gm) == 5
        pinv = units * 32 * 1024 if gm == 0 else 0
        want = pinv + pad(units * 4 * 6 * d * d * 4) + units * 5 * 2 * d * d * 4
        assert q(2, 3, 1000, 64, 16, 1, gm) == want
    # forced beyond the stages: one segment per stage (T = 64: two)
    assert seg(1, 1, 64, 64, 16, 1, 0) == 2
    # only the bf16 MFMA path splits
    assert seg(2, 3, 1000, 64, 16, 0, 0) == 1
    assert seg(2, 3, 1000, 32, 16, 1, 0) == 1
