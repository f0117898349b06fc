"""Python binding of libttt.so: the TTT forward scan on MI355X (gfx950).

Argument marshalling only.  Every step of the scan runs in the HIP kernels
behind the C ABI declared in include/ttt.h; this module checks tensor
properties, allocates outputs and workspaces with torch (device memory only)
and passes raw device pointers plus the current HIP stream.  There is no CPU fallback: if
libttt.so is missing or a call fails, an exception is raised.

Functions (same names as the C ABI):
    ttt_linear_forward(Q, K, V, W0, eta, b)           -> (Y, W_out)
    ttt_linear_forward_ex(Q, K, V, W0, eta, b, eta_tok, ln_q, ln_k, ln_eps)
                                                      -> (Y, W_out)
    ttt_mlp_forward(Q, K, V, W1, W2, eta, b)          -> (Y, W1_out, W2_out)
    ttt_linear_decode_step(q, k, v, W, eta)           -> y   (W updated in place)
    ttt_linear_backward(Q, K, V, W0, eta, b, dY, dW_out)
                                                      -> (dQ, dK, dV, dW0, deta)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libttt.so")

TTT_F32 = 0
TTT_BF16 = 1
TTT_OK = 0
TTT_ERR_INVALID_ARG = -1
TTT_ERR_UNSUPPORTED = -2
TTT_ERR_HIP = -3

_lib = None


class TTTError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def load_library():
    """Load libttt.so (built in place by test_sequence_layers_linear_amd/build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                           "or python test_sequence_layers_linear_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.ttt_linear_forward.argtypes = [P, P, P, I, P, I, P, L, L, L, I, I, P, P, P, L, P]
    lib.ttt_linear_forward.restype = I
    lib.ttt_linear_forward_ex.argtypes = [P, P, P, I, P, I, P, P, P, P, ctypes.c_float, I,
                                          L, L, L, I, I, P, P, P, L, P]
    lib.ttt_linear_forward_ex.restype = I
    lib.ttt_mlp_forward.argtypes = [P, P, P, I, P, P, I, P, L, L, L, I, I, I, P, P, P, P]
    lib.ttt_mlp_forward.restype = I
    lib.ttt_linear_decode_step.argtypes = [P, P, P, I, P, P, L, L, I, P, P]
    lib.ttt_linear_decode_step.restype = I
    lib.ttt_linear_decode_step_ex.argtypes = [P, P, P, I, P, P, P, P, P, ctypes.c_float, I,
                                              L, L, I, P, P]
    lib.ttt_linear_decode_step_ex.restype = I
    lib.ttt_linear_backward.argtypes = [P, P, P, I, P, I, P, L, L, L, I, I, P, P,
                                        P, P, P, P, P, P, L, P]
    lib.ttt_linear_backward.restype = I
    lib.ttt_linear_backward_ex.argtypes = [P, P, P, I, P, I, P, P, P, P, ctypes.c_float, I,
                                           L, L, L, I, I, P, P, P, P, P, P, P, P, P, P, P, L, P]
    lib.ttt_linear_backward_ex.restype = I
    lib.ttt_linear_backward_segments.argtypes = [L, L, L, I, I, I]
    lib.ttt_linear_backward_segments.restype = I
    lib.ttt_linear_segments.argtypes = [L, L, L, I, I, I]
    lib.ttt_linear_segments.restype = I
    lib.ttt_linear_fused.argtypes = [L, L, L, I, I, I]
    lib.ttt_linear_fused.restype = I
    lib.ttt_linear_forward_noalloc.argtypes = [P, P, P, I, P, I, P, L, L, L, I, I, P, P, P]
    lib.ttt_linear_forward_noalloc.restype = I
    lib.ttt_linear_noalloc_max_workspace_bytes.argtypes = []
    lib.ttt_linear_noalloc_max_workspace_bytes.restype = L
    lib.ttt_linear_workspace_bytes.argtypes = [L, L, L, I, I, I]
    lib.ttt_linear_workspace_bytes.restype = L
    lib.ttt_linear_backward_workspace_bytes.argtypes = [L, L, L, I, I, I]
    lib.ttt_linear_backward_workspace_bytes.restype = L
    lib.ttt_linear_momentum_forward.argtypes = [P, P, P, I, P, I, P, P, P, I, L, L, L, I, I,
                                                P, P, P, P, L, P]
    lib.ttt_linear_momentum_forward.restype = I
    lib.ttt_linear_momentum_workspace_bytes.argtypes = [L, L, L, I, I, I, I]
    lib.ttt_linear_momentum_workspace_bytes.restype = L
    lib.ttt_linear_momentum_segments.argtypes = [L, L, L, I, I, I, I]
    lib.ttt_linear_momentum_segments.restype = I
    lib.ttt_status_string.argtypes = [I]
    lib.ttt_status_string.restype = ctypes.c_char_p
    lib.ttt_abi_version.argtypes = []
    lib.ttt_abi_version.restype = I
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ttt_status_string(int(status)).decode()


def _check(status: int):
    if status != TTT_OK:
        raise TTTError(status, status_string(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TTT_F32
    if t.dtype == torch.bfloat16:
        return TTT_BF16
    raise TypeError(f"Q/K/V must be float32 or bfloat16, got {t.dtype}")


def _need(t: torch.Tensor, name: str, device, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be in GPU memory (got {t.device})")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, device, workspace):
    """The workspace tensor of a call: the caller's (uint8, on the device,
    at least nbytes) or a new torch allocation of nbytes."""
    if nbytes < 0:
        _check(nbytes)
    if workspace is None:
        return torch.empty(max(int(nbytes), 0), dtype=torch.uint8, device=device)
    _need(workspace, "workspace", device, torch.uint8)
    return workspace


def _ws_args(ws):
    return (ws.data_ptr() if ws.numel() else None), ws.numel()


def _stream_handle(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def ttt_linear_forward(Q, K, V, W0, eta, b: int, Y=None, W_out=None, workspace=None,
                       stream=None):
    """TTT-Linear dual-form forward.  Q,K,V [B,H,T,d] fp32/bf16 on a GPU;
    W0 fp32 [H,d,d] (shared over the batch) or [B,H,d,d]; eta fp32 [H].
    workspace: a uint8 device tensor for the segment maps (None: one of
    ttt_linear_workspace_bytes bytes is allocated with torch).
    Returns (Y [B,H,T,d] in Q's dtype, W_out fp32 [B,H,d,d])."""
    lib = load_library()
    if Q.dim() != 4:
        raise ValueError("Q must be [B,H,T,d]")
    dev = Q.device
    B, H, T, d = Q.shape
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, n, dev, Q.dtype)
        if t.shape != Q.shape:
            raise ValueError(f"{n} shape {tuple(t.shape)} != Q shape {tuple(Q.shape)}")
    _need(W0, "W0", dev, torch.float32)
    _need(eta, "eta", dev, torch.float32)
    per_batch = W0.dim() == 4
    if W0.shape != ((B, H, d, d) if per_batch else (H, d, d)) or eta.shape != (H,):
        raise ValueError("W0 must be [H,d,d] or [B,H,d,d] and eta [H]")
    if Y is None:
        Y = torch.empty_like(Q)
    if W_out is None:
        W_out = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    _need(Y, "Y", dev, Q.dtype)
    _need(W_out, "W_out", dev, torch.float32)
    ws = _workspace(lib.ttt_linear_workspace_bytes(B, H, T, d, int(b), _dtype_code(Q))
                    if workspace is None else 0, dev, workspace)
    _check(lib.ttt_linear_forward(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q),
                                  W0.data_ptr(), int(per_batch), eta.data_ptr(),
                                  B, H, T, d, int(b), Y.data_ptr(), W_out.data_ptr(),
                                  *_ws_args(ws), _stream_handle(dev, stream)))
    return Y, W_out


def ttt_linear_forward_noalloc(Q, K, V, W0, eta, b: int, Y, W_out, stream=None):
    """ttt_linear_forward through the entry point that allocates nothing: the
    segment maps live in the library's static device scratch.  Y and W_out
    must be given (preallocated).  Calls that overlap on one device race on
    that scratch."""
    lib = load_library()
    if Q.dim() != 4:
        raise ValueError("Q must be [B,H,T,d]")
    dev = Q.device
    B, H, T, d = Q.shape
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, n, dev, Q.dtype)
        if t.shape != Q.shape:
            raise ValueError(f"{n} shape {tuple(t.shape)} != Q shape {tuple(Q.shape)}")
    _need(W0, "W0", dev, torch.float32)
    _need(eta, "eta", dev, torch.float32)
    per_batch = W0.dim() == 4
    if W0.shape != ((B, H, d, d) if per_batch else (H, d, d)) or eta.shape != (H,):
        raise ValueError("W0 must be [H,d,d] or [B,H,d,d] and eta [H]")
    _need(Y, "Y", dev, Q.dtype)
    _need(W_out, "W_out", dev, torch.float32)
    if Y.shape != Q.shape or W_out.shape != (B, H, d, d):
        raise ValueError("Y must be shaped like Q and W_out [B,H,d,d]")
    _check(lib.ttt_linear_forward_noalloc(Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                                          _dtype_code(Q), W0.data_ptr(), int(per_batch),
                                          eta.data_ptr(), B, H, T, d, int(b), Y.data_ptr(),
                                          W_out.data_ptr(), _stream_handle(dev, stream)))
    return Y, W_out


def ttt_linear_forward_ex(Q, K, V, W0, eta, b: int, eta_tok=None, ln_q=None, ln_k=None,
                          ln_eps: float = 1e-5, read_chunk_start: bool = False, Y=None,
                          W_out=None, workspace=None, stream=None):
    """ttt_linear_forward with the input prologue: q and k LayerNorm'd over
    the head dim (ln_q / ln_k fp32 [H,2,d]: gamma, beta) and a step size per
    token (eta_tok fp32 [B,H,T]); None leaves that part out.
    read_chunk_start: tokens read out with their mini-batch's start weights."""
    lib = load_library()
    if Q.dim() != 4:
        raise ValueError("Q must be [B,H,T,d]")
    dev = Q.device
    B, H, T, d = Q.shape
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, n, dev, Q.dtype)
        if t.shape != Q.shape:
            raise ValueError(f"{n} shape {tuple(t.shape)} != Q shape {tuple(Q.shape)}")
    _need(W0, "W0", dev, torch.float32)
    _need(eta, "eta", dev, torch.float32)
    per_batch = W0.dim() == 4
    if W0.shape != ((B, H, d, d) if per_batch else (H, d, d)) or eta.shape != (H,):
        raise ValueError("W0 must be [H,d,d] or [B,H,d,d] and eta [H]")
    ptrs = []
    for t, n, shape in ((eta_tok, "eta_tok", (B, H, T)), (ln_q, "ln_q", (H, 2, d)),
                        (ln_k, "ln_k", (H, 2, d))):
        if t is None:
            ptrs.append(None)
            continue
        _need(t, n, dev, torch.float32)
        if t.shape != shape:
            raise ValueError(f"{n} must be {list(shape)}, got {tuple(t.shape)}")
        ptrs.append(t.data_ptr())
    if Y is None:
        Y = torch.empty_like(Q)
    if W_out is None:
        W_out = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    _need(Y, "Y", dev, Q.dtype)
    _need(W_out, "W_out", dev, torch.float32)
    ws = _workspace(lib.ttt_linear_workspace_bytes(B, H, T, d, int(b), _dtype_code(Q))
                    if workspace is None else 0, dev, workspace)
    _check(lib.ttt_linear_forward_ex(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q),
                                     W0.data_ptr(), int(per_batch), eta.data_ptr(), ptrs[0],
                                     ptrs[1], ptrs[2], float(ln_eps), int(bool(read_chunk_start)),
                                     B, H, T, d, int(b),
                                     Y.data_ptr(), W_out.data_ptr(), *_ws_args(ws),
                                     _stream_handle(dev, stream)))
    return Y, W_out


def ttt_mlp_forward(Q, K, V, W1, W2, eta, b: int, Y=None, W1_out=None, W2_out=None,
                    stream=None):
    """TTT-MLP dual-form forward, f(z) = SiLU(z W1) W2.  W1 fp32 [H,d,m] or
    [B,H,d,m]; W2 fp32 [H,m,d] or [B,H,m,d].  Returns (Y, W1_out, W2_out)."""
    lib = load_library()
    if Q.dim() != 4:
        raise ValueError("Q must be [B,H,T,d]")
    dev = Q.device
    B, H, T, d = Q.shape
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, n, dev, Q.dtype)
        if t.shape != Q.shape:
            raise ValueError(f"{n} shape {tuple(t.shape)} != Q shape {tuple(Q.shape)}")
    _need(W1, "W1", dev, torch.float32)
    _need(W2, "W2", dev, torch.float32)
    _need(eta, "eta", dev, torch.float32)
    per_batch = W1.dim() == 4
    m = W1.shape[-1]
    lead = (B, H) if per_batch else (H,)
    if W1.shape != lead + (d, m) or W2.shape != lead + (m, d) or eta.shape != (H,):
        raise ValueError("W1 must be [H,d,m] / [B,H,d,m], W2 [H,m,d] / [B,H,m,d], eta [H]")
    if Y is None:
        Y = torch.empty_like(Q)
    if W1_out is None:
        W1_out = torch.empty((B, H, d, m), device=dev, dtype=torch.float32)
    if W2_out is None:
        W2_out = torch.empty((B, H, m, d), device=dev, dtype=torch.float32)
    _need(Y, "Y", dev, Q.dtype)
    _need(W1_out, "W1_out", dev, torch.float32)
    _need(W2_out, "W2_out", dev, torch.float32)
    _check(lib.ttt_mlp_forward(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q),
                               W1.data_ptr(), W2.data_ptr(), int(per_batch), eta.data_ptr(),
                               B, H, T, d, m, int(b), Y.data_ptr(), W1_out.data_ptr(),
                               W2_out.data_ptr(), _stream_handle(dev, stream)))
    return Y, W1_out, W2_out


def ttt_linear_decode_step(q, k, v, W, eta, y=None, stream=None):
    """One TTT-Linear token step: q,k,v [B,H,d] fp32/bf16; W fp32 [B,H,d,d]
    updated in place; eta fp32 [H].  Returns y [B,H,d] in q's dtype."""
    lib = load_library()
    if q.dim() != 3:
        raise ValueError("q must be [B,H,d]")
    dev = q.device
    B, H, d = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dev, q.dtype)
        if t.shape != q.shape:
            raise ValueError(f"{n} shape {tuple(t.shape)} != q shape {tuple(q.shape)}")
    _need(W, "W", dev, torch.float32)
    _need(eta, "eta", dev, torch.float32)
    if W.shape != (B, H, d, d) or eta.shape != (H,):
        raise ValueError("W must be [B,H,d,d] and eta [H]")
    if y is None:
        y = torch.empty_like(q)
    _need(y, "y", dev, q.dtype)
    _check(lib.ttt_linear_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q),
                                      W.data_ptr(), eta.data_ptr(), B, H, d, y.data_ptr(),
                                      _stream_handle(dev, stream)))
    return y


def ttt_linear_backward(Q, K, V, W0, eta, b: int, dY, dW_out=None, dQ=None, dK=None, dV=None,
                        dW0=None, deta=None, workspace=None, stream=None):
    """Gradients of <dY, Y> + <dW_out, W_out> for (Y, W_out) =
    ttt_linear_forward(Q, K, V, W0, eta, b), with respect to Q, K, V, W0 and
    eta.  dY has Q's shape and dtype; dW_out fp32 [B,H,d,d] (None: zeros).
    Returns (dQ, dK, dV in Q's dtype, dW0 fp32 shaped like W0 (summed over the
    batch when W0 is [H,d,d]), deta fp32 [H] (summed over the batch))."""
    lib = load_library()
    if Q.dim() != 4:
        raise ValueError("Q must be [B,H,T,d]")
    dev = Q.device
    B, H, T, d = Q.shape
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (dY, "dY")):
        _need(t, n, dev, Q.dtype)
        if t.shape != Q.shape:
            raise ValueError(f"{n} shape {tuple(t.shape)} != Q shape {tuple(Q.shape)}")
    _need(W0, "W0", dev, torch.float32)
    _need(eta, "eta", dev, torch.float32)
    per_batch = W0.dim() == 4
    if W0.shape != ((B, H, d, d) if per_batch else (H, d, d)) or eta.shape != (H,):
        raise ValueError("W0 must be [H,d,d] or [B,H,d,d] and eta [H]")
    if dW_out is None:
        dW_out = torch.zeros((B, H, d, d), device=dev, dtype=torch.float32)
    _need(dW_out, "dW_out", dev, torch.float32)
    if dW_out.shape != (B, H, d, d):
        raise ValueError("dW_out must be [B,H,d,d]")
    dQ = torch.empty_like(Q) if dQ is None else dQ
    dK = torch.empty_like(Q) if dK is None else dK
    dV = torch.empty_like(Q) if dV is None else dV
    dW0 = torch.empty_like(W0) if dW0 is None else dW0
    deta = torch.empty_like(eta) if deta is None else deta
    for t, n in ((dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        _need(t, n, dev, Q.dtype)
    _need(dW0, "dW0", dev, torch.float32)
    _need(deta, "deta", dev, torch.float32)
    ws = _workspace(lib.ttt_linear_backward_workspace_bytes(B, H, T, d, int(b), _dtype_code(Q))
                    if workspace is None else 0, dev, workspace)
    _check(lib.ttt_linear_backward(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q),
                                   W0.data_ptr(), int(per_batch), eta.data_ptr(), B, H, T, d,
                                   int(b), dY.data_ptr(), dW_out.data_ptr(), dQ.data_ptr(),
                                   dK.data_ptr(), dV.data_ptr(), dW0.data_ptr(), deta.data_ptr(),
                                   *_ws_args(ws), _stream_handle(dev, stream)))
    return dQ, dK, dV, dW0, deta


def ttt_linear_backward_ex(Q, K, V, W0, eta, b: int, dY, dW_out=None, eta_tok=None, ln_q=None,
                           ln_k=None, ln_eps: float = 1e-5, read_chunk_start: bool = False,
                           workspace=None, stream=None):
    """Gradients of <dY, Y> + <dW_out, W_out> for (Y, W_out) =
    ttt_linear_forward_ex(Q, K, V, W0, eta, b, eta_tok, ln_q, ln_k, ln_eps,
    read_chunk_start).  Returns a dict: dQ, dK, dV (of the raw rows, Q's
    dtype), dW0 (shaped like W0, summed over the batch when shared), deta [H]
    (zero when eta_tok is given), and deta_tok [B,H,T], dln_q, dln_k [H,2,d]
    for the prologue inputs that are given."""
    lib = load_library()
    if Q.dim() != 4:
        raise ValueError("Q must be [B,H,T,d]")
    dev = Q.device
    B, H, T, d = Q.shape
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (dY, "dY")):
        _need(t, n, dev, Q.dtype)
        if t.shape != Q.shape:
            raise ValueError(f"{n} shape {tuple(t.shape)} != Q shape {tuple(Q.shape)}")
    _need(W0, "W0", dev, torch.float32)
    _need(eta, "eta", dev, torch.float32)
    per_batch = W0.dim() == 4
    if W0.shape != ((B, H, d, d) if per_batch else (H, d, d)) or eta.shape != (H,):
        raise ValueError("W0 must be [H,d,d] or [B,H,d,d] and eta [H]")
    if dW_out is None:
        dW_out = torch.zeros((B, H, d, d), device=dev, dtype=torch.float32)
    _need(dW_out, "dW_out", dev, torch.float32)
    if dW_out.shape != (B, H, d, d):
        raise ValueError("dW_out must be [B,H,d,d]")
    out = {"dQ": torch.empty_like(Q), "dK": torch.empty_like(Q), "dV": torch.empty_like(Q),
           "dW0": torch.empty_like(W0), "deta": torch.empty_like(eta)}
    ins, grads = [], []
    for t, n, shape in ((eta_tok, "eta_tok", (B, H, T)), (ln_q, "ln_q", (H, 2, d)),
                        (ln_k, "ln_k", (H, 2, d))):
        if t is None:
            ins.append(None)
            grads.append(None)
            continue
        _need(t, n, dev, torch.float32)
        if t.shape != shape:
            raise ValueError(f"{n} must be {list(shape)}, got {tuple(t.shape)}")
        g = torch.empty(shape, device=dev, dtype=torch.float32)
        out["d" + n] = g
        ins.append(t.data_ptr())
        grads.append(g.data_ptr())
    ws = _workspace(lib.ttt_linear_backward_workspace_bytes(B, H, T, d, int(b), _dtype_code(Q))
                    if workspace is None else 0, dev, workspace)
    _check(lib.ttt_linear_backward_ex(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q),
                                      W0.data_ptr(), int(per_batch), eta.data_ptr(), ins[0],
                                      ins[1], ins[2], float(ln_eps), int(bool(read_chunk_start)),
                                      B, H, T, d, int(b), dY.data_ptr(), dW_out.data_ptr(),
                                      out["dQ"].data_ptr(), out["dK"].data_ptr(),
                                      out["dV"].data_ptr(), out["dW0"].data_ptr(),
                                      out["deta"].data_ptr(), grads[0], grads[1], grads[2],
                                      *_ws_args(ws), _stream_handle(dev, stream)))
    return out


def ttt_linear_decode_step_ex(q, k, v, W, eta, eta_tok=None, ln_q=None, ln_k=None,
                              ln_eps: float = 1e-5, read_chunk_start: bool = False, y=None,
                              stream=None):
    """ttt_linear_decode_step with the input prologue of ttt_linear_forward_ex
    (eta_tok fp32 [B,H]; ln_q / ln_k fp32 [H,2,d]); W updated in place."""
    lib = load_library()
    if q.dim() != 3:
        raise ValueError("q must be [B,H,d]")
    dev = q.device
    B, H, d = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dev, q.dtype)
        if t.shape != q.shape:
            raise ValueError(f"{n} shape {tuple(t.shape)} != q shape {tuple(q.shape)}")
    _need(W, "W", dev, torch.float32)
    _need(eta, "eta", dev, torch.float32)
    if W.shape != (B, H, d, d) or eta.shape != (H,):
        raise ValueError("W must be [B,H,d,d] and eta [H]")
    ptrs = []
    for t, n, shape in ((eta_tok, "eta_tok", (B, H)), (ln_q, "ln_q", (H, 2, d)),
                        (ln_k, "ln_k", (H, 2, d))):
        if t is None:
            ptrs.append(None)
            continue
        _need(t, n, dev, torch.float32)
        if t.shape != shape:
            raise ValueError(f"{n} must be {list(shape)}, got {tuple(t.shape)}")
        ptrs.append(t.data_ptr())
    if y is None:
        y = torch.empty_like(q)
    _need(y, "y", dev, q.dtype)
    _check(lib.ttt_linear_decode_step_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q),
                                         W.data_ptr(), eta.data_ptr(), ptrs[0], ptrs[1], ptrs[2],
                                         float(ln_eps), int(bool(read_chunk_start)), B, H, d,
                                         y.data_ptr(), _stream_handle(dev, stream)))
    return y


def ttt_linear_momentum_forward(Q, K, V, W0, eta, beta, b: int = 16, M0=None, grad_mode: int = 0,
                                Y=None, W_out=None, M_out=None, workspace=None, stream=None):
    """TTT-Linear with momentum gradient descent.  Q,K,V [B,H,T,d] fp32/bf16;
    W0 fp32 [H,d,d] or [B,H,d,d]; M0 fp32 [B,H,d,d] or None (zero); eta,
    beta fp32 [H]; grad_mode 0 (exact token steps) or 1 (chunk-start
    gradients).  workspace: uint8 device tensor (None: one of
    ttt_linear_momentum_workspace_bytes bytes is allocated with torch).
    Returns (Y, W_out, M_out)."""
    lib = load_library()
    if Q.dim() != 4:
        raise ValueError("Q must be [B,H,T,d]")
    dev = Q.device
    B, H, T, d = Q.shape
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, n, dev, Q.dtype)
        if t.shape != Q.shape:
            raise ValueError(f"{n} shape {tuple(t.shape)} != Q shape {tuple(Q.shape)}")
    for t, n in ((W0, "W0"), (eta, "eta"), (beta, "beta")):
        _need(t, n, dev, torch.float32)
    per_batch = W0.dim() == 4
    if W0.shape != ((B, H, d, d) if per_batch else (H, d, d)) or eta.shape != (H,) \
            or beta.shape != (H,):
        raise ValueError("W0 must be [H,d,d] or [B,H,d,d], eta and beta [H]")
    if M0 is not None:
        _need(M0, "M0", dev, torch.float32)
        if M0.shape != (B, H, d, d):
            raise ValueError("M0 must be [B,H,d,d]")
    if Y is None:
        Y = torch.empty_like(Q)
    if W_out is None:
        W_out = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    if M_out is None:
        M_out = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    _need(Y, "Y", dev, Q.dtype)
    _need(W_out, "W_out", dev, torch.float32)
    _need(M_out, "M_out", dev, torch.float32)
    code = _dtype_code(Q)
    ws = _workspace(lib.ttt_linear_momentum_workspace_bytes(B, H, T, d, int(b), code,
                                                            int(grad_mode))
                    if workspace is None else 0, dev, workspace)
    _check(lib.ttt_linear_momentum_forward(Q.data_ptr(), K.data_ptr(), V.data_ptr(), code,
                                           W0.data_ptr(), int(per_batch),
                                           None if M0 is None else M0.data_ptr(),
                                           eta.data_ptr(), beta.data_ptr(), int(grad_mode),
                                           B, H, T, d, int(b), Y.data_ptr(), W_out.data_ptr(),
                                           M_out.data_ptr(), *_ws_args(ws),
                                           _stream_handle(dev, stream)))
    return Y, W_out, M_out


def ttt_linear_momentum_workspace_bytes(B: int, H: int, T: int, d: int, b: int,
                                        dtype=torch.bfloat16, grad_mode: int = 0) -> int:
    """Workspace bytes ttt_linear_momentum_forward uses for these sizes on the
    current device (its planned sequence segments included)."""
    code = TTT_F32 if dtype == torch.float32 else TTT_BF16
    n = load_library().ttt_linear_momentum_workspace_bytes(int(B), int(H), int(T), int(d),
                                                           int(b), code, int(grad_mode))
    _check(min(n, 0))
    return n


def ttt_linear_momentum_segments(B: int, H: int, T: int, d: int, b: int,
                                 dtype=torch.bfloat16, grad_mode: int = 0) -> int:
    """Sequence segments ttt_linear_momentum_forward cuts each chain into for
    these sizes on the current device (1 = unsegmented)."""
    code = TTT_F32 if dtype == torch.float32 else TTT_BF16
    n = load_library().ttt_linear_momentum_segments(int(B), int(H), int(T), int(d), int(b), code,
                                                    int(grad_mode))
    _check(min(n, 0))
    return n


def ttt_linear_segments(B: int, H: int, T: int, d: int, b: int, dtype=torch.bfloat16) -> int:
    """Sequence segments ttt_linear_forward cuts each chain into for these
    sizes on the current device (1 = unsegmented)."""
    code = TTT_F32 if dtype == torch.float32 else TTT_BF16
    n = load_library().ttt_linear_segments(int(B), int(H), int(T), int(d), int(b), code)
    _check(min(n, 0))
    return n


def ttt_linear_fused(B: int, H: int, T: int, d: int, b: int, dtype=torch.bfloat16) -> bool:
    """Whether ttt_linear_forward uses the fused segment layout (segment 0
    scanned beside the maps) for these sizes on the current device."""
    code = TTT_F32 if dtype == torch.float32 else TTT_BF16
    n = load_library().ttt_linear_fused(int(B), int(H), int(T), int(d), int(b), code)
    _check(min(n, 0))
    return bool(n)


def ttt_linear_workspace_bytes(B: int, H: int, T: int, d: int, b: int,
                               dtype=torch.bfloat16) -> int:
    """Workspace bytes ttt_linear_forward uses for these sizes on the current
    device (0 when the scan is not segmented)."""
    code = TTT_F32 if dtype == torch.float32 else TTT_BF16
    n = load_library().ttt_linear_workspace_bytes(int(B), int(H), int(T), int(d), int(b), code)
    _check(min(n, 0))
    return n


def ttt_linear_backward_workspace_bytes(B: int, H: int, T: int, d: int, b: int,
                                        dtype=torch.bfloat16) -> int:
    """Workspace bytes that serve every ttt_linear_backward(_ex) call of these sizes."""
    code = TTT_F32 if dtype == torch.float32 else TTT_BF16
    n = load_library().ttt_linear_backward_workspace_bytes(int(B), int(H), int(T), int(d),
                                                           int(b), code)
    _check(min(n, 0))
    return n


def ttt_linear_backward_segments(B: int, H: int, T: int, d: int, b: int,
                                 dtype=torch.bfloat16) -> int:
    """Sequence segments ttt_linear_backward cuts each chain into for these
    sizes on the current device (1 = unsegmented)."""
    code = TTT_F32 if dtype == torch.float32 else TTT_BF16
    n = load_library().ttt_linear_backward_segments(int(B), int(H), int(T), int(d), int(b), code)
    _check(min(n, 0))
    return n


__all__ = [
    "ttt_linear_forward", "ttt_linear_forward_ex", "ttt_linear_forward_noalloc",
    "ttt_mlp_forward", "ttt_linear_decode_step",
    "ttt_linear_decode_step_ex", "ttt_linear_backward",
    "ttt_linear_segments", "ttt_linear_fused", "ttt_linear_backward_segments", "ttt_linear_workspace_bytes",
    "ttt_linear_backward_workspace_bytes", "ttt_linear_momentum_forward",
    "ttt_linear_momentum_workspace_bytes", "ttt_linear_momentum_segments",
    "load_library",
    "status_string", "TTTError", "LIB_PATH", "TTT_F32", "TTT_BF16",
]
