#!/usr/bin/env python3
"""Throughput of the TTT forward scan on one MI355X; prints ONE JSON line.

Metric: TTT forward tokens/s = B*T / (seconds per step), at d = 64, b = 16,
plus the fraction of the MFMA or HBM roofline reached by the dominant kernel.

A step is one pass of the hot path over one batch of synthetic inputs that
are already resident in HBM:
  - TTT-Linear workloads: ttt_linear_forward, then the workload's single-token
    decode steps (ttt_linear_decode_step) from the final state, if any;
  - TTT-MLP workloads: ttt_mlp_forward.
--config picks the workload (1..5, default 4: TTT-Linear B2 H24 d64 T32768
b16 bf16 plus 256 decode steps, the largest d = 64, b = 16 TTT-Linear
workload on one GPU).  value = B*T / seconds per step (the decode steps'
time included).  Unless --quick is given, the other d = 64 workloads are
measured too and reported under "workloads" in the same line.

roofline.achieved = algorithmic bytes (HBM bound) or flops (MFMA bound) of
one forward call / its mean duration from HIP events recorded on the launch
stream, for back-to-back calls that cycle through copies of the inputs, so
many that at least 512 MB of other inputs are read between two uses of a copy:
the 256 MB last-level cache cannot serve them (the cold-cache protocol of
rotated input sets; no flush kernel runs between the calls; the cycle first
runs untimed for 50 ms of GPU time, so the timed calls see the steady state
rather than the slower first calls after the decode graph); the same figure
for back-to-back calls on one input set in
the timed region is roofline.warm.  A call is one kernel launch, except a
segmented TTT-Linear scan: maps, start-state composition and segment scans,
three launches back to back on the stream, or two for the fp32 column-split
scan, whose segments compose their own start states (roofline.kernel names
them).  roofline.peak is the datasheet figure; roofline.peak_measured is what
a plain streaming copy or a dense MFMA loop (include/ttt_roofs.h) reaches on
this GPU, and frac_of_measured the fraction of that.  The decode steps of a
workload run as one captured HIP graph.
cpu_baseline = the fp64 oracle (plain loops, OpenMP over chains) timed on
this host's cores on a bounded sample of the same workload: with all host
threads (one chain each), and with one thread (single_thread).

Each TTT-Linear workload also reports "backward": ttt_linear_backward (the
gradients of Q, K, V, W0 and eta for seeded cotangents dY, dW_out), timed
back to back on one input set after 50 ms of untimed calls, with its own roofline (the MFMA peak of the input dtype: bf16
inputs run on bf16 MFMA, fp32 inputs on fp32 MFMA).  It is reported beside the forward, not folded into the
headline value.  "prologue" times ttt_linear_forward_ex on the same inputs
with LayerNorm of q and k and a step size per token fused into the scan, and
"backward_prologue" ttt_linear_backward_ex, the backward through them.
The bf16 TTT-Linear workloads also report "momentum": ttt_linear_momentum_forward
(momentum gradient descent, beta per head from make_momentum) on the same
inputs, for exact token steps and for chunk-start gradients (sequence
segments as ttt_linear_momentum_forward plans them), each timed on cycled
input copies (cold cache) and back to back on one copy, with its own
roofline object.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TTT forward tokens/sec (B·T/s) at d=64,b=16; % of MFMA/HBM roofline"
PEAK_HBM = 8.0e12            # bytes/s, MI355X HBM3E
PEAK_FLOPS = {"bf16": 2.5e15, "fp32": 157.3e12}   # dense MFMA
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "linear_mfma_kernel[scan]": "ttt_linear_mfma.hip",
    "linear_mfma_kernel[maps]": "ttt_linear_mfma.hip",
    "linear_fused_kernel": "ttt_linear_mfma.hip",
    "linear_mfma_f32_kernel[scan]": "ttt_linear_mfma_f32.hip",
    "linear_mfma_f32_kernel[maps]": "ttt_linear_mfma_f32.hip",
    "linear_cols_f32_kernel[scan]": "ttt_linear_cols_f32.hip",
    "linear_cols_f32_kernel[maps]": "ttt_linear_cols_f32.hip",
    "linear_combine_kernel": "ttt_linear_combine.hip",
    "linear_backward_reduce_kernel": "ttt_linear_backward.hip",
    "linear_backward_kernel[gmaps]": "ttt_linear_backward.hip",
    "linear_backward_kernel[segments]": "ttt_linear_backward.hip",
    "linear_backward_bf16_kernel[gmaps]": "ttt_linear_backward_bf16.hip",
    "linear_backward_bf16_kernel[segments]": "ttt_linear_backward_bf16.hip",
    "linear_backward_kernel[gmaps+prologue]": "ttt_linear_backward.hip",
    "linear_backward_kernel[segments+prologue]": "ttt_linear_backward.hip",
    "linear_backward_bf16_kernel[gmaps+prologue]": "ttt_linear_backward_bf16.hip",
    "linear_backward_bf16_kernel[segments+prologue]": "ttt_linear_backward_bf16.hip",
    "linear_generic_kernel": "ttt_generic.hip",
    "mlp_generic_kernel": "ttt_generic.hip",
    "mlp_mfma_kernel": "ttt_mlp_mfma.hip",
    "decode_kernel": "ttt_decode.hip",
    "momentum_inverse_kernel": "ttt_momentum_mfma.hip",
    "momentum_mfma_kernel[exact]": "ttt_momentum_mfma.hip",
    "momentum_mfma_kernel[chunk_start]": "ttt_momentum_mfma.hip",
    "momentum_mfma_kernel[exact+maps]": "ttt_momentum_mfma.hip",
    "momentum_mfma_kernel[chunk_start+maps]": "ttt_momentum_mfma.hip",
    "momentum_combine_kernel": "ttt_linear_combine.hip",
}


# ---------------------------------------------------------------------------
# algorithmic work of one launch
# ---------------------------------------------------------------------------
def _chunks(T, b):
    full, rem = divmod(T, b)
    return [b] * full + ([rem] if rem else [])


def linear_work(w):
    """flops and HBM bytes of one ttt_linear_forward call (dense b x b tiles)."""
    s = 4 if w.dtype == "fp32" else 2
    d, units = w.d, w.B * w.H
    flops = units * sum(6 * n * d * d + 4 * n * n * d for n in _chunks(w.T, w.b))
    nbytes = units * w.T * 4 * d * s + w.H * d * d * 4 + units * d * d * 4
    return flops, nbytes


def linear_backward_work(w):
    """flops and HBM bytes of one ttt_linear_backward call.  Flops per chunk
    of n tokens: E, P (K G), dQ (dY W^T), two in dK, two in G -- 14 n d^2 --
    and S, A^T dY, dA, dA K, dA^T Q -- 10 n^2 d.  Bytes: Q, K, V, dY read,
    dQ, dK, dV written, W0, dW_out, dW0 once (the recomputed chunk-start
    states that the kernel stores and reloads are extra traffic, not
    algorithmic)."""
    s = 4 if w.dtype == "fp32" else 2
    d, units = w.d, w.B * w.H
    flops = units * sum(14 * n * d * d + 10 * n * n * d for n in _chunks(w.T, w.b))
    nbytes = units * w.T * 7 * d * s + (w.H + 2 * units) * d * d * 4
    return flops, nbytes


def mlp_work(w):
    s = 4 if w.dtype == "fp32" else 2
    d, m, units = w.d, w.m, w.B * w.H
    flops = units * sum(14 * n * d * m + 4 * n * n * d + 4 * n * n * m for n in _chunks(w.T, w.b))
    nbytes = units * w.T * 4 * d * s + (w.H + units) * 2 * d * m * 4
    return flops, nbytes


def momentum_work(w, exact):
    """flops and HBM bytes of one ttt_linear_momentum_forward call.  Per chunk
    of n tokens: K W, K M (exact steps only), Q W, Q M and the two state
    updates -- 2 n d^2 each -- and S = Q K^T, S R, plus for exact steps K K^T
    and P RHS -- 2 n^2 d each.  Bytes: Q, K, V read, Y written, W0 once and
    W_out, M_out written (the per-chunk inverses that the first launch writes
    and the scan reads are extra traffic, not algorithmic)."""
    s = 4 if w.dtype == "fp32" else 2
    d, units = w.d, w.B * w.H
    nd2, n2d = (6, 4) if exact else (5, 2)
    flops = units * sum(2 * nd2 * n * d * d + 2 * n2d * n * n * d for n in _chunks(w.T, w.b))
    nbytes = units * w.T * 4 * d * s + w.H * d * d * 4 + 2 * units * d * d * 4
    return flops, nbytes


def decode_work(w):
    s = 4 if w.dtype == "fp32" else 2
    units, d = w.B * w.H, w.d
    return units * 6 * d * d, units * (2 * d * d * 4 + 4 * d * s)


def kernel_names(w, nseg, fused=False):
    """Kernels one forward call dispatches (segmented TTT-Linear: the maps
    launch, or with the fused layout segment 0's scan beside the maps, the
    start-state composition and the segment scans)."""
    if w.kind == "mlp":
        return ["mlp_mfma_kernel" if (w.dtype == "bf16" and w.d == 64 and w.m == 256 and w.b == 16)
                else "mlp_generic_kernel"]
    if w.d == 64 and w.b == 16:
        if w.dtype == "fp32" and f32_cols(w):
            # the segment scans compose their own start states: no combine launch
            k = "linear_cols_f32_kernel"
            return [k + "[maps]", k + "[scan]"] if nseg > 1 else [k + "[scan]"]
        k = "linear_mfma_kernel" if w.dtype == "bf16" else "linear_mfma_f32_kernel"
        if nseg > 1 and fused:
            return ["linear_fused_kernel", "linear_combine_kernel", k + "[scan]"]
        return [k + "[maps]", "linear_combine_kernel", k + "[scan]"] if nseg > 1 else [k + "[scan]"]
    return ["linear_generic_kernel"]


def f32_cols(w):
    """Whether the library runs this fp32 TTT-Linear scan with each chain's W
    split by columns over 4 workgroups (while B*H*4 fits the CUs, unless
    TTT_LINEAR_F32_COLS=0)."""
    import torch
    if os.environ.get("TTT_LINEAR_F32_COLS", "1").strip() == "0":
        return False
    return w.B * w.H * 4 <= torch.cuda.get_device_properties(0).multi_processor_count


def backward_kernel_names(w):
    """Kernels one ttt_linear_backward call dispatches."""
    import torch
    import test_sequence_layers_linear_amd as ttt
    n = ttt.ttt_linear_backward_segments(w.B, w.H, w.T, w.d, w.b,
                                         torch.float32 if w.dtype == "fp32" else torch.bfloat16)
    b = "linear_backward_bf16_kernel" if w.dtype == "bf16" else "linear_backward_kernel"
    k = [b + "[segments]", "linear_backward_reduce_kernel"]
    if n > 1:
        f = "linear_mfma_kernel[maps]" if w.dtype == "bf16" else "linear_mfma_f32_kernel[maps]"
        k = [f, "linear_combine_kernel", b + "[gmaps]", "linear_combine_kernel"] + k
    return k


def fused(w):
    """Whether the library runs this TTT-Linear forward in the fused segment
    layout."""
    if w.kind != "linear":
        return False
    import torch
    import test_sequence_layers_linear_amd as ttt
    return ttt.ttt_linear_fused(w.B, w.H, w.T, w.d, w.b,
                                torch.float32 if w.dtype == "fp32" else torch.bfloat16)


def segments(w):
    if w.kind != "linear":
        return 1
    import torch
    import test_sequence_layers_linear_amd as ttt
    return ttt.ttt_linear_segments(w.B, w.H, w.T, w.d, w.b,
                                   torch.float32 if w.dtype == "fp32" else torch.bfloat16)


def source_sha(kernel):
    path = os.path.join(ROOT, "test_sequence_layers_linear_amd", "csrc", KERNEL_SOURCES[kernel])
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def stored_traffic(kernels, workload):
    """HBM bytes of one forward call (summed over its kernels) from committed
    rocprofv3 --pmc summaries, if every kernel's figure was taken on its
    current source; else None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        table = json.load(open(path))
    except (ValueError, OSError):
        return None
    total = 0
    for k in kernels:
        rec = table.get(k, {}).get(workload)
        if not rec or rec.get("source_sha") != source_sha(k):
            return None
        total += rec.get("bytes_per_launch", 0)
    return total


COLD_TIMING = ("HIP events around back-to-back calls cycling through copies of the inputs; "
               ">= 512 MB of other inputs read between two uses of a copy; the cycle warmed "
               "for 50 ms of GPU time first")


def roofline(w, flops, nbytes, seconds, kernels, roofs=None, warm_seconds=None,
             timing=COLD_TIMING):
    """Roofline object of one call: `seconds` is its mean duration as `timing`
    states (for a forward: cold cache, calls cycling through input copies),
    `warm_seconds` (optional) the back-to-back one; `roofs` the measured copy
    bandwidth and MFMA throughputs."""
    dt = "bf16" if w.dtype == "bf16" else "fp32"
    ridge = PEAK_FLOPS[dt] / PEAK_HBM
    roofs = roofs or {}
    if flops / nbytes > ridge:
        ach, peak, unit, bound = flops / seconds / 1e12, PEAK_FLOPS[dt] / 1e12, "TFLOP/s", "mfma"
        meas = roofs.get("mfma_" + dt + "_tflops")
        warm = flops / warm_seconds / 1e12 if warm_seconds else None
    else:
        ach, peak, unit, bound = nbytes / seconds / 1e9, PEAK_HBM / 1e9, "GB/s", "hbm"
        meas = roofs.get("copy_GBps")
        warm = nbytes / warm_seconds / 1e9 if warm_seconds else None
    out = {"bound": bound, "achieved": round(ach, 3), "peak": peak, "unit": unit,
           "frac": round(ach / peak, 5), "traffic": stored_traffic(kernels, w.name),
           "kernel": " + ".join(kernels), "mean_launch_us": round(seconds * 1e6, 3),
           "timing": timing,
           "peak_measured": round(meas, 3) if meas else None,
           "frac_of_measured": round(ach / meas, 5) if meas else None,
           "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
           "active_cu_ceiling": round(min(1.0, w.B * w.H / 256), 4)}
    if warm_seconds:
        out["warm"] = {"achieved": round(warm, 3), "frac": round(warm / peak, 5),
                       "mean_launch_us": round(warm_seconds * 1e6, 3),
                       "timing": "mean over the back-to-back calls of the timed region"}
    return out


def warm_up(torch, call, calls, seconds=0.05):
    """At least `calls` untimed calls, and more until they have kept the GPU
    busy for `seconds` (see cycle_timed for why)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    done, busy = 0, 0.0
    while done < calls or busy < seconds:
        torch.cuda.synchronize()
        a.record()
        call()
        b.record()
        torch.cuda.synchronize()
        busy += a.elapsed_time(b) / 1e3
        done += 1


def cycle_timed(torch, call, sets, reps, warm_seconds=0.05):
    """Mean duration of back-to-back calls that cycle through the input sets
    (at least `reps` calls and at least two passes), from HIP events at the
    two ends.  Before the timed calls the cycle runs untimed passes until
    they have kept the GPU busy for `warm_seconds`: after an idle spell or a
    phase of short launches (decode steps), the first few dozen large calls
    run up to 15% slower than the steady state that a serving loop sees
    (B2 H24 T32768: 266, 246, then 228 us per call over three 30-call
    passes, 225 us from then on)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warmed = 0.0
    while True:
        torch.cuda.synchronize()
        a.record()
        for x in sets:
            call(x)
        b.record()
        torch.cuda.synchronize()
        warmed += a.elapsed_time(b) / 1e3
        if warmed >= warm_seconds:
            break
    n = max(reps, 2 * len(sets))
    n = -(-n // len(sets)) * len(sets)
    torch.cuda.synchronize()
    a.record()
    for i in range(n):
        call(sets[i % len(sets)])
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / n


def measure_roofs():
    """Achievable HBM bandwidth (a 1 GiB streaming copy) and dense MFMA
    throughput (bf16 16x16x32 and fp32 16x16x4 loops on 8 waves per CU) on
    this GPU, from the plain kernels of include/ttt_roofs.h; median of 5."""
    import ctypes
    import torch
    import test_sequence_layers_linear_amd as ttt
    lib = ttt.load_library()
    lib.ttt_roof_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.ttt_roof_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        ts.sort()
        return ts[len(ts) // 2]

    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    t = timed(lambda: ttt._check(lib.ttt_roof_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream)))
    out = {"copy_GBps": 2 * nbytes / t / 1e9, "copy_bytes": nbytes}
    del src, dst
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    waves = cus * 8
    sink = torch.empty(waves * 64, device="cuda")
    for dt, name, iters in ((1, "bf16", 20000), (0, "fp32", 10000)):
        fl = ctypes.c_double(0.0)
        t = timed(lambda: ttt._check(lib.ttt_roof_mfma(sink.data_ptr(), dt, waves, iters,
                                                       ctypes.byref(fl), stream)), reps=3)
        out[f"mfma_{name}_tflops"] = fl.value / t / 1e12
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# GPU measurement
# ---------------------------------------------------------------------------
class Runner:
    def __init__(self, w, seed):
        import torch
        import test_sequence_layers_linear_amd as ttt
        from test_sequence_layers_linear_amd.inputs import make_inputs

        self.torch, self.ttt, self.w = torch, ttt, w
        self.host = make_inputs(w, seed)
        self.g = {k: v.cuda() for k, v in self.host.items()}
        g = self.g
        self.Y = torch.empty_like(g["Q"])
        if w.kind == "linear":
            self.W = torch.empty((w.B, w.H, w.d, w.d), device="cuda")
        else:
            self.W1 = torch.empty((w.B, w.H, w.d, w.m), device="cuda")
            self.W2 = torch.empty((w.B, w.H, w.m, w.d), device="cuda")
        if w.decode_steps:
            self.y = torch.empty_like(g["dq"][0])
        if w.kind == "linear":
            self.ws = torch.empty(ttt.ttt_linear_workspace_bytes(w.B, w.H, w.T, w.d, w.b,
                                                                 w.torch_dtype),
                                  dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()

    def input_sets(self):
        """Copies of Q, K, V (the first is the original), enough that at
        least 512 MB of other inputs are read between two uses of a copy
        when calls cycle through them: a call then finds none of its inputs
        in the 256 MB last-level cache."""
        if getattr(self, "_sets", None) is None:
            w = self.w
            per_call = (linear_work if w.kind == "linear" else mlp_work)(w)[1]
            n = max(3, 1 + math.ceil(512e6 / per_call))
            self._sets = [self.g] + [dict(self.g, Q=self.g["Q"].clone(), K=self.g["K"].clone(),
                                           V=self.g["V"].clone()) for _ in range(n - 1)]
        return self._sets

    def forward(self, g=None):
        g, ttt = g or self.g, self.ttt
        if self.w.kind == "linear":
            ttt.ttt_linear_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], self.w.b,
                                   Y=self.Y, W_out=self.W, workspace=self.ws)
        else:
            ttt.ttt_mlp_forward(g["Q"], g["K"], g["V"], g["W1"], g["W2"], g["eta"], self.w.b,
                                Y=self.Y, W1_out=self.W1, W2_out=self.W2)

    def decode_eager(self):
        g, ttt = self.g, self.ttt
        for s in range(self.w.decode_steps):
            ttt.ttt_linear_decode_step(g["dq"][s], g["dk"][s], g["dv"][s], self.W, g["eta"],
                                       y=self.y)

    def capture_decode(self):
        """The decode steps as one HIP graph (one launch per token, replayed
        as a unit), so that a token costs its kernel rather than a host call."""
        torch = self.torch
        self.graph = None
        if not self.w.decode_steps:
            return
        self.decode_eager()                  # warm the launch path
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.decode_eager()
        torch.cuda.synchronize()
        self.graph = graph

    def decode(self):
        if getattr(self, "graph", None) is not None:
            self.graph.replay()
        else:
            self.decode_eager()

    def measure_decode_floor(self, reps=10):
        """Per-step time of the decode graph replayed back to back (its
        inputs then sit in the caches, as a projection just before would leave
        them), and of a graph of as many empty launches of the step's grid
        (B*H*ceil(d/32) workgroups of 64 threads): the launch floor."""
        torch, ttt, w = self.torch, self.ttt, self.w
        if getattr(self, "graph", None) is None:
            return None
        import ctypes
        lib = ttt.load_library()
        lib.ttt_roof_launch.argtypes = [ctypes.c_int64, ctypes.c_void_p]
        groups = w.B * w.H * max(1, -(-w.d // 32))

        def empties():
            stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for _ in range(w.decode_steps):
                ttt._check(lib.ttt_roof_launch(groups, stream))

        empties()
        torch.cuda.synchronize()
        floor_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(floor_graph):
            empties()
        torch.cuda.synchronize()
        out = {}
        for name, gr in (("cached_inputs", self.graph), ("empty_kernel", floor_graph)):
            gr.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                gr.replay()
            b.record()
            torch.cuda.synchronize()
            out[name] = a.elapsed_time(b) * 1e3 / (reps * w.decode_steps)
        return out

    def measure(self, steps, warmup):
        """Time exactly `steps` steps between two synchronisations.  HIP events
        on the launch stream mark the start, the end and (with decode steps)
        the end of each step's forward call, so the forward duration comes from
        the same timed region without an event between consecutive launches."""
        torch = self.torch
        self.capture_decode()
        for _ in range(warmup):
            self.forward()
            self.decode()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        mids = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(steps)] if self.w.decode_steps else []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            if mids:
                mids[i][0].record()
            self.forward()
            if mids:
                mids[i][1].record()
            self.decode()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total = start.elapsed_time(end) / 1e3
        if mids:
            fwd = sum(a.elapsed_time(b) for a, b in mids) / steps / 1e3
            dec = (total - fwd * steps) / steps
        else:
            fwd, dec = total / steps, 0.0
        return wall / steps, fwd, dec

    def measure_backward(self, steps, warmup, prologue=False):
        """Mean duration of ttt_linear_backward over `steps` calls between two
        synchronisations (HIP events on the launch stream at both ends); with
        `prologue`, of ttt_linear_backward_ex through LayerNorm of q and k and
        per-token step sizes."""
        torch, g, w = self.torch, self.g, self.w
        from test_sequence_layers_linear_amd.inputs import make_cotangents, make_prologue
        cot = {k: v.cuda() for k, v in make_cotangents(w, 7).items()}
        outs = dict(dQ=torch.empty_like(g["Q"]), dK=torch.empty_like(g["Q"]),
                    dV=torch.empty_like(g["Q"]), dW0=torch.empty_like(g["W0"]),
                    deta=torch.empty_like(g["eta"]))
        pro = {k: v.cuda() for k, v in make_prologue(w, 11).items()}
        ws = torch.empty(self.ttt.ttt_linear_backward_workspace_bytes(w.B, w.H, w.T, w.d, w.b,
                                                                      w.torch_dtype),
                         dtype=torch.uint8, device="cuda")

        def call():
            if prologue:
                self.ttt.ttt_linear_backward_ex(g["Q"], g["K"], g["V"], g["W0"], pro["eta"], w.b,
                                                cot["dY"], cot["dW_out"], eta_tok=pro["eta_tok"],
                                                ln_q=pro["ln_q"], ln_k=pro["ln_k"], workspace=ws)
            else:
                self.ttt.ttt_linear_backward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], w.b,
                                             cot["dY"], cot["dW_out"], workspace=ws, **outs)
        warm_up(torch, call, warmup)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            call()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / 1e3 / steps

    def measure_prologue(self, steps, warmup):
        """Mean duration of ttt_linear_forward_ex with the whole prologue
        (LayerNorm of q and k, per-token step sizes)."""
        torch, g, w = self.torch, self.g, self.w
        from test_sequence_layers_linear_amd.inputs import make_prologue
        pro = {k: v.cuda() for k, v in make_prologue(w, 11).items()}

        def call():
            self.ttt.ttt_linear_forward_ex(g["Q"], g["K"], g["V"], g["W0"], pro["eta"], w.b,
                                           eta_tok=pro["eta_tok"], ln_q=pro["ln_q"],
                                           ln_k=pro["ln_k"], Y=self.Y, W_out=self.W,
                                           workspace=self.ws)
        warm_up(torch, call, warmup)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            call()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / 1e3 / steps

    def measure_momentum(self, steps, warmup, grad_mode, cold_reps):
        """ttt_linear_momentum_forward: (mean back to back over `steps` calls,
        mean over at least `cold_reps` back-to-back calls cycling through the
        input copies)."""
        torch, g, w = self.torch, self.g, self.w
        from test_sequence_layers_linear_amd.inputs import make_momentum
        beta = make_momentum(w, 31)["beta"].cuda()
        M = torch.empty_like(self.W)
        ws = torch.empty(self.ttt.ttt_linear_momentum_workspace_bytes(w.B, w.H, w.T, w.d, w.b,
                                                                      w.torch_dtype, grad_mode),
                         dtype=torch.uint8, device="cuda")

        def call(x=g):
            self.ttt.ttt_linear_momentum_forward(x["Q"], x["K"], x["V"], x["W0"], x["eta"], beta,
                                                 w.b, None, grad_mode, Y=self.Y, W_out=self.W,
                                                 M_out=M, workspace=ws)
        warm_up(torch, call, warmup)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            call()
        end.record()
        torch.cuda.synchronize()
        warm = start.elapsed_time(end) / 1e3 / steps
        cold = cycle_timed(torch, call, self.input_sets(), cold_reps)
        del ws
        return warm, cold

    def measure_cold(self, reps):
        """Mean forward duration over at least `reps` back-to-back calls that
        cycle through the input copies (none of a call's inputs in the
        last-level cache)."""
        return cycle_timed(self.torch, self.forward, self.input_sets(), reps)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample
# ---------------------------------------------------------------------------
def _select(host, chains, T):
    import torch
    out = {k: torch.stack([host[k][b, h, :T] for b, h in chains])[None] for k in ("Q", "K", "V")}
    out["eta"] = torch.stack([host["eta"][h] for _, h in chains])
    for k in ("W0", "W1", "W2"):
        if k in host:
            out[k] = torch.stack([host[k][h] for _, h in chains])
    return out


def run_cpu_baseline(w, host, target_s):
    """The oracle on a bounded sample of the workload: k = min(chains, host
    threads) (batch, head) chains at full length, one OpenMP thread each,
    repeated to about target_s seconds; then one chain on one thread."""
    import oracle
    threads = max(1, oracle.max_threads())
    units = [(b, h) for b in range(w.B) for h in range(w.H)]

    def timed(chains, nthreads, budget):
        sub = _select(host, chains, w.T)

        def once():
            if w.kind == "linear":
                oracle.linear_forward(sub["Q"], sub["K"], sub["V"], sub["W0"], sub["eta"], w.b,
                                      nthreads=nthreads)
            else:
                oracle.mlp_forward(sub["Q"], sub["K"], sub["V"], sub["W1"], sub["W2"], sub["eta"],
                                   w.b, nthreads=nthreads)
        t0 = time.perf_counter()
        once()
        first = time.perf_counter() - t0
        reps = max(1, min(1000, int(math.ceil((budget - first) / max(first, 1e-6)))))
        t0 = time.perf_counter()
        for _ in range(reps):
            once()
        el = time.perf_counter() - t0
        # B*T-equivalent tokens: a token of the workload covers all H heads
        return len(chains) * w.T * reps / w.H / el, reps, el

    k = min(len(units), threads)
    v_all, reps, el = timed(units[:k], k, target_s)
    v_one, reps1, el1 = timed(units[:1], 1, target_s / 2)
    return {"value": round(v_all, 3), "unit": "tokens/s", "cores": k, "kind": "oracle",
            "sample": f"{k} of {len(units)} (batch, head) chains at full T={w.T} on {k} threads, "
                      f"{reps} repetitions, {el:.1f} s; tokens counted as chains*T/H",
            "single_thread": {"value": round(v_one, 3), "cores": 1,
                              "sample": f"chain (0, 0) at full T={w.T}, {reps1} repetitions, "
                                        f"{el1:.1f} s"},
            "host_threads_available": threads, "host_cpu": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---------------------------------------------------------------------------
def measure_workload(cfg, steps, warmup, cold_reps, roofs=None):
    from test_sequence_layers_linear_amd.inputs import WORKLOADS, default_seed
    w = WORKLOADS[cfg]
    r = Runner(w, default_seed(cfg))
    per_step, fwd, dec = r.measure(steps, warmup)
    flops, nbytes = (linear_work if w.kind == "linear" else mlp_work)(w)
    nseg = segments(w)
    kern = kernel_names(w, nseg, fused(w))
    cold_mean = r.measure_cold(cold_reps)
    out = {"workload": w.name, "config": cfg, "tokens_per_s": w.B * w.T / per_step,
           "segments_per_chain": nseg, "fused_segments": fused(w),
           "ms_per_step": per_step * 1e3, "forward_us": fwd * 1e6,
           "forward_us_cold_llc": cold_mean * 1e6, "input_copies": len(r.input_sets()),
           "forward_tokens_per_s": w.B * w.T / fwd,
           "roofline": roofline(w, flops, nbytes, cold_mean, kern, roofs, warm_seconds=fwd)}
    if w.kind == "linear" and w.d == 64 and w.b == 16:
        bt = r.measure_backward(max(3, steps // 2), 2)
        bf, bb = linear_backward_work(w)
        kern = backward_kernel_names(w)
        # bf16 inputs run on bf16 MFMA, fp32 on fp32
        rf = roofline(w, bf, bb, bt, kern,
                      timing="HIP events around back-to-back calls on one input set")
        rf["traffic"] = stored_traffic(kern, w.name + "/backward")
        out["backward"] = {"us": bt * 1e6, "tokens_per_s": w.B * w.T / bt, "roofline": rf}
        pt = r.measure_prologue(max(3, steps // 2), 2)
        out["prologue"] = {"us": pt * 1e6, "tokens_per_s": w.B * w.T / pt,
                           "vs_plain_forward": pt / fwd}
        bpt = r.measure_backward(max(3, steps // 2), 2, prologue=True)
        out["backward_prologue"] = {"us": bpt * 1e6, "tokens_per_s": w.B * w.T / bpt,
                                    "vs_plain_backward": bpt / bt}
    if w.kind == "linear" and w.d == 64 and w.b == 16 and w.dtype == "bf16":
        out["momentum"] = {}
        for mode, gm in (("exact", 0), ("chunk_start", 1)):
            warm, cold = r.measure_momentum(max(3, steps // 2), 2, gm, max(3, cold_reps // 3))
            mf, mb = momentum_work(w, gm == 0)
            nseg = r.ttt.ttt_linear_momentum_segments(w.B, w.H, w.T, w.d, w.b, w.torch_dtype, gm)
            kern = ((["momentum_inverse_kernel"] if gm == 0 else []) +
                    ([f"momentum_mfma_kernel[{mode}+maps]", "momentum_combine_kernel"]
                     if nseg > 1 else []) + [f"momentum_mfma_kernel[{mode}]"])
            out["momentum"][mode] = {"us": warm * 1e6, "us_cold_llc": cold * 1e6,
                                     "segments_per_chain": nseg,
                                     "tokens_per_s": w.B * w.T / warm,
                                     "roofline": roofline(w, mf, mb, cold, kern, roofs,
                                                          warm_seconds=warm)}
    if w.decode_steps:
        df, db = decode_work(w)
        per = dec / w.decode_steps
        out["decode"] = {"steps": w.decode_steps, "us_per_step": per * 1e6,
                         "hip_graph": r.graph is not None,
                         "GB_per_s": db / per / 1e9, "hbm_frac": db / per / PEAK_HBM,
                         "bytes_per_step": db}
        floor = r.measure_decode_floor()
        if floor:
            # in the timed step the decode inputs come cold from HBM (the
            # forward before them streams far more than the caches hold)
            out["decode"]["us_per_step_cached_inputs"] = floor["cached_inputs"]
            out["decode"]["launch_floor_us"] = floor["empty_kernel"]
            out["decode"]["vs_launch_floor"] = per * 1e6 / floor["empty_kernel"]
    return w, r, out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--quick", action="store_true", help="only the selected workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested). (batch, head) chains are independent, so "
              "several GPUs would each run this same kernel on their share.", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    print(f"[bench] workload config {args.config}: steps {args.steps} warmup {args.warmup}",
          file=sys.stderr, flush=True)
    print("[bench] measured roofs (stream copy, MFMA loops)", file=sys.stderr, flush=True)
    roofs = measure_roofs()
    print(f"[bench]   copy {roofs['copy_GBps']:.0f} GB/s, bf16 MFMA {roofs['mfma_bf16_tflops']:.0f} "
          f"TFLOP/s, fp32 MFMA {roofs['mfma_fp32_tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    w, runner, main_res = measure_workload(args.config, args.steps, args.warmup, cold_reps=30,
                                           roofs=roofs)
    print(f"[bench] {w.name}: {main_res['tokens_per_s']:.4g} tokens/s", file=sys.stderr, flush=True)

    extras = {}
    if not args.quick:
        for cfg in (2, 3, 4, 5):
            if cfg == args.config:
                continue
            st = 10 if cfg != 5 else 3
            print(f"[bench] extra workload config {cfg}", file=sys.stderr, flush=True)
            _, rr, res = measure_workload(cfg, st, 2, cold_reps=10, roofs=roofs)
            extras[str(cfg)] = res
            del rr
            torch.cuda.empty_cache()
            print(f"[bench]   {res['workload']}: {res['tokens_per_s']:.4g} tokens/s, "
                  f"roofline frac {res['roofline']['frac']}", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = run_cpu_baseline(w, runner.host, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(main_res["tokens_per_s"], 3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if w.dtype == "fp32" else "bf16",
        "data": "synthetic (seeded Gaussian Q/K/V, see inputs.py)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d": w.d, "b": w.b,
                   "m": w.m or None, "decode_steps": w.decode_steps, "global_batch": w.B,
                   "seq_len": w.T,
                   "parallelism": (f"one GPU; {main_res['segments_per_chain']} sequence segments "
                                   "per (batch, head) chain" if main_res["segments_per_chain"] > 1
                                   else "one GPU; one workgroup per (batch, head) chain")},
        "roofline": main_res["roofline"],
        "cpu_baseline": cpu,
        "measured_roofs": roofs,
        "detail": {k: v for k, v in main_res.items() if k not in ("roofline",)},
        "workloads": extras,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
