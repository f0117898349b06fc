"""Fixed workload for rocprofv3 runs: one benchmark configuration's hot path
launched a few times, then one plain device copy of known size whose HBM
counters calibrate the byte counters of the kernels above.

    rocprofv3 --kernel-trace --stats -- python3 <repo>/test_sequence_layers_linear_amd/prof_workload.py --config 2
    rocprofv3 --pmc FETCH_SIZE       -- python3 <repo>/test_sequence_layers_linear_amd/prof_workload.py --config 2
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--copy-mib", type=int, default=256)
    ap.add_argument("--decode", action="store_true", help="also run the workload's decode steps")
    ap.add_argument("--backward", action="store_true",
                    help="run ttt_linear_backward (seeded cotangents) instead of the forward")
    ap.add_argument("--cold", action="store_true",
                    help="cycle the calls through copies of the inputs, enough that at least "
                         "512 MB of other inputs are read between two uses of a copy (the "
                         "256 MB last-level cache cannot serve them), as bench.py's roofline "
                         "timing does")
    ap.add_argument("--prologue", action="store_true",
                    help="with the input prologue (LayerNorm of q and k, per-token step sizes): "
                         "ttt_linear_forward_ex / ttt_linear_backward_ex")
    ap.add_argument("--momentum", choices=["exact", "chunk_start"],
                    help="run ttt_linear_momentum_forward (beta per head from make_momentum) "
                         "instead of the forward")
    args = ap.parse_args()

    import torch
    import test_sequence_layers_linear_amd as ttt
    from test_sequence_layers_linear_amd.inputs import (WORKLOADS, default_seed, make_cotangents,
                                                        make_inputs, make_momentum, make_prologue)

    w = WORKLOADS[args.config]
    g = {k: v.cuda() for k, v in make_inputs(w, default_seed(args.config)).items()}
    Y = torch.empty_like(g["Q"])
    if w.kind == "linear":
        W = torch.empty((w.B, w.H, w.d, w.d), device="cuda")
    else:
        W1 = torch.empty((w.B, w.H, w.d, w.m), device="cuda")
        W2 = torch.empty((w.B, w.H, w.m, w.d), device="cuda")
    if args.backward:
        cot = {k: v.cuda() for k, v in make_cotangents(w, 7).items()}
    if args.prologue:
        pro = {k: v.cuda() for k, v in make_prologue(w, 11).items()}
        pkw = {k: pro[k] for k in ("eta_tok", "ln_q", "ln_k")}
    ws = None
    gm = 0 if args.momentum == "exact" else 1
    if args.momentum:
        beta = make_momentum(w, 31)["beta"].cuda()
        M = torch.empty_like(W)
        nbytes = ttt.ttt_linear_momentum_workspace_bytes(w.B, w.H, w.T, w.d, w.b, w.torch_dtype, gm)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    elif w.kind == "linear":
        nbytes = (ttt.ttt_linear_backward_workspace_bytes if args.backward
                  else ttt.ttt_linear_workspace_bytes)(w.B, w.H, w.T, w.d, w.b, w.torch_dtype)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sets = [g]
    if args.cold:
        per_call = sum(g[k].numel() * g[k].element_size() for k in ("Q", "K", "V")) * 4 // 3
        n = max(3, 1 + -(-512 * 10**6 // per_call))
        sets += [dict(g, Q=g["Q"].clone(), K=g["K"].clone(), V=g["V"].clone())
                 for _ in range(n - 1)]
    torch.cuda.synchronize()
    for rep in range(args.reps):
        g = sets[rep % len(sets)]
        if args.momentum:
            ttt.ttt_linear_momentum_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], beta, w.b,
                                            None, gm, Y=Y, W_out=W, M_out=M, workspace=ws)
        elif args.backward and args.prologue:
            ttt.ttt_linear_backward_ex(g["Q"], g["K"], g["V"], g["W0"], pro["eta"], w.b, cot["dY"],
                                       cot["dW_out"], workspace=ws, **pkw)
        elif args.backward:
            ttt.ttt_linear_backward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], w.b, cot["dY"],
                                    cot["dW_out"], workspace=ws)
        elif args.prologue:
            ttt.ttt_linear_forward_ex(g["Q"], g["K"], g["V"], g["W0"], pro["eta"], w.b, Y=Y,
                                      W_out=W, workspace=ws, **pkw)
        elif w.kind == "linear":
            ttt.ttt_linear_forward(g["Q"], g["K"], g["V"], g["W0"], g["eta"], w.b, Y=Y, W_out=W,
                                   workspace=ws)
            if args.decode:
                y = torch.empty_like(g["dq"][0])
                for s in range(w.decode_steps):
                    ttt.ttt_linear_decode_step(g["dq"][s], g["dk"][s], g["dv"][s], W, g["eta"], y=y)
        else:
            ttt.ttt_mlp_forward(g["Q"], g["K"], g["V"], g["W1"], g["W2"], g["eta"], w.b,
                                Y=Y, W1_out=W1, W2_out=W2)
    torch.cuda.synchronize()
    n = args.copy_mib * 1024 * 1024 // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)          # reads and writes exactly copy_mib MiB
    torch.cuda.synchronize()
    print(f"prof_workload: config {args.config} ({w.name}) x{args.reps}, copy {args.copy_mib} MiB",
          flush=True)


if __name__ == "__main__":
    main()
