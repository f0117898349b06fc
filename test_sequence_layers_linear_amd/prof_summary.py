"""Turn rocprofv3 CSV output of prof_workload.py runs into the short text
summaries kept under profiles/ and the per-launch HBM byte table bench.py
reports as roofline.traffic.

    python3 -m test_sequence_layers_linear_amd.prof_summary --config 2 \
        --trace DIR_WITH_kt_kernel_stats.csv --fetch DIR_FETCH --write DIR_WRITE \
        --command "..." --out profiles/linear_fp32_B1_H4_T2048.md

FETCH_SIZE and WRITE_SIZE are in KiB per dispatch.  Each is scaled by the
ratio of the known bytes of the plain 256 MiB device copy in the same run to
what the same counter reads for that copy.

--sq DIR [DIR ...]: rocprofv3 --pmc runs of SQ counters (any split into
passes); adds a table of instructions per wave and MFMA utilisation per
kernel.  SQ_WAVE_CYCLES counts quad-cycles (4 clocks) per wave, and
SQ_VALU_MFMA_BUSY_CYCLES clocks per SIMD, so the MFMA busy fraction of the
chip is MFMA_BUSY / (GRBM_GUI_ACTIVE x 1024 SIMDs) (rocprofv3's own derived
metric) and of a wave's lifetime MFMA_BUSY / (4 x SQ_WAVE_CYCLES) (one wave
per SIMD).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "test_sequence_layers_linear_amd", "csrc")
KERNEL_FILES = {
    "linear_mfma_kernel[scan]": "ttt_linear_mfma.hip",
    "linear_mfma_kernel[maps]": "ttt_linear_mfma.hip",
    "linear_fused_kernel": "ttt_linear_mfma.hip",
    "linear_mfma_f32_kernel[scan]": "ttt_linear_mfma_f32.hip",
    "linear_mfma_f32_kernel[maps]": "ttt_linear_mfma_f32.hip",
    "linear_cols_f32_kernel[scan]": "ttt_linear_cols_f32.hip",
    "linear_cols_f32_kernel[maps]": "ttt_linear_cols_f32.hip",
    "linear_mfma_kernel[scan+prologue]": "ttt_linear_mfma.hip",
    "linear_mfma_kernel[maps+prologue]": "ttt_linear_mfma.hip",
    "linear_mfma_f32_kernel[scan+prologue]": "ttt_linear_mfma_f32.hip",
    "linear_mfma_f32_kernel[maps+prologue]": "ttt_linear_mfma_f32.hip",
    "linear_cols_f32_kernel[scan+prologue]": "ttt_linear_cols_f32.hip",
    "linear_cols_f32_kernel[maps+prologue]": "ttt_linear_cols_f32.hip",
    "linear_combine_kernel": "ttt_linear_combine.hip",
    "linear_backward_kernel[gmaps]": "ttt_linear_backward.hip",
    "linear_backward_kernel[segments]": "ttt_linear_backward.hip",
    "linear_backward_bf16_kernel[gmaps]": "ttt_linear_backward_bf16.hip",
    "linear_backward_bf16_kernel[segments]": "ttt_linear_backward_bf16.hip",
    "linear_backward_kernel[gmaps+prologue]": "ttt_linear_backward.hip",
    "linear_backward_kernel[segments+prologue]": "ttt_linear_backward.hip",
    "linear_backward_bf16_kernel[gmaps+prologue]": "ttt_linear_backward_bf16.hip",
    "linear_backward_bf16_kernel[segments+prologue]": "ttt_linear_backward_bf16.hip",
    "linear_backward_reduce_kernel": "ttt_linear_backward.hip",
    "linear_generic_kernel": "ttt_generic.hip",
    "mlp_generic_kernel": "ttt_generic.hip",
    "mlp_mfma_kernel": "ttt_mlp_mfma.hip",
    "decode_kernel": "ttt_decode.hip",
    "momentum_inverse_kernel": "ttt_momentum_mfma.hip",
    "momentum_mfma_kernel[exact]": "ttt_momentum_mfma.hip",
    "momentum_mfma_kernel[exact+maps]": "ttt_momentum_mfma.hip",
    "momentum_mfma_kernel[chunk_start+maps]": "ttt_momentum_mfma.hip",
    "momentum_combine_kernel": "ttt_linear_combine.hip",
    "momentum_mfma_kernel[chunk_start]": "ttt_momentum_mfma.hip",
}
COPY_NAME = "__amd_rocclr_copyBuffer"


def short_name(full: str) -> str:
    """Kernel key: the function name, with [maps] / [scan] for the two
    instantiations of the TTT-Linear forward kernels (the fused layout's first
    launch, segment 0's scan beside the maps, is linear_fused_kernel) and [gmaps] / [segments]
    for the backward's cotangent maps and segment backward (+prologue for
    the instantiations with the input prologue)."""
    if "linear_fused_kernel<" in full:       # kStream only: one key
        return "linear_fused_kernel"
    if "momentum_mfma_kernel<" in full:      # kExact, kMap
        args = [a.strip() for a in full.split("momentum_mfma_kernel<", 1)[1].split(">", 1)[0].split(",")]
        mode = "exact" if args[0] == "true" else "chunk_start"
        return f"momentum_mfma_kernel[{mode}{'+maps' if len(args) > 1 and args[1] == 'true' else ''}]"
    for base in ("linear_backward_kernel", "linear_backward_bf16_kernel"):
        if base + "<" in full:
            args = [a.strip() for a in full.split(base + "<", 1)[1].split(">", 1)[0].split(",")]
            flags = [a for a in args if a in ("true", "false")]     # kGMap, kPro
            role = "gmaps" if flags[0] == "true" else "segments"
            return f"{base}[{role}{'+prologue' if flags[1] == 'true' else ''}]"
    for k in KERNEL_FILES:
        base = k.split("[")[0]
        if base in ("linear_backward_kernel", "linear_backward_bf16_kernel"):
            continue
        if base + "<true" in full or base + "<false" in full:
            args = [a.strip() for a in full.split(base + "<", 1)[1].split(">", 1)[0].split(",")]
            flags = [a for a in args if a in ("true", "false")]     # kMaps, kPro
            pro = "+prologue" if len(flags) > 1 and flags[1] == "true" else ""
            return f"{base}[{'maps' if flags[0] == 'true' else 'scan'}{pro}]"
        if base + "(" in full or base + "<" in full:
            return k
    return full.split("(")[0][-60:]


def source_sha(kernel: str) -> str:
    path = os.path.join(CSRC, KERNEL_FILES[kernel])
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def one_csv(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def counter_per_kernel(d: str):
    vals = {}
    for r in csv.DictReader(open(one_csv(d, "counter_collection.csv"))):
        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


SIMDS = 1024          # 256 CUs x 4 SIMDs


def sq_table(dirs, command, chunks_per_wave):
    """Per-kernel SQ counter summary: mean per dispatch over every run."""
    per = {}
    for d in dirs:
        for r in csv.DictReader(open(one_csv(d, "counter_collection.csv"))):
            name = short_name(r["Kernel_Name"])
            if name not in KERNEL_FILES:
                continue
            per.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = ["SQ counters (mean per dispatch):", "", "```", command, "```", "",
           "| kernel | waves | VALU/wave | MFMA/wave | LDS/wave | SALU/wave | VMEM rd/wave | "
           "wave cycles | MFMA busy, chip | MFMA busy, wave lifetime | wait-inst / wave cycles | "
           "LDS bank conflicts / LDS inst |" + (" cycles per chunk |" if chunks_per_wave else ""),
           "|---|" + "---|" * (11 + (1 if chunks_per_wave else 0))]

    for name, c in sorted(per.items()):
        m = {k: sum(v) / len(v) for k, v in c.items()}
        waves = m.get("SQ_WAVES", float("nan"))
        wc = 4 * m.get("SQ_WAVE_CYCLES", float("nan"))
        busy = m.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan"))
        grbm = m.get("GRBM_GUI_ACTIVE", float("nan"))
        pw = lambda k: m.get(k, float("nan")) / waves
        row = (f"| {name} | {waves:.0f} | {pw('SQ_INSTS_VALU'):.0f} | {pw('SQ_INSTS_MFMA'):.0f} | "
               f"{pw('SQ_INSTS_LDS'):.0f} | {pw('SQ_INSTS_SALU'):.0f} | {pw('SQ_INSTS_VMEM_RD'):.0f} | "
               f"{wc / waves:.0f} | {100 * busy / (grbm * SIMDS):.2f}% | {100 * busy / wc:.1f}% | "
               f"{m.get('SQ_WAIT_INST_ANY', float('nan')) * 4 / wc:.3f} | "
               f"{m.get('SQ_LDS_BANK_CONFLICT', float('nan')) / m.get('SQ_INSTS_LDS', float('nan')):.3f} |")
        if chunks_per_wave:
            # only for the scans, whose every wave walks its chain's chunks
            scan = not any(x in name for x in ("inverse", "combine", "maps", "reduce"))
            row += f" {wc / waves / chunks_per_wave:.0f} |" if scan else " |"
        out.append(row)
    out.append("")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, required=True)
    ap.add_argument("--trace", help="rocprofv3 --kernel-trace --stats output (omit: counters only)")
    ap.add_argument("--fetch", help="rocprofv3 --pmc FETCH_SIZE output (omit: no byte counts)")
    ap.add_argument("--write", help="rocprofv3 --pmc WRITE_SIZE output")
    ap.add_argument("--title", help="heading (default: the workload name)")
    ap.add_argument("--command", required=True, help="the rocprofv3 command lines that made the data")
    ap.add_argument("--copy-mib", type=int, default=256)
    ap.add_argument("--call", default="forward",
                    choices=["forward", "backward", "forward_prologue", "backward_prologue"],
                    help="which call the trace covers (the traffic table keys the kernels of "
                         "any call but the forward under '<workload>/<call>')")
    ap.add_argument("--out", required=True)
    ap.add_argument("--sq", nargs="*", default=[], help="rocprofv3 --pmc runs of SQ counters")
    ap.add_argument("--sq-command", default="", help="the commands of the --sq runs")
    ap.add_argument("--chunks-per-wave", type=float, default=0.0,
                    help="chunks each wave of the scan processes (for cycles per chunk)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"))
    args = ap.parse_args()

    import sys
    sys.path.insert(0, ROOT)
    from test_sequence_layers_linear_amd.inputs import WORKLOADS
    w = WORKLOADS[args.config]

    stats = list(csv.DictReader(open(one_csv(args.trace, "kernel_stats.csv")))) if args.trace else []
    have_bytes = bool(args.fetch and args.write)
    fetch = counter_per_kernel(args.fetch) if have_bytes else {}
    write = counter_per_kernel(args.write) if have_bytes else {}
    lines = [f"# rocprofv3 summary: {args.title or w.name}", "",
             "Commands (run from /tmp on the MI355X host, repo at $R):", "", "```", args.command, "```", ""]
    f_scale = w_scale = 1.0
    if have_bytes:
        copy_bytes = args.copy_mib * 1024 * 1024
        copy_fetch = max(v for k, vs in fetch.items() if COPY_NAME in k for v in vs) * 1024
        copy_write = max(v for k, vs in write.items() if COPY_NAME in k for v in vs) * 1024
        f_scale, w_scale = copy_bytes / copy_fetch, copy_bytes / copy_write
        lines += [f"Copy calibration ({args.copy_mib} MiB device copy): FETCH_SIZE reads "
                  f"{copy_fetch / 1024:.1f} KiB (scale {f_scale:.3f}), WRITE_SIZE reads "
                  f"{copy_write / 1024:.1f} KiB (scale {w_scale:.3f}).", ""]
    if stats:
        lines += ["| kernel | calls | avg us | min us | max us | HBM read MB/launch | HBM write MB/launch |",
                  "|---|---|---|---|---|---|---|"]
    table = json.load(open(args.traffic)) if os.path.exists(args.traffic) else {}
    for r in stats:
        name = short_name(r["Name"])
        if name not in KERNEL_FILES:
            continue
        fr = [v for k, vs in fetch.items() if short_name(k) == name for v in vs]
        wr = [v for k, vs in write.items() if short_name(k) == name for v in vs]
        rd = sum(fr) / len(fr) * 1024 * f_scale if fr else float("nan")
        wb = sum(wr) / len(wr) * 1024 * w_scale if wr else float("nan")
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{rd / 1e6:.3f} | {wb / 1e6:.3f} |")
        if fr and wr:
            key = w.name if args.call == "forward" else w.name + "/" + args.call
            table.setdefault(name, {})[key] = {
                "source_sha": source_sha(name), "bytes_per_launch": int(rd + wb),
                "read_bytes": int(rd), "write_bytes": int(wb),
                "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                "avg_us": round(float(r["AverageNs"]) / 1e3, 3)}
    lines.append("")
    if args.sq:
        lines += sq_table(args.sq, args.sq_command, args.chunks_per_wave)
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    with open(args.traffic, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
