"""Build libttt.so (hipcc, gfx950) from csrc/ in place.

Each source is compiled to an object under _build/ with the common flags plus
its own, then the objects are linked into libttt.so.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libttt.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]

# Per-file flags.  The MFMA kernels whose accumulators fit in VGPRs keep them
# there: otherwise the compiler places MFMA results in AGPRs and copies each
# one back to a VGPR before its VALU use (about a quarter of the instructions
# of a chunk of the TTT-Linear scan, and about three thousand copies in the
# momentum scans).  The TTT-MLP kernel's weights already sit in VGPRs without
# the flag.
EXTRA = {
    "ttt_linear_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "ttt_linear_mfma_f32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "ttt_linear_backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "ttt_linear_cols_f32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "ttt_linear_combine.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "ttt_momentum_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    # the MFMA loop of the measured roof: AGPR accumulators make the compiler
    # rotate them through VGPRs every iteration
    "ttt_roofs.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)
