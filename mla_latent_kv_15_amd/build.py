"""Builds libmla.so (all HIP kernels + the C-ABI host code) for gfx950.

Every source is compiled with hipcc in-tree; the shared library lands next to
this file, where ``mla_latent_kv_15_amd.lib`` loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# Kernels that must not touch scratch memory: their inner loops count
# outstanding vector-memory operations by hand (a spill reload would both
# break that count and stall on it), and their inline-asm MFMA chains rely on
# the compiler never placing spill code between them.
NO_SCRATCH = ("attn_v2_kernel",)


def _check_scratch(src: str, remarks: str):
    """Parse -Rpass-analysis=kernel-resource-usage remarks for NO_SCRATCH kernels."""
    cur = None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            cur = line.split("Function Name:")[1].strip()
        elif "ScratchSize [bytes/lane]:" in line and cur is not None:
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
            if size and any(k in cur for k in NO_SCRATCH):
                raise RuntimeError(f"{os.path.basename(src)}: kernel {cur} uses {size} B of scratch "
                                   f"per lane; its hand-counted memory waits require none")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    _check_scratch(src, r.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,-z,defs", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
