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


# Kernels whose MFMA blocks must be free of spill code.  Their inner loops
# count outstanding vector-memory operations by hand and chain inline-asm
# MFMAs whose hazards the compiler does not see, so no scratch access and no
# accumulation-register copy may land in a basic block that issues MFMAs.
# Spills elsewhere in the kernel (at entry, around a segment's epilogue) are
# allowed up to a small cap.
HOT_KERNELS = {"k_attn_v2.hip": "attn_v2_kernel"}
MAX_SCRATCH = 256   # bytes per lane
# Kernels that must not touch scratch at all: a spilled load array turns a
# batch of loads in flight into a chain of round trips (a merge kernel once
# ran 2x slower that way).
NO_SCRATCH = {"k_attn_v2.hip": ("combine_v2", "qtile_pack"), "k_gemm_v2.hip": ("wgemm", "absorb"),
              "k_mha.hip": ("mha_decode",),
              "k_prefill.hip": ("attn_prefill_v2", "prefill_rows_v2", "prefill_rope_q_v2"),
              "k_backward_v2.hip": ("attn_bwd_dq_v2", "attn_bwd_dkv_v2", "transpose16",
                                    "bwd_inputs_v2"),
              "k_tgemm.hip": ("tgemm",)}
# Kernels that chain inline-asm MFMAs: the compiler does not model their
# hazards, so a register copy it places between two of them (a VGPR restored
# from an AGPR under register pressure, an accumulator moved) can read or
# overwrite a register an MFMA still uses.  From the first MFMA of each
# instantiation to its last, no scratch access and no AGPR copy is allowed.
# (A 160-row weight-streaming tile with a four-step load ring once compiled to
# such restores and returned garbage.)
MFMA_SPAN_KERNELS = {"k_gemm_v2.hip": ("wgemm_kernel", "wgemm_plan_kernel"),
                     "k_tgemm.hip": ("tgemm_kernel",),
                     "k_prefill.hip": ("attn_prefill_v2_kernel",)}
_SPAN_OPS = ("scratch_", "v_accvgpr_read", "v_accvgpr_write", "v_accvgpr_mov")
_SPILL_OPS = ("scratch_", "buffer_store", "buffer_load", "v_accvgpr_read", "v_accvgpr_write",
              "v_accvgpr_mov")


def _is_spill(line: str) -> bool:
    """A scratch access or accumulation-register copy.  MUBUF loads with the
    lds modifier are the kernels' own direct-to-LDS loads, not spills."""
    code = line.split(";")[0]
    if code.split() and code.split()[-1] == "lds":
        return False
    return any(op in code for op in _SPILL_OPS)


def _check_scratch(src: str, remarks: str):
    """Parse -Rpass-analysis=kernel-resource-usage remarks: the hot kernel's
    scratch stays under its cap, the NO_SCRATCH kernels use none."""
    base = os.path.basename(src)
    caps = {}
    if base in HOT_KERNELS:
        caps[HOT_KERNELS[base]] = MAX_SCRATCH
    for name in NO_SCRATCH.get(base, ()):
        caps[name] = 0
    if not caps:
        return
    cur = None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            cur = line.split("Function Name:")[1].strip()
        elif "ScratchSize [bytes/lane]:" in line and cur is not None:
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
            for name, cap in caps.items():
                if name in cur and size > cap:
                    raise RuntimeError(f"{base}: {cur} uses {size} B of scratch per lane "
                                       f"(cap {cap})")


def _check_hot_blocks(src: str, asm: str):
    """No spill code inside a basic block of the hot kernel that issues MFMAs
    (every instantiation of it)."""
    kernel = HOT_KERNELS[os.path.basename(src)]
    lines = asm.splitlines()
    code = [l.split(";")[0].rstrip() for l in lines]   # drop the assembler's comments
    begins = [i for i, c in enumerate(code)
              if c.endswith(":") and kernel in c and not c.startswith((".", "\t"))]
    if not begins:
        raise RuntimeError(f"{os.path.basename(src)}: {kernel} not found in the assembly")
    bad = []
    for begin in begins:
        block, label = [], lines[begin]
        for l, c in zip(lines[begin + 1:], code[begin + 1:]):
            if c.startswith(".Lfunc_end"):
                break
            is_label = (c.endswith(":") and c.startswith(".LBB")) or l.startswith("; %bb.")
            if is_label:
                if any("v_mfma" in x for x in block):
                    bad += [f"{label.split()[0]} {x.strip()}" for x in block if _is_spill(x)]
                block, label = [], l
            else:
                block.append(l)
    if bad:
        raise RuntimeError(f"{os.path.basename(src)}: spill code in MFMA blocks of {kernel}:\n  "
                           + "\n  ".join(bad[:10]))


def _check_mfma_spans(src: str, asm: str):
    """No scratch access or AGPR copy between the first and the last MFMA of
    any instantiation of the MFMA_SPAN_KERNELS of this source."""
    base = os.path.basename(src)
    names = MFMA_SPAN_KERNELS[base]
    bad, found, cur, body = [], 0, None, []

    def close():
        if cur is None:
            return
        idx = [i for i, x in enumerate(body) if x.startswith("v_mfma")]
        if idx:
            bad.extend(f"{cur[:60]}: {x}" for x in body[idx[0]:idx[-1]]
                       if x.startswith(_SPAN_OPS))

    for line in asm.splitlines():
        c = line.split(";")[0].rstrip()
        if c.endswith(":") and not c.startswith((".", "\t", " ")):
            close()
            cur = c[:-1] if any(n in c for n in names) else None
            found += cur is not None
            body = []
        elif cur is not None:
            body.append(c.strip())
    close()
    if not found:
        raise RuntimeError(f"{base}: none of {names} found in the assembly")
    if bad:
        raise RuntimeError(f"{base}: register copies between inline-asm MFMAs:\n  "
                           + "\n  ".join(bad[:10]))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    _check_scratch(src, r.stderr)
    base = os.path.basename(src)
    if base in HOT_KERNELS or base in MFMA_SPAN_KERNELS:
        s_file = os.path.join(BUILD, base + ".s")
        cmd = [HIPCC, *CFLAGS, "--cuda-device-only", "-S", src, "-o", s_file]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        with open(s_file) as f:
            asm = f.read()
        if base in HOT_KERNELS:
            _check_hot_blocks(src, asm)
        if base in MFMA_SPAN_KERNELS:
            _check_mfma_spans(src, asm)
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


# The host code (the C ABI and its argument checks, mla_api.cpp) under
# AddressSanitizer and UndefinedBehaviorSanitizer, linked with the kernels'
# ordinary objects.  Host-only flags: device code is never built with them.
SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libmla_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The shared ASan runtime of the toolchain's clang (to preload into an
    uninstrumented interpreter)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin",
                         "clang")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the clang ASan runtime was not found")
    return path


def build_sanitized(verbose: bool = True) -> str:
    """libmla with mla_api.cpp compiled under ASan + UBSan (into _build/san)."""
    host_src = os.path.join(CSRC, "mla_api.cpp")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(p) + ".o") for p in srcs]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    os.makedirs(SAN_DIR, exist_ok=True)
    san_obj = os.path.join(SAN_DIR, "mla_api.cpp.o")
    cmd = [HIPCC, *CFLAGS, *SAN_FLAGS, "-c", host_src, "-o", san_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", SAN_LIB, *objs, san_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB} (host code under ASan + UBSan)", file=sys.stderr)
    return SAN_LIB


if __name__ == "__main__":
    build_sanitized() if "--sanitized" in sys.argv else build()
