"""Build libidx.so for gfx950 in-tree with hipcc (no GPU needed).

    python sparse_attention_token_fp8_amd/build.py

This file imports nothing from the package (whose import needs the built
library), so it is run or loaded by its file path.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libidx.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source extras.  The scoring kernels: ReLU on MFMA results needs no NaN
# canonicalisation, and MFMA results stay in VGPRs (no AGPR round trip).
SCORE_FLAGS = ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA = {
    "score.hip": SCORE_FLAGS,
    "fused.hip": SCORE_FLAGS,
    "fp4.hip": SCORE_FLAGS,
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


# Scratch memory a kernel may use per lane: a few spilled registers outside
# its loops (the prefill scoring kernel holds 256 VGPRs and spills two before
# its block loop); more means a register array was put in memory.
SCRATCH_LIMIT = 16


def _scratch_kernels(remarks):
    """Kernels whose resource-usage remarks report more than SCRATCH_LIMIT
    bytes of scratch memory per lane."""
    bad, name = [], None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split()[0]
        elif "ScratchSize [bytes/lane]:" in line:
            n = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
            if n > SCRATCH_LIMIT and name is not None:
                bad.append(f"{name} ({n} bytes/lane)")
    return bad


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []),
           "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stderr}")
    # every kernel keeps its state in registers and LDS: scratch memory in a
    # hot loop costs more than the kernel's whole K stream
    bad = _scratch_kernels(r.stderr)
    if bad:
        raise RuntimeError(f"{os.path.basename(src)}: kernels using scratch memory: " + ", ".join(bad))
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
