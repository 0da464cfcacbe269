"""Build line for tests/c/abi_check.c, the C program that drives libidx
through include/idx.h and the HIP runtime alone (no Python binding)."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_token_fp8_amd")
SRC = os.path.join(ROOT, "tests", "c", "abi_check.c")
EXE = os.path.join(ROOT, "tests", "c", "abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out=EXE):
    return ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM}/include", SRC, "-o", out,
            f"-L{PKG}", "-lidx", f"-L{ROCM}/lib", "-lamdhip64",
            "-Wl,-rpath,$ORIGIN/../../sparse_attention_token_fp8_amd", f"-Wl,-rpath,{ROCM}/lib"]


def build(out=EXE):
    """Compile and link against the built libidx.so; raises on failure."""
    r = subprocess.run(command(out), capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"abi_check.c failed to build:\n{r.stderr}")
    return out
