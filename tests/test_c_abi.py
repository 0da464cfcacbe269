"""The C ABI used from C alone: tests/c/abi_check.c includes only idx.h and
the HIP runtime, builds a batch whose top-k rows are known in closed form and
checks every entry point it calls (see the program's header)."""

import os
import subprocess

import pytest

from tests import c_abi_build


def test_c_program_compiles_against_header(tmp_path):
    """idx.h is valid C11 and every call the program makes links against libidx.so."""
    if not os.path.exists(os.path.join(c_abi_build.PKG, "libidx.so")):
        pytest.fail("libidx.so is not built")
    c_abi_build.build(out=str(tmp_path / "abi_check"))
    assert os.path.getsize(tmp_path / "abi_check") > 0


@pytest.mark.gpu
def test_c_program_on_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(c_abi_build.EXE), "tests/c/abi_check is built by __graft_entry__.build()"
    print("running", c_abi_build.EXE, flush=True)
    r = subprocess.run([c_abi_build.EXE], capture_output=True, text=True, timeout=100)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "abi_check: ok" in r.stdout
