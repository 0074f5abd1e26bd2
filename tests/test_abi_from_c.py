"""The C ABI from plain C: tests/abi_from_c.c is compiled with gcc against
include/ab_attn.h, linked to the built libabattn.so and run (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

import block_sparse_attention_ibcs_amd as ab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_usable_from_c(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib = ab.library_path()
    if not os.path.exists(lib):
        pytest.fail("libabattn.so not built")
    exe = tmp_path / "abi_from_c"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "abi_from_c.c"), lib, "-Wl,-rpath," + os.path.dirname(lib),
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert "all checks passed" in res.stdout
