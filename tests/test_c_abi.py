"""The header is plain C: a C99 program includes it, links the library and checks the
host-side refusals (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

from gated_deltanet_linear_decode_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_uses_the_header_and_library(tmp_path):
    lib_dir = os.path.dirname(abi.LIB_PATH)
    assert os.path.exists(abi.LIB_PATH), "build the library first"
    exe = tmp_path / "abi_refusals"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_refusals.c"), "-o", str(exe),
                    "-L", lib_dir, "-l:libgdn_block.so", "-Wl,-rpath," + lib_dir], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failed" in r.stdout
