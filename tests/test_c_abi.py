"""The C ABI from C: tests/c_abi_check.c includes include/sa2.h under a C99
compiler, links libsa2.so and checks host-side validation (no GPU needed)."""
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
PKG = ROOT / "block_sparse_attention_sa2_amd"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_caller(tmp_path):
    assert (PKG / "libsa2.so").exists(), "build libsa2.so first"
    exe = tmp_path / "c_abi_check"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", str(ROOT / "include"), str(ROOT / "tests" / "c_abi_check.c"),
                    "-L", str(PKG), "-lsa2", f"-Wl,-rpath,{PKG}", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("c abi ok"), r.stdout
