"""The C-ABI checker (tests/c_abi_check.c) against a build of libsa2 whose
host code carries AddressSanitizer and UndefinedBehaviorSanitizer: every
validation path it drives (null, misaligned and undersized arguments,
unsupported shapes, masks without plans, the allocation-free builder's
limit) runs instrumented, on a host without a GPU.  The device code is
built as usual; only the host half of each HIP source is instrumented."""
import concurrent.futures as cf
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CLANG = Path("/opt/rocm/llvm/bin/clang")
CLANGXX = Path("/opt/rocm/llvm/bin/clang++")

# each sanitizer flag applies to the host compilation only
HOST_SANITIZERS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (CLANG.exists() and CLANGXX.exists()), reason="no ROCm clang")
def test_c_caller_under_host_sanitizers(tmp_path):
    from block_sparse_attention_sa2_amd import build as B
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("no hipcc")
    flags = [f for f in B.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SANITIZERS
    sources = sorted(B.CSRC.glob("*.hip"))

    def compile_one(src: Path) -> Path:
        obj = tmp_path / (src.stem + ".o")
        r = subprocess.run([hipcc, *flags, "-c", str(src), "-o", str(obj)], capture_output=True,
                           text=True)
        assert r.returncode == 0, f"{src.name}:\n{r.stderr[-3000:]}"
        return obj

    with cf.ThreadPoolExecutor(min(len(sources), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, sources))
    lib = tmp_path / "libsa2.so"
    r = subprocess.run([hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", str(lib),
                        *map(str, objs)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]

    # the checker, with the same compiler's sanitizer runtime (linked by the
    # C++ driver so that the library's C++ allocations are intercepted too)
    obj = tmp_path / "c_abi_check.o"
    exe = tmp_path / "c_abi_check"
    r = subprocess.run([str(CLANG), "-std=c99", "-g", "-fsanitize=address,undefined",
                        "-fno-omit-frame-pointer", "-I", str(ROOT / "include"),
                        "-c", str(ROOT / "tests" / "c_abi_check.c"), "-o", str(obj)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(CLANGXX), "-fsanitize=address,undefined", str(obj), "-L",
                        str(tmp_path), "-lsa2", f"-Wl,-rpath,{tmp_path}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]

    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("c abi ok"), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
