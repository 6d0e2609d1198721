"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): sparsepr.cpp is rebuilt with both sanitizers on its host side only
(the kernels' objects are the library's own), linked into
tests/cabi_host_check.c, a driver that walks every validation path -- workspace
sizing for valid and invalid arguments, null pointers, short workspaces, the
allocation-free route's size limit, the eigensolver's sizing, the timing hook --
and run.  It must exit 0 with no sanitizer report."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "free_block_sparse_group_amd", "csrc")
KERNEL_OBJS = ["partition", "assign", "linalg", "route", "attention", "probe", "correct", "peak"]
ROCM = "/opt/rocm"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.fixture(scope="module")
def sanitized_driver(tmp_path_factory):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm toolchain not found")
    objs = [os.path.join(ROOT, "_build", n + ".o") for n in KERNEL_OBJS]
    if not all(os.path.exists(o) for o in objs):
        from free_block_sparse_group_amd.build import build_library
        build_library(verbose=False)
    d = tmp_path_factory.mktemp("san")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    abi = str(d / "sparsepr_san.o")
    _run([hipcc, "-x", "hip", "-c", os.path.join(CSRC, "sparsepr.cpp"), "-o", abi, "-O1", "-g", "-fPIC",
          "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include")] + san)
    drv = str(d / "check.o")
    _run([clang, "-x", "c", "-std=c11", "-c", os.path.join(ROOT, "tests", "cabi_host_check.c"), "-o", drv, "-O1",
          "-g", "-I", os.path.join(ROOT, "include"), "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"])
    exe = str(d / "check")
    _run([hipcc, "-o", exe, drv, abi] + objs + ["--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                                                 "-Xarch_host", "-fsanitize=undefined"])
    return exe


def test_cabi_host_paths_clean_under_asan_and_ubsan(sanitized_driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sanitized_driver], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert r.returncode == 0 and "all host checks passed" in out, out
