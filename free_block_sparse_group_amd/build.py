"""Build libsparsepr.so (HIP kernels + C ABI) for gfx950 with hipcc.

Usage: python -m free_block_sparse_group_amd.build   (or call build_library()).
The library is written next to this file; objects go to _build/ at the
repository root.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparsepr.so")
SOURCES = ["partition.hip", "assign.hip", "linalg.hip", "route.hip", "attention.hip", "probe.hip", "correct.hip", "peak.hip",
           "sparsepr.cpp"]
ARCH = os.environ.get("SPARSEPR_ARCH", "gfx950")

# packed fp32 VALU forms are kept out of generated code on purpose
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# matrix-core results in ordinary vector registers (no accumulator-register
# copies before the VALU epilogues; fewer registers, higher occupancy) for
# the k-means assignment and the float64 row GEMMs
PER_SOURCE_FLAGS = {
    "assign.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "partition.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wno-unused-result",
          "-I", os.path.join(ROOT, "include")]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _compile(hipcc, src, obj):
    cmd = [hipcc, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + DEVICE_FLAGS + \
        PER_SOURCE_FLAGS.get(src, [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build_library(verbose=True) -> str:
    hipcc = _hipcc()
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)), 8)
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _compile(hipcc, *so), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_library()
    sys.exit(0)
