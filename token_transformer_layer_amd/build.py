"""Build the gfx950 shared library libtpshard.so in-tree with hipcc.

    python -m token_transformer_layer_amd.build

The library is the product: every kernel of the layer shard and the C-ABI
declared in include/tpshard.h.  It is always rebuilt from source.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtpshard.so")
SOURCES = ["gemm_tn.hip", "gemm_nn.hip", "gemm_nt.hip", "gemm_mk.hip", "attention.hip", "norm.hip", "gemm.hip", "api.cpp", "trace.cpp",
           "slicing.cpp", "noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off (only scalar/vector fp32 code is emitted)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libtpshard.so")
    return path


def build(verbose=False, jobs=None):
    """Compile every source to an object file (in parallel: the kernel files
    dominate), then link the shared library."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    base = [cc] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = base + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        return obj, res

    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(compile_one, SOURCES))
    failed = [r for _, r in results if r.returncode != 0]
    for r in failed:
        sys.stderr.write(r.stdout + r.stderr)
    if failed:
        raise RuntimeError("hipcc failed building libtpshard.so")
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for o, _ in results] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking libtpshard.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
