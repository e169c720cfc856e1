"""Build liblmoe.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m sparse_moe_transformer_gemm_amd.build [-v]

Objects go to sparse_moe_transformer_gemm_amd/_build/, the library next to
this file.  Every call compiles from scratch.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblmoe.so")

SOURCES = ["kernels.hip", "lmoe_api.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 ALU ops stay off: scalar fp32 only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblmoe.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose: bool = False, defines=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every HIP source for gfx950 and link liblmoe.so; returns its
    path.  `defines` (NAME=VALUE strings) and `out` build a variant elsewhere."""
    hipcc = _hipcc()
    os.makedirs(build_dir, exist_ok=True)
    flags = FLAGS + [f"-D{d}" for d in defines]
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        for s in SOURCES:
            o = os.path.join(build_dir, os.path.splitext(s)[0] + ".o")
            objs.append(o)
            jobs.append(ex.submit(_run, [hipcc, *flags, "-c", os.path.join(CSRC, s), "-o", o], verbose))
        for j in jobs:
            log = j.result()
            if verbose and log.strip():
                print(log)
    tmp = out + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
