"""Build libga.so (the HIP kernels for gfx950 plus the C-ABI) in place.

    python -m gated_activation_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Packed-fp32 instructions are
switched off (-packed-fp32-ops): the kernels are memory-bound and gain nothing
from them.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libga.so")
SOURCES = ["api.hip", "gelu_sparse.hip", "gelu_sparse_split.hip", "gelu_sparse_unaligned.hip", "gelu_sparse_rows.hip",
           "gelu_sparse_rep.hip", "gelu_sparse_decode.hip", "gelu_sparse_staged.hip", "gelu_sparse_tiled.hip",
           "elementwise.hip"]
ARCH = "gfx950"


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    objs = []
    procs = []
    flags = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]
    for src in SOURCES:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = [hipcc] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True))
        objs.append(obj)
        if len(procs) >= jobs:
            _wait(procs)
    _wait(procs)
    link = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    for o in objs:
        os.remove(o)
    return LIB


def _wait(procs):
    failed = []
    while procs:
        p = procs.pop(0)
        _, err = p.communicate()
        err = "\n".join(ln for ln in err.splitlines()
                        if "packed-fp32-ops" not in ln and "warning: argument unused" not in ln)
        if err.strip():
            sys.stderr.write(err + "\n")
        if p.returncode != 0:
            failed.append(p.args)
    if failed:
        raise RuntimeError(f"hipcc failed: {failed}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
