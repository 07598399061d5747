"""Write the regression fixtures in this folder.  Calls only the oracle and the
seeded generator; no value here comes from the GPU path.

The pages print no worked example with numbers, so these fixtures are not
values from the pages: they freeze the oracle's output on the small check
case (T=4, d=2048, bf16, gate and up N(0,1), seed 0, z = 1.6448536) so that a
later change to the oracle or the generator shows up as a diff.

Usage:  python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

Z = float(np.float32(1.6448536))


def main():
    o = oracle.get()
    x = synth.gelu_iid(4, 2048, seed=0)
    y, st = o.gelu_and_mul_sparse(x, oracle.BF16, Z, want_stats=True)
    path = os.path.join(HERE, "gelu_T4_d2048_bf16_seed0.txt")
    with open(path, "w") as f:
        f.write("# gelu_and_mul_sparse, T=4, d=2048, bf16, gate/up N(0,1) seed 0, "
                "z=(float)1.6448536\n")
        f.write("# Op: vLLM PR 48498, section Purpose (per-row mean/variance, "
                "Gaussian cutoff, tanh GELU, times up).\n")
        f.write("# Written by tests/golden/make_golden.py from the fp64 oracle.\n")
        f.write(f"input_sha256 = {hashlib.sha256(x.tobytes()).hexdigest()}\n")
        f.write(f"output_sha256 = {hashlib.sha256(y.tobytes()).hexdigest()}\n")
        for r in range(4):
            f.write(f"row{r} mean = {float(st[0, r])!r}  std = {float(st[1, r])!r}  cutoff = {float(st[2, r])!r}\n")
        nz = np.flatnonzero(o.decode(y, oracle.BF16).ravel())
        f.write(f"nonzero_count = {nz.size}\n")
        for i in nz[:8]:
            f.write(f"out[{i // 2048},{i % 2048}] = 0x{int(y.ravel()[i]):04x}\n")
    print(path)


if __name__ == "__main__":
    main()
