"""The oracle against the frozen fixture of the small check case."""
import hashlib
import os
import re

import numpy as np

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "gelu_T4_d2048_bf16_seed0.txt")


def _fields():
    out = {}
    for ln in open(GOLD):
        if ln.startswith("#"):
            continue
        for k, v in re.findall(r"(\S+) = (\S+)", ln):
            out[(ln.split()[0], k) if ln.startswith("row") else k] = v
    return out


def test_oracle_matches_frozen_small_case(oracle_lib):
    f = _fields()
    x = synth.gelu_iid(4, 2048, seed=0)
    assert hashlib.sha256(x.tobytes()).hexdigest() == f["input_sha256"]
    y, st = oracle_lib.gelu_and_mul_sparse(x, oracle.BF16, float(np.float32(1.6448536)),
                                           want_stats=True)
    assert hashlib.sha256(y.tobytes()).hexdigest() == f["output_sha256"]
    for r in range(4):
        assert float(f[(f"row{r}", "cutoff")]) == st[2, r]
    assert int(f["nonzero_count"]) == int(np.count_nonzero(oracle_lib.decode(y, oracle.BF16)))
