"""CPU checks of the round-trip matching rules (tests/rt_match.py): they must
accept the oracle's own output and reject an output made with a cutoff one
element-type step away, so the GPU test cannot pass a wrong cutoff."""
import numpy as np
import pytest

import oracle
import synth
from parity import BF16, F16, Z95, decode
from rt_match import _next_up16, cut_candidates, rows_match


def test_next_up16_walks_the_number_line():
    vals = []
    b = 0xBF80          # bf16 -1.0
    for _ in range(20000):
        vals.append(decode(np.array([b], np.uint16), BF16)[0])
        b = _next_up16(b)
    v = np.array(vals)
    assert np.all(np.diff(v) > 0) and v[0] == -1.0 and (v == 0).sum() == 1


@pytest.mark.parametrize("dt", [BF16, F16], ids=["bf16", "f16"])
def test_candidates_hold_the_oracle_cut_and_reject_a_neighbour(dt):
    o = oracle.get()
    x = synth.gelu_offset_rows(48, 2048) if dt == BF16 else synth.gelu_iid(48, 2048, seed=9, dtype=dt)
    d = x.shape[1] // 2
    ref, st = o.gelu_and_mul_sparse_rt(x, dt, Z95)
    cands = cut_candidates(o, decode(x[:, :d], dt), dt, Z95)
    assert all(c is not None and st[2][i] in c for i, c in enumerate(cands))
    assert rows_match(ref, ref, dt).all()
    # A cutoff one step up (the next representable value) must fail the
    # rows where it is not itself a candidate.
    up = np.array([decode(np.array([_next_up16(o.encode(np.array([c]), dt)[0])], np.uint16), dt)[0]
                   for c in st[2]])
    shifted, _ = o.gelu_and_mul_sparse_rt(x, dt, Z95, cut=up)
    single = np.array([len(c) == 1 for c in cands])
    assert single.sum() >= 40
    assert not rows_match(shifted, ref, dt)[single].any()
