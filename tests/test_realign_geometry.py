"""CPU check of the realigning gelu_and_mul_sparse kernel's data movement.

tests/host/realign_emulate.cpp runs every lane of one workgroup through the
kernel's loads, LDS window writes and reads and stores, on the kernel's own
geometry helpers (gated_activation_amd/csrc/ga_realign.h), and checks bounds,
alignment, races on window slots and that each output element meets the
gate and up elements of its own index, with the up row loaded up front or
chunk by chunk.  Cases: both element sizes, the
planner's geometry and the smallest covering geometry of every wave count,
and gate / up / output phases (all of them for short rows, a seeded sample
plus the extremes for long ones).
"""
import itertools
import os
import random
import shutil
import subprocess

import pytest

import gated_activation_amd as ga

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host", "realign_emulate.cpp")

D_VALUES = [1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 63, 64, 65, 127, 128, 129, 500, 1000, 1023, 1024, 1025,
            3000, 4095, 4096, 4097, 8191, 8193, 16383, 16384, 16385, 32767]


@pytest.fixture(scope="module")
def emulator(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("emu") / "realign_emulate")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", "-o", exe, SRC], check=True)
    return exe


def _blocks_max(d, per):
    return (d + 2 * per - 2) // per


def _geometries(d, dtype, per):
    out = set()
    for T in (1, 2048):
        p = ga.plan_gelu_and_mul_sparse(T, d, dtype, aligned=False)
        if p.path == 2:
            out.add((p.waves_per_row, p.per_lane))
    for w in (1, 2, 4, 8, 16):
        v = -(-_blocks_max(d, per) // (64 * w))
        if 1 <= v <= 8:
            out.add((w, v))
    return sorted(out)


def _phases(per, d, rng):
    allp = list(itertools.product(range(per), repeat=3))
    if per == 4 or d <= 130:
        return allp
    ext = [(0, 0, 0), (per - 1, 0, 0), (0, per - 1, 0), (0, 0, per - 1), (per - 1, per - 1, 0),
           (0, per - 1, per - 1), (per - 1, 0, per - 1), (per - 1, per - 1, per - 1)]
    return ext + rng.sample(allp, 24)


def test_realign_kernel_data_movement(emulator):
    rng = random.Random(1234)
    lines = []
    for es, dtype in ((2, ga.GA_BF16), (4, ga.GA_F32)):
        per = 16 // es
        for d in D_VALUES:
            for w, v in _geometries(d, dtype, per):
                for pg, pu, po in _phases(per, d, rng):
                    for late in (0, 1):
                        lines.append(f"{es} {d} {w} {v} {pg} {pu} {po} {late}")
    r = subprocess.run([emulator], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.strip() == f"ok {len(lines)}", r.stdout[-2000:]


def test_planner_uses_the_realigning_path_when_it_covers_the_row():
    for dtype, per, dmax in ((ga.GA_BF16, 8, 65536), (ga.GA_F16, 8, 65536), (ga.GA_F32, 4, 65536)):
        for d in (1, 31, 1000, 8191, 16384, 32767, 32768, 65535, 65536):
            if d > dmax:
                continue
            p = ga.plan_gelu_and_mul_sparse(100, d, dtype, aligned=False)
            if _blocks_max(d, per) <= 8192:
                assert p.path == 2 and p.splits == 1, (dtype, d, p.as_dict())
                assert p.waves_per_row * 64 * p.per_lane >= _blocks_max(d, per)
                assert 1 <= p.per_lane <= 8
            else:
                assert p.path == 1, (dtype, d, p.as_dict())
    # headline-sized rows off a 16-byte boundary
    p = ga.plan_gelu_and_mul_sparse(2048, 16384, ga.GA_BF16, aligned=False)
    assert (p.path, p.waves_per_row, p.per_lane, p.up_late) == (2, 8, 5, 1)
    p = ga.plan_gelu_and_mul_sparse(256, 16384, ga.GA_BF16, aligned=False)
    assert (p.path, p.waves_per_row, p.per_lane, p.up_late) == (2, 16, 3, 0)
