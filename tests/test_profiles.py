"""The committed rocprofv3 summaries that bench.py reads match the kernel
sources they were taken on.

bench.py reports a kernel's measured HBM traffic (the roofline object's
`traffic`) only when the summary's recorded source digest equals the digest
of the current kernel sources; otherwise it reports null.  This test fails
as soon as a kernel source changes without its counters being taken again,
and checks that each record's figures are self-consistent.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _fields(path):
    out = {}
    for ln in open(path):
        if "=" in ln and not ln.lstrip().startswith("#"):
            k, v = ln.split("=", 1)
            out[k.strip()] = v.split()[0]
    return out


def test_headline_traffic_record_is_current():
    got = bench.recorded_traffic()
    assert got is not None, "headline counters were taken on other kernel sources"
    f = _fields(bench.TRAFFIC_FILE)
    assert got == int(f["hbm_bytes_per_launch"])
    assert int(f["algorithmic_bytes_per_launch"]) == 2048 * 16384 * 3 * 2
    assert 1.0 <= got / int(f["algorithmic_bytes_per_launch"]) < 1.01


def test_silu_traffic_record_is_current():
    got = bench.recorded_traffic(bench.SILU_TRAFFIC_FILE, bench.SILU_SOURCES,
                                 f"live{bench.SILU_M}_hbm_bytes_per_launch")
    assert got is not None, "silu counters were taken on other kernel sources"
    assert 1.0 <= got / (bench.SILU_M * bench.SILU_D * 3 * 2 + 4) < 1.01


def test_down_projection_traffic_record_is_current():
    got = bench.recorded_traffic(bench.DOWN_TRAFFIC_FILE, bench.DOWN_SOURCES,
                                 f"T{bench.DOWN_ROOFLINE_T}_hbm_bytes_per_call")
    assert got is not None, "fused down-projection counters were taken on other kernel sources"
    T, d, H = bench.DOWN_ROOFLINE_T, bench.DOWN_D, bench.DOWN_H
    alg = H * d * 2 + T * 2 * d * 2 + T * H * 2
    assert int(_fields(bench.DOWN_TRAFFIC_FILE)[f"T{T}_algorithmic_bytes_per_call"]) == alg
    assert 1.0 <= got / alg < 1.02
