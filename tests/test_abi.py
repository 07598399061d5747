"""The C-ABI on the host: exports, argument checks and the launch planner.

No kernel runs here: every call below is rejected by a host-side check, or has
zero rows, before the library makes any HIP call.
"""
import ctypes
import os
import re

import pytest

import gated_activation_amd as ga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ga.h")
L = ga.lib
BF16, F16, F32 = ga.GA_BF16, ga.GA_F16, ga.GA_F32
OK, EINVAL, EUNSUP = ga.GA_OK, ga.GA_EINVAL, ga.GA_EUNSUPPORTED
Z = ctypes.c_float(1.6448536)
# Fake device addresses: never dereferenced, since every call is rejected (or
# has no rows) before a launch.
IN = ctypes.c_void_p(0x7F0000000000)
OUT = ctypes.c_void_p(0x7F1000000000)
LIVE = ctypes.c_void_p(0x7F2000000000)
WS = ctypes.c_void_p(0x7F3000000000)
WS_BYTES = 1 << 30


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ga_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "ga_gelu_and_mul_sparse" in names and "ga_silu_and_mul_bounded" in names
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    assert L.ga_status_str(OK) == b"GA_OK"
    assert L.ga_status_str(EINVAL) == b"GA_EINVAL"
    assert L.ga_status_str(EUNSUP) == b"GA_EUNSUPPORTED"
    assert L.ga_status_str(ga.GA_EHIP) == b"GA_EHIP"
    assert L.ga_version() >= 100


def gelu(in_=IN, out=OUT, T=4, d=2048, dt=BF16, z=Z, live=None):
    return L.ga_gelu_and_mul_sparse(in_, out, T, d, dt, z, live, None)


def silu(in_=IN, out=OUT, M=16, d=768, dt=BF16, live=LIVE):
    return L.ga_silu_and_mul_bounded(in_, out, M, d, dt, live, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(in_=None), EINVAL),
    (dict(out=None), EINVAL),
    (dict(T=-1), EINVAL),
    (dict(T=2 ** 31), EINVAL),
    (dict(d=0), EINVAL),
    (dict(d=-5), EINVAL),
    (dict(d=65537), EUNSUP),
    (dict(dt=3), EINVAL),
    (dict(dt=-1), EINVAL),
    (dict(z=ctypes.c_float(float("nan"))), EINVAL),
    (dict(z=ctypes.c_float(float("inf"))), EINVAL),
    (dict(out=IN), EINVAL),                                    # in place
    (dict(out=ctypes.c_void_p(0x7F0000000000 + 4 * 4096 * 2 - 2)), EINVAL),  # partial overlap
    (dict(in_=ctypes.c_void_p(0x7F0000000001)), EINVAL),       # not element aligned
    (dict(T=0), OK),                                           # nothing to do, no launch
    (dict(T=0, d=1, dt=F32), OK),
])
def test_gelu_argument_checks(kwargs, status):
    assert gelu(**kwargs) == status
    if status != OK:
        assert len(L.ga_last_error()) > 0


@pytest.mark.parametrize("kwargs,status", [
    (dict(in_=None), EINVAL),
    (dict(live=None), EINVAL),
    (dict(M=-1), EINVAL),
    (dict(d=0), EINVAL),
    (dict(dt=9), EINVAL),
    (dict(d=65537), EUNSUP),
    (dict(M=2 ** 21, d=1024), EUNSUP),                         # M * d >= 2^31
    (dict(out=IN), EINVAL),
    (dict(M=0), OK),
])
def test_silu_argument_checks(kwargs, status):
    assert silu(**kwargs) == status


def test_misaligned_live_count_is_rejected():
    bad = ctypes.c_void_p(0x7F2000000002)
    assert L.ga_gelu_and_mul_sparse(IN, OUT, 4, 2048, BF16, Z, bad, None) == EINVAL
    assert L.ga_silu_and_mul_bounded(IN, OUT, 16, 768, BF16, bad, None) == EINVAL
    assert L.ga_squared_relu_bounded(IN, OUT, 16, 768, BF16, bad, None) == EINVAL
    assert L.ga_gelu_and_mul(IN, OUT, 16, 768, BF16, 1, bad, None) == EINVAL
    assert b"aligned" in L.ga_last_error()


def test_stream_xor_rows_checks():
    assert L.ga_stream_xor_rows(IN, OUT, 4, 24, None) == EINVAL       # not a multiple of 16
    assert L.ga_stream_xor_rows(None, OUT, 4, 32, None) == EINVAL
    assert L.ga_stream_xor_rows(IN, IN, 4, 32, None) == EINVAL
    assert L.ga_stream_xor_rows(IN, OUT, 0, 32, None) == OK


def test_gelu_planner_known_shapes():
    # (T, d) -> (path, waves per workgroup, vectors per lane, up loaded late, splits)
    want = {(2048, 16384): (0, 8, 4, 1, 1), (2048, 32768): (0, 16, 4, 1, 1), (4096, 65536): (0, 16, 8, 1, 1),
            # few rows: replicated statistics (path 4) or split rows (path 0, with a workspace)
            (1, 32768): (4, 16, 4, 0, 8), (64, 16384): (4, 8, 4, 0, 4), (64, 32768): (4, 8, 8, 0, 4),
            (128, 32768): (4, 16, 4, 0, 2), (1, 8192): (4, 8, 2, 0, 8), (8, 32768): (0, 4, 2, 0, 8),
            (64, 65536): (0, 8, 4, 0, 4)}
    for (T, d), w in want.items():
        p = ga.plan_gelu_and_mul_sparse(T, d, BF16)
        assert (p.path, p.waves_per_row, p.per_lane, p.up_late, p.splits) == w, (T, d, p.as_dict())
        grid = (T + 7) // 8 * 8 * p.splits if p.path == 4 else T * p.splits
        assert p.block == 64 * p.waves_per_row and p.grid == grid


def test_row_geometry_follows_the_measured_table():
    """One workgroup per row: the planner's geometry is the one the measured
    table's interpolation rule picks, checked against the independent Python
    statement of that rule in tests/planner_rule.py over on- and off-grid
    shapes; every choice is a compiled geometry covering the row."""
    import planner_rule as mt
    table = mt.read_inc(os.path.join(ROOT, "gated_activation_amd", "csrc", "planner_table.inc"))
    rep = mt.read_inc(os.path.join(ROOT, "gated_activation_amd", "csrc", "planner_table_rep.inc"), "kRep")
    Ts = sorted(set(table[0]) | {1, 7, 33, 100, 300, 700, 900, 1800, 2500, 3500, 5000, 10000, 20000, 65535})
    Ns = sorted(set(table[1]) | {33, 63, 65, 72, 88, 140, 200, 300, 420, 600, 700, 1100, 1376, 1664, 1792,
                                 2368, 2752, 3200, 3800, 4500, 8191})
    for T in Ts:
        for n in Ns:
            p = ga.plan_gelu_and_mul_sparse(T, n * 8, BF16, with_workspace=False)
            r = mt.choose_rep(rep, T, n, with_workspace=False)
            if r is not None:     # few rows: replicated statistics (checked in the test below)
                assert p.path == 4, (T, n, p.as_dict())
                continue
            assert p.path == 0 and p.splits == 1
            got = (p.waves_per_row, p.per_lane, p.up_late)
            assert p.waves_per_row * 64 * p.per_lane >= n
            want = mt.choose(table, T, n)
            if got != want:
                # only a floating-point tie may differ
                sc = mt.scores(table, T, n)
                gi = mt.GEOS.index(got)
                wi = mt.GEOS.index(want)
                assert sc[gi] is not None and abs(sc[gi] - sc[wi]) < 1e-9, (T, n, got, want)
    # the headline shape keeps 8 waves of 4 vectors with up loaded late
    p = ga.plan_gelu_and_mul_sparse(2048, 16384, BF16)
    assert (p.waves_per_row, p.per_lane, p.up_late) == (8, 4, 1)
    # rows off 16-byte alignment: the unaligned path's own table, the same rule
    una = mt.read_inc(os.path.join(ROOT, "gated_activation_amd", "csrc", "planner_table_una.inc"), "kUna")
    for T in Ts:
        for n in Ns:
            if n <= 32:
                continue
            for d in (n * 8, n * 8 - 3):          # a shifted base; an odd d (partial last vector)
                p = ga.plan_gelu_and_mul_sparse(T, d, BF16, aligned=False)
                nv = -(-d * 2 // 16)
                assert p.path == 2 and p.splits == 1 and p.waves_per_row * 64 * p.per_lane >= nv
                got, want = (p.waves_per_row, p.per_lane, p.up_late), mt.choose(una, T, nv)
                if got != want:
                    sc = mt.scores(una, T, nv)
                    assert abs(sc[mt.GEOS.index(got)] - sc[mt.GEOS.index(want)]) < 1e-9, (T, d, got, want)


def test_split_choice_follows_the_measured_table():
    """Few long rows with a workspace: whether and how the planner splits rows
    is the split table's choice under the interpolation rule, checked against
    the independent Python statement in tests/planner_rule.py on and off the
    grid; outside the table (more rows, shorter rows) nothing is split."""
    import planner_rule as mt
    table = mt.read_inc(os.path.join(ROOT, "gated_activation_amd", "csrc", "planner_table_split.inc"), "kSplit")
    rep = mt.read_inc(os.path.join(ROOT, "gated_activation_amd", "csrc", "planner_table_rep.inc"), "kRep")
    Ts = sorted(set(table[0]) | {3, 5, 12, 40, 72, 100, 112, 200, 224})
    Ns = sorted(set(table[1]) | {1100, 1400, 1700, 2047, 2049, 2200, 2816, 3328, 4608, 5632, 7680, 8191})
    for T in Ts:
        for n in Ns:
            p = ga.plan_gelu_and_mul_sparse(T, n * 8, BF16, with_workspace=True)
            if mt.choose_rep(rep, T, n, with_workspace=True) is not None:
                assert p.path == 4, (T, n, p.as_dict())
                continue
            want = mt.choose_split(table, T, n)
            if want is None:
                assert p.splits == 1, (T, n, p.as_dict())
                continue
            got = (p.waves_per_row, p.per_lane, p.splits)
            if got != want:
                sc = mt.scores(table, T, n, [c for c in range(mt.ROW + 1) if mt.split_valid(c, n)])
                gi = mt.ROW if p.splits == 1 else mt.SPLIT_CHUNKS.index(got[:2])
                wi = mt.SPLIT_CHUNKS.index(want[:2])
                assert sc[gi] is not None and abs(sc[gi] - sc[wi]) < 1e-9, (T, n, got, want)
            assert p.up_late == 0 and p.grid == T * p.splits
            chunk = p.waves_per_row * 64 * p.per_lane
            assert chunk * p.splits >= n > chunk * (p.splits - 1)
    for T, n in ((257, 8192), (4096, 8192), (8, 1023), (1, 1024), (64, 1024)):
        p = ga.plan_gelu_and_mul_sparse(T, n * 8, BF16, with_workspace=True)
        assert p.path == 4 or p.splits == 1, (T, n, p.as_dict())     # no split rows here


def test_rep_choice_follows_the_measured_table():
    """Few rows: whether and how the planner replicates the statistics is the
    replicated table's choice under the interpolation rule, checked against
    the independent Python statement in tests/planner_rule.py on and off the
    grid, with and without a workspace (without one the split plans are not
    candidates); every replicated geometry covers the row."""
    import planner_rule as mt
    rep = mt.read_inc(os.path.join(ROOT, "gated_activation_amd", "csrc", "planner_table_rep.inc"), "kRep")
    Ts = sorted(set(rep[0]) | {3, 5, 12, 40, 80, 112, 160, 224, 257, 300})
    Ns = sorted(set(rep[1]) | {255, 300, 640, 900, 1280, 2500, 3584, 5120, 7000})
    n_rep = 0
    for T in Ts:
        for n in Ns:
            for ws in (True, False):
                p = ga.plan_gelu_and_mul_sparse(T, n * 8, BF16, with_workspace=ws)
                want = mt.choose_rep(rep, T, n, with_workspace=ws)
                if p.path == 4:
                    n_rep += 1
                    got = (p.waves_per_row, p.per_lane, p.splits)
                    assert p.waves_per_row * 64 * p.per_lane >= n and p.up_late == 0
                    assert p.grid == (T + 7) // 8 * 8 * p.splits and p.block == 64 * p.waves_per_row
                    if got != want:
                        valid = [c for c in range(mt.REP_SPLIT + 1) if mt.rep_valid(c, n, ws)]
                        sc = mt.scores(rep, T, n, valid)
                        assert want is not None and abs(sc[mt.REP_GEOS.index(got)] - sc[mt.REP_GEOS.index(want)]) < 1e-9, \
                            (T, n, ws, got, want)
                else:
                    assert want is None, (T, n, ws, p.as_dict(), want)
    assert n_rep > 50
    # beyond 256 rows, beyond the table's row sizes and off 16-byte alignment: never replicated
    for T, d, aligned in ((257, 8192, True), (1, 2040, True), (1, 65544, True), (4, 8192, False)):
        if d <= 65536:
            assert ga.plan_gelu_and_mul_sparse(T, d, BF16, aligned=aligned).path != 4


def test_planner_paths_by_row_size():
    # short rows: packed, several rows per wavefront
    for d, g, v in ((8, 4, 1), (24, 4, 1), (64, 8, 1), (128, 16, 1), (256, 32, 1), (200, 32, 1)):
        p = ga.plan_gelu_and_mul_sparse(4096, d, BF16)
        assert (p.path, p.lanes_per_row, p.per_lane, p.block, p.grid) == (3, g, v, 256, 4096 * g // 256), (d, p.as_dict())
    assert ga.plan_gelu_and_mul_sparse(4096, 264, BF16).path == 0      # 33 vectors: one row per workgroup
    # short rows off 16-byte alignment are packed too (unaligned 16-byte vectors, a partial last one)
    for d, aligned, g, v in ((7, True, 4, 1), (1, True, 4, 1), (255, True, 32, 1), (64, False, 8, 1),
                             (129, True, 32, 1), (33, False, 8, 1)):
        p = ga.plan_gelu_and_mul_sparse(4096, d, BF16, aligned=aligned)
        assert (p.path, p.lanes_per_row, p.per_lane) == (3, g, v), (d, aligned, p.as_dict())
    assert ga.plan_gelu_and_mul_sparse(4096, 257, BF16).path == 2      # 33 vectors: unaligned path
    assert ga.plan_gelu_and_mul_sparse(4096, 127, F32).path == 3       # 32 vectors of fp32
    # without a workspace the rows are never split (few rows may still replicate the statistics)
    p = ga.plan_gelu_and_mul_sparse(1, 32768, BF16, with_workspace=False)
    assert (p.path, p.splits, p.waves_per_row, p.per_lane) == (4, 8, 16, 4)
    p = ga.plan_gelu_and_mul_sparse(300, 32768, BF16, with_workspace=False)
    assert (p.path, p.splits) == (0, 1)
    # rows off 16-byte alignment: the unaligned path (its geometry: see the table test)
    p = ga.plan_gelu_and_mul_sparse(7, 8191, F16)            # odd d
    assert p.path == 2 and p.splits == 1 and p.waves_per_row * 64 * p.per_lane >= (8191 + 7) // 8
    p = ga.plan_gelu_and_mul_sparse(7, 8192, F16, aligned=False)
    assert p.path == 2 and p.waves_per_row * 64 * p.per_lane >= 1024
    p = ga.plan_gelu_and_mul_sparse(7, 65536, F32)           # beyond the vector reach
    assert p.path == 1 and p.waves_per_row * 64 * p.per_lane >= 65536
    p = ga.plan_gelu_and_mul_sparse(7, 65536, BF16, aligned=False)   # 8192 vectors: still unaligned path
    assert (p.path, p.waves_per_row, p.per_lane) == (2, 16, 8)
    p = ga.plan_gelu_and_mul_sparse(7, 32769, F32, aligned=False)    # 8193 vectors: element path
    assert p.path == 1


def test_workspace_size_and_split_plan_checks():
    assert L.ga_gelu_and_mul_sparse_workspace_bytes(0) == 0
    assert L.ga_gelu_and_mul_sparse_workspace_bytes(1) == 256
    assert L.ga_gelu_and_mul_sparse_workspace_bytes(64) == 64 * 256
    split = ga.Plan(path=0, waves_per_row=4, per_lane=2, splits=4, block=256)
    call = lambda p, T=8, ws=WS, nb=WS_BYTES, d=16384: L.ga_gelu_and_mul_sparse_with_plan(  # noqa: E731
        IN, OUT, T, d, BF16, Z, None, ctypes.byref(p), ws, nb, None)
    assert call(split, ws=None) == EINVAL                                # needs a workspace
    assert call(split, nb=8 * 256 - 1) == EINVAL                          # too small
    assert call(split, ws=ctypes.c_void_p(0x7F3000000010)) == EINVAL     # not 256-byte aligned
    assert call(split, T=0) == OK
    bad = ga.Plan(path=0, waves_per_row=8, per_lane=1, block=512, splits=5)   # 5 x 512 > 2048 + 512
    assert call(bad, T=0) == EUNSUP
    bad = ga.Plan(path=0, waves_per_row=8, per_lane=1, block=512, splits=3)   # 3 x 512 < 2048
    assert call(bad, T=0) == EUNSUP
    bad = ga.Plan(path=0, waves_per_row=8, per_lane=1, up_late=1, block=512, splits=4)
    assert call(bad, T=0) == EUNSUP
    bad = ga.Plan(path=0, waves_per_row=8, per_lane=8, block=512, splits=2)   # 8 per lane: no split kernel
    assert call(bad, T=0, d=65536) == EUNSUP
    bad = ga.Plan(path=1, waves_per_row=4, per_lane=16, block=256, splits=2)
    assert call(bad, T=0, d=4096) == EUNSUP
    assert call(ga.Plan(path=0, waves_per_row=4, per_lane=2, block=256, splits=3), T=0, d=12288) == OK
    assert call(split, T=65536, nb=1 << 40) == EUNSUP                    # beyond the grid's y limit
    # the workspace entry point validates like the others
    assert L.ga_gelu_and_mul_sparse_ws(None, OUT, 4, 64, BF16, Z, None, WS, WS_BYTES, None) == EINVAL
    assert L.ga_gelu_and_mul_sparse_ws(IN, OUT, 0, 64, BF16, Z, None, WS, WS_BYTES, None) == OK


def test_noalloc_entry_point_host_checks():
    """The no-allocation entry point checks its arguments like the others
    and serves at most GA_SPLIT_PLAN_ROWS rows; every rejection happens
    before any HIP call."""
    f = L.ga_gelu_and_mul_sparse_noalloc
    assert f(IN, OUT, 257, 32768, BF16, Z, None, None) == EUNSUP
    assert b"at most 256 rows" in L.ga_last_error()
    assert f(IN, OUT, 1 << 20, 64, BF16, Z, None, None) == EUNSUP
    assert f(None, OUT, 4, 2048, BF16, Z, None, None) == EINVAL
    assert f(IN, IN, 4, 2048, BF16, Z, None, None) == EINVAL
    assert f(IN, OUT, 4, 0, BF16, Z, None, None) == EINVAL
    assert f(IN, OUT, 4, 65537, BF16, Z, None, None) == EUNSUP
    assert f(IN, OUT, 4, 2048, 7, Z, None, None) == EINVAL
    assert f(IN, OUT, 4, 2048, BF16, ctypes.c_float(float("nan")), None, None) == EINVAL
    assert f(IN, OUT, 4, 2048, BF16, Z, ctypes.c_void_p(0x7F2000000002), None) == EINVAL
    assert f(IN, OUT, -1, 2048, BF16, Z, None, None) == EINVAL
    assert f(IN, OUT, 0, 2048, BF16, Z, None, None) == OK          # no rows: nothing launched
    # its source resolves the array's device address and never names the array
    # in a kernel argument or copy
    src = open(os.path.join(ROOT, "gated_activation_amd", "csrc", "api.hip")).read()
    assert "hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))" in src
    assert "hipMalloc" not in src and "hipFree" not in src


def test_launches_of_2pow32_work_items_are_unsupported():
    """One launch holds fewer than 2^32 work-items (grid x block).  One
    workgroup per row reaches that at T = 2^26 rows of d = 512 bf16 (one
    64-lane wave per row); the packed short rows (32 lanes per row) at
    T = 2^27 rows of d = 256.  Both inputs fit in HBM, so the planner and the
    entry points return GA_EUNSUPPORTED, before any HIP call."""
    far_in = ctypes.c_void_p(0x100000000000)      # 128 GiB inputs: no overlap with far_out
    far_out = ctypes.c_void_p(0x700000000000)
    p = ga.Plan()
    for T, d in ((1 << 26, 512), (1 << 27, 256), ((1 << 31) - 1, 8), ((1 << 31) - 1, 65536)):
        assert L.ga_plan_gelu_and_mul_sparse(T, d, BF16, 1, 256, 0, ctypes.byref(p)) == EUNSUP, (T, d)
        assert b"2^32" in L.ga_last_error()
        if T * 3 * d * 2 < 0x600000000000:      # buffers that fit between far_in and far_out
            assert L.ga_gelu_and_mul_sparse(far_in, far_out, T, d, BF16, Z, None, None) == EUNSUP, (T, d)
    # just below: the plan is returned, and its launch stays under 2^32
    for T, d in (((1 << 26) - 1, 512), ((1 << 27) - 8, 256), (1 << 20, 65536)):
        assert L.ga_plan_gelu_and_mul_sparse(T, d, BF16, 1, 256, 0, ctypes.byref(p)) == OK, (T, d)
        assert p.grid * p.block < 1 << 32
    # an explicit plan is held to the same bound (rejected before a launch)
    one_wave = ga.Plan(path=0, waves_per_row=1, per_lane=1, block=64)
    st = L.ga_gelu_and_mul_sparse_with_plan(far_in, far_out, 1 << 26, 512, BF16, Z, None, ctypes.byref(one_wave),
                                            None, 0, None)
    assert st == EUNSUP
    sixteen = ga.Plan(path=0, waves_per_row=16, per_lane=1, block=1024)
    st = L.ga_gelu_and_mul_sparse_with_plan(far_in, far_out, 1 << 22, 512, BF16, Z, None, ctypes.byref(sixteen),
                                            None, 0, None)
    assert st == EUNSUP


def test_split_rows_only_in_calls_of_few_rows():
    """The planner splits rows only in calls of at most GA_SPLIT_PLAN_ROWS
    rows (the header's constant, mirrored by the binding), so the binding's
    fixed workspace of workspace_bytes(GA_SPLIT_PLAN_ROWS) serves every call."""
    m = re.search(r"#define GA_SPLIT_PLAN_ROWS (\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == ga.GA_SPLIT_PLAN_ROWS == 256
    assert ga.WORKSPACE_BYTES == L.ga_gelu_and_mul_sparse_workspace_bytes(ga.GA_SPLIT_PLAN_ROWS) == 256 * 256
    assert ga.plan_gelu_and_mul_sparse(224, 65536, BF16).splits > 1
    for d in (8192, 12288, 16384, 24576, 32768, 49152, 65536):
        for T in (257, 300, 1000, 65535):
            assert ga.plan_gelu_and_mul_sparse(T, d, BF16, with_workspace=True).splits == 1, (T, d)


@pytest.mark.parametrize("dt", [BF16, F16, F32])
def test_gelu_planner_covers_every_d(dt):
    """Every d the library takes maps to an instantiated kernel covering the
    row (checked by the library's own plan validation, with zero rows)."""
    es = 4 if dt == F32 else 2
    ds = sorted(set(list(range(1, 600)) + [2 ** k + o for k in range(9, 17) for o in (-9, -1, 0, 1, 8)]
                    + [2000, 3000, 8191, 65536]))
    for d in ds:
        if d > 65536:
            continue
        for aligned in (True, False):
            p = ga.plan_gelu_and_mul_sparse(3, d, dt, aligned=aligned)
            if p.path == 3:   # packed rows: 256 lanes, 256 / lanes_per_row rows per workgroup
                assert p.block == 256 and p.grid == -(-3 // (256 // p.lanes_per_row))
                assert d * es <= 32 * 16
            elif p.path == 4:  # replicated statistics: rows rounded up to a group of 8
                assert aligned and p.block == p.waves_per_row * 64 and p.grid == 8 * p.splits
            else:
                assert d * es > 32 * 16
                assert p.block == p.waves_per_row * 64 and p.grid == 3 * p.splits
            if p.path == 0:
                assert aligned and (d * es) % 16 == 0 and d * es > 32 * 16
            # With zero rows the entry point validates the plan and returns.
            base_in = ctypes.c_void_p(0x7F0000000000)
            base_out = ctypes.c_void_p(0x7F8000000000)
            st = L.ga_gelu_and_mul_sparse_with_plan(base_in, base_out, 0, d, dt, Z, None,
                                                    ctypes.byref(p), WS, WS_BYTES, None)
            assert st == OK, (d, dt, aligned, p.as_dict(), L.ga_last_error())


def test_gelu_with_plan_rejects_bad_geometry():
    p = ga.Plan(path=0, waves_per_row=1, per_lane=1, block=64, grid=1)
    st = L.ga_gelu_and_mul_sparse_with_plan(IN, OUT, 0, 2048, BF16, Z, None, ctypes.byref(p), WS, WS_BYTES, None)
    assert st == EUNSUP                                           # covers 512 < 2048
    p = ga.Plan(path=0, waves_per_row=4, per_lane=1, up_late=2, block=256, grid=1)
    assert L.ga_gelu_and_mul_sparse_with_plan(IN, OUT, 0, 2048, BF16, Z, None, ctypes.byref(p), WS, WS_BYTES, None) == EUNSUP
    p = ga.Plan(path=0, waves_per_row=4, per_lane=1, up_late=1, block=256, grid=1)
    assert L.ga_gelu_and_mul_sparse_with_plan(IN, OUT, 0, 2048, BF16, Z, None, ctypes.byref(p), WS, WS_BYTES, None) == OK
    p = ga.Plan(path=0, waves_per_row=3, per_lane=8, block=192, grid=1)
    assert L.ga_gelu_and_mul_sparse_with_plan(IN, OUT, 0, 64, BF16, Z, None, ctypes.byref(p), WS, WS_BYTES, None) == EUNSUP
    p = ga.Plan(path=1, waves_per_row=16, per_lane=2, block=1024, grid=1)
    assert L.ga_gelu_and_mul_sparse_with_plan(IN, OUT, 0, 64, BF16, Z, None, ctypes.byref(p), WS, WS_BYTES, None) == EUNSUP
    p = ga.Plan(path=5, waves_per_row=1, per_lane=4, block=64, grid=1)
    assert L.ga_gelu_and_mul_sparse_with_plan(IN, OUT, 0, 64, BF16, Z, None, ctypes.byref(p), WS, WS_BYTES, None) == EINVAL
    # replicated statistics: REP 2, 4 or 8, up with the gate, no round-trip form, covering the row; no workspace
    rep = lambda d=64, **kw: L.ga_gelu_and_mul_sparse_with_plan(  # noqa: E731
        IN, OUT, 0, d, BF16, Z, None, ctypes.byref(ga.Plan(path=4, block=64 * kw.get("waves_per_row", 1), **kw)),
        None, 0, None)
    assert rep(waves_per_row=1, per_lane=1, splits=2) == OK and rep(waves_per_row=16, per_lane=8, splits=8, d=65536) == OK
    assert rep(waves_per_row=1, per_lane=1, splits=1) == EUNSUP and rep(waves_per_row=1, per_lane=1, splits=3) == EUNSUP
    assert rep(waves_per_row=1, per_lane=1, splits=16) == EUNSUP
    assert rep(waves_per_row=1, per_lane=1, splits=2, up_late=1) == EUNSUP
    assert rep(waves_per_row=1, per_lane=1, splits=2, flags=ga.GA_ROUND_INTERMEDIATES) == EUNSUP
    assert rep(waves_per_row=1, per_lane=1, splits=2, d=1024) == EUNSUP          # covers 64 < 128 vectors
    assert L.ga_gelu_and_mul_sparse_with_plan(ctypes.c_void_p(0x7F0000000002), OUT, 0, 64, BF16, Z, None,
                                              ctypes.byref(ga.Plan(path=4, waves_per_row=1, per_lane=1, splits=2)),
                                              None, 0, None) == EUNSUP       # 16-byte rows and bases only
    # packed rows: lanes_per_row in {4, 8, 16, 32}, 1, 2 or 4 vectors per lane, covering d
    rows = lambda g, v, d=256, **kw: L.ga_gelu_and_mul_sparse_with_plan(  # noqa: E731
        IN, OUT, 0, d, BF16, Z, None, ctypes.byref(ga.Plan(path=3, lanes_per_row=g, per_lane=v, **kw)),
        WS, WS_BYTES, None)
    assert rows(16, 2) == OK and rows(32, 1) == OK and rows(4, 4, d=128) == OK
    assert rows(16, 1) == EUNSUP                      # 16 x 1 x 8 < 256
    assert rows(64, 1) == EUNSUP and rows(8, 3) == EUNSUP
    assert rows(16, 2, up_late=1) == EUNSUP
    assert L.ga_gelu_and_mul_sparse_with_plan(ctypes.c_void_p(0x7F0000000002), OUT, 0, 256, BF16, Z, None,
                                              ctypes.byref(ga.Plan(path=3, lanes_per_row=16, per_lane=2)),
                                              WS, WS_BYTES, None) == OK       # any alignment
    assert rows(32, 1, d=257) == EUNSUP and rows(16, 4, d=257) == OK   # 257 elements: 33 vectors
    # lanes_per_row belongs to the packed-rows path; reserved must be zero
    assert L.ga_gelu_and_mul_sparse_with_plan(IN, OUT, 0, 2048, BF16, Z, None, ctypes.byref(
        ga.Plan(path=0, waves_per_row=4, per_lane=1, lanes_per_row=8)), WS, WS_BYTES, None) == EINVAL
    assert rows(16, 2, reserved=1) == EINVAL
    # unaligned path: must cover the row's 16-byte vectors, 1..8 per lane
    wp = lambda p, d: L.ga_gelu_and_mul_sparse_with_plan(  # noqa: E731
        IN, OUT, 0, d, BF16, Z, None, ctypes.byref(p), WS, WS_BYTES, None)
    assert wp(ga.Plan(path=2, waves_per_row=8, per_lane=4, block=512), 16384) == OK     # 2048 vectors
    assert wp(ga.Plan(path=2, waves_per_row=8, per_lane=4, block=512), 16385) == EUNSUP  # 2049 > 2048
    assert wp(ga.Plan(path=2, waves_per_row=8, per_lane=5, block=512), 16385) == OK
    assert wp(ga.Plan(path=2, waves_per_row=8, per_lane=9, block=512), 16384) == EUNSUP
    assert wp(ga.Plan(path=2, waves_per_row=3, per_lane=8, block=192), 64) == EUNSUP
    assert wp(ga.Plan(path=2, waves_per_row=8, per_lane=5, up_late=1, block=512), 16384) == OK
    assert wp(ga.Plan(path=2, waves_per_row=8, per_lane=5, up_late=2, block=512), 16384) == EUNSUP
    assert wp(ga.Plan(path=2, waves_per_row=1, per_lane=1, block=64), 1) == OK
    # vector path on a base that is not 16-byte aligned
    p = ga.plan_gelu_and_mul_sparse(1, 2048, BF16)
    assert p.path == 0
    st = L.ga_gelu_and_mul_sparse_with_plan(ctypes.c_void_p(0x7F0000000002), OUT, 0, 2048, BF16, Z, None,
                                            ctypes.byref(p), WS, WS_BYTES, None)
    assert st == EUNSUP


def test_round_trip_flag_checks():
    """The round-trip form: accepted on the plain and element paths, refused
    with split rows; unknown bits are malformed; silu plans take no flags."""
    RT = ga.GA_ROUND_INTERMEDIATES
    ex = lambda flags, T=0, d=2048, ws=None, nb=0: L.ga_gelu_and_mul_sparse_ex(  # noqa: E731
        IN, OUT, T, d, BF16, Z, None, flags, ws, nb, None)
    assert ex(0) == OK and ex(RT) == OK
    assert ex(2) == EINVAL and ex(RT | 4) == EINVAL and ex(-1) == EINVAL
    assert ex(RT, T=0, ws=WS, nb=WS_BYTES) == OK
    assert L.ga_gelu_and_mul_sparse_ex(None, OUT, 4, 64, BF16, Z, None, RT, None, 0, None) == EINVAL
    wp = lambda p, d=16384: L.ga_gelu_and_mul_sparse_with_plan(  # noqa: E731
        IN, OUT, 0, d, BF16, Z, None, ctypes.byref(p), WS, WS_BYTES, None)
    for d in (64, 2048, 16384, 65536, 777):
        p = ga.plan_gelu_and_mul_sparse(2048, d, BF16, aligned=d % 8 == 0)
        assert p.flags == 0
        p.flags = RT
        assert wp(p, d) == OK, (d, L.ga_last_error())
    split = ga.plan_gelu_and_mul_sparse(8, 16384, BF16)
    assert split.splits > 1
    split.flags = RT
    assert wp(split) == EUNSUP
    split.flags = 8
    assert wp(split) == EINVAL
    s = ga.plan_silu_and_mul_bounded(16384, 768, BF16)
    s.flags = RT
    assert L.ga_silu_and_mul_bounded_with_plan(IN, OUT, 0, 768, BF16, LIVE, ctypes.byref(s), None) == EINVAL


def test_silu_planner_depends_on_capacity_only():
    p = ga.plan_silu_and_mul_bounded(16384, 768, BF16, num_cus=256)
    assert p.path == 0 and p.block == 256 and 1 <= p.grid <= 256 * 16
    # The planner has no live-count input at all; the grid grows with M up to
    # sixteen workgroups per compute unit, then the kernel strides.
    small = ga.plan_silu_and_mul_bounded(4, 768, BF16, num_cus=256)
    assert small.grid == 2          # 4 rows x 96 vectors, 256 per workgroup
    big = ga.plan_silu_and_mul_bounded(1 << 20, 768, BF16, num_cus=256)
    assert big.grid == 256 * 32 and big.per_lane == 2     # > 4M items: 2 per lane, 32 per CU
    mid = ga.plan_silu_and_mul_bounded(16384, 1536, BF16, num_cus=256)
    assert mid.per_lane == 2 and mid.grid == 256 * 16     # 3.1M items
    assert ga.plan_silu_and_mul_bounded(100, 777, BF16).path == 2      # rows off 16 bytes: unaligned vectors
    assert ga.plan_silu_and_mul_bounded(100, 768, BF16, aligned=False).path == 2
    for M in (1, 7, 64, 1000, 16384):
        for d in (1, 8, 768, 777, 4096):
            p = ga.plan_silu_and_mul_bounded(M, d, BF16)
            st = L.ga_silu_and_mul_bounded_with_plan(IN, OUT, 0, d, BF16, LIVE, ctypes.byref(p), None)
            assert st == OK


def test_silu_with_plan_rejects_bad_geometry():
    p = ga.Plan(path=0, waves_per_row=0, per_lane=3, block=256, grid=4)
    assert L.ga_silu_and_mul_bounded_with_plan(IN, OUT, 0, 768, BF16, LIVE, ctypes.byref(p), None) == EUNSUP
    p = ga.Plan(path=0, waves_per_row=0, per_lane=2, block=256, grid=0)
    assert L.ga_silu_and_mul_bounded_with_plan(IN, OUT, 0, 768, BF16, LIVE, ctypes.byref(p), None) == EINVAL
    p = ga.Plan(path=0, waves_per_row=0, per_lane=4, block=256, grid=2 ** 22)
    assert L.ga_silu_and_mul_bounded_with_plan(IN, OUT, 0, 768, BF16, LIVE, ctypes.byref(p), None) == EUNSUP


def test_python_wrapper_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ga.gelu_and_mul_sparse(x)
    with pytest.raises(ValueError):
        ga.silu_and_mul_bounded(x, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(approx=2), EINVAL), (dict(approx=-1), EINVAL), (dict(in_=None), EINVAL),
    (dict(d=0), EINVAL), (dict(d=65537), EUNSUP), (dict(out=IN), EINVAL),
    (dict(T=0), OK), (dict(T=0, approx=0), OK),
])
def test_gelu_and_mul_argument_checks(kwargs, status):
    a = dict(in_=IN, out=OUT, T=4, d=768, dt=BF16, approx=1, live=None)
    a.update(kwargs)
    assert L.ga_gelu_and_mul(a["in_"], a["out"], a["T"], a["d"], a["dt"], a["approx"], a["live"], None) == status


@pytest.mark.parametrize("kwargs,status", [
    (dict(live=None), EINVAL), (dict(in_=None), EINVAL), (dict(M=-2), EINVAL),
    (dict(out=IN), EINVAL),
    # ungated layout: in is [M, d], so an output right after it does not overlap
    (dict(out=ctypes.c_void_p(0x7F0000000000 + 16 * 768 * 2), M=0), OK),
    (dict(M=0), OK),
])
def test_squared_relu_argument_checks(kwargs, status):
    a = dict(in_=IN, out=OUT, M=16, d=768, dt=BF16, live=LIVE)
    a.update(kwargs)
    assert L.ga_squared_relu_bounded(a["in_"], a["out"], a["M"], a["d"], a["dt"], a["live"], None) == status


def test_z_from_sparsity_against_scipy_and_closed_form():
    import math
    from scipy.stats import norm
    ps = [1e-12, 1e-6, 0.01, 0.05, 0.25, 0.5, 0.75, 0.9, 0.95, 0.99, 0.999, 1 - 1e-9]
    for p in ps:
        z = ga.z_from_sparsity(p)
        assert math.isclose(z, norm.ppf(p), rel_tol=1e-13, abs_tol=1e-15), p
        assert math.isclose(0.5 * math.erfc(-z / math.sqrt(2.0)), p, rel_tol=1e-12), p   # Phi(z) = p
        q = 1.0 - p                                   # Phi^-1(q) = -Phi^-1(1 - q)
        assert math.isclose(ga.z_from_sparsity(q), -ga.z_from_sparsity(1.0 - q), rel_tol=1e-13, abs_tol=1e-15)
    assert ga.z_from_sparsity(0.95) == pytest.approx(1.6448536269514722, rel=1e-15)
    for bad in (0.0, 1.0, -0.5, 2.0, float("nan")):
        assert math.isnan(ga.z_from_sparsity(bad))


# ---------------------------------------------------------------------------
# the activation fused with the down projection
# ---------------------------------------------------------------------------
W_ = ctypes.c_void_p(0x7F4000000000)
Y_ = ctypes.c_void_p(0x7F5000000000)


def down(gu=IN, w=W_, y=Y_, T=16, d=16384, H=2048, dt=BF16, z=Z, live=None, ws=WS, ws_bytes=WS_BYTES):
    return L.ga_gelu_and_mul_sparse_down(gu, w, y, T, d, H, dt, z, live, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(gu=None), EINVAL),
    (dict(w=None), EINVAL),
    (dict(y=None), EINVAL),
    (dict(T=-1), EINVAL),
    (dict(d=0), EINVAL),
    (dict(H=0), EINVAL),
    (dict(dt=7), EINVAL),
    (dict(dt=F32), EUNSUP),
    (dict(T=257), EUNSUP),
    (dict(d=2044), EUNSUP),                                   # not a multiple of 8
    (dict(d=65544), EUNSUP),
    (dict(H=2040), EUNSUP),                                   # not a multiple of 16
    (dict(H=65552), EUNSUP),
    (dict(gu=ctypes.c_void_p(0x7F0000000008)), EUNSUP),       # 16-byte alignment
    (dict(y=ctypes.c_void_p(0x7F5000000008)), EUNSUP),
    (dict(z=ctypes.c_float(float("nan"))), EINVAL),
    (dict(live=ctypes.c_void_p(0x7F2000000002)), EINVAL),
    (dict(y=IN), EINVAL),                                     # y over gu
    (dict(y=ctypes.c_void_p(0x7F4000000000 + 2048 * 16384 * 2 - 16)), EINVAL),   # y over w's tail
    (dict(ws=None), EINVAL),
    (dict(ws=ctypes.c_void_p(0x7F3000000010)), EINVAL),       # workspace not 256-byte aligned
    (dict(ws_bytes=4096), EINVAL),
    (dict(d=512, H=16, ws=None), EINVAL),                     # one slice still needs the stored activation
    (dict(T=0), OK),
    (dict(T=0, ws=None, ws_bytes=0), OK),
])
def test_down_argument_checks(kwargs, status):
    assert down(**kwargs) == status
    if status != OK:
        assert len(L.ga_last_error()) > 0


def _down_plan(T, d, H, dt=BF16):
    p = ga.DownPlan()
    assert L.ga_plan_gelu_and_mul_sparse_down(T, d, H, dt, ctypes.byref(p)) == OK
    return p


# Workspace layout of the staged and tiled forms: 256 bytes, the tiled form's
# output-tile counters (16384 words, a fixed region), the stored activation,
# then the tiled form's fp32 partial tiles.
ACT_OFFSET = 256 + 16384 * 4


def test_down_planner_and_workspace():
    # the measured choice by token count (d = 16384, H = 2048)
    assert ctypes.sizeof(ga.DownPlan) == 40 and ga.DownPlan.grid.offset == 32     # the C layout
    assert ga.DownPlan.depth.offset == 28                                           # in the padding before grid
    # one token: the decode form (one launch, no workspace); two: the staged
    # form (the activation stored into the workspace, then the product)
    for T, form, tmax, f, waves in ((1, ga.GA_DOWN_DECODE, 1, 4, 8), (2, ga.GA_DOWN_STAGED, 2, 4, 16)):
        p = _down_plan(T, 16384, 2048)
        assert (p.form, p.rows_per_block, p.features_per_block, p.waves, p.k_step, p.k_chunk, p.splits,
                p.depth, p.grid) == (form, tmax, f, waves, 0, 16384, 1, 0, 2048 // f), T
        want_ws = 0 if form == ga.GA_DOWN_DECODE else ACT_OFFSET + -(-T * 16384 * 2 // 256) * 256
        assert ga.gelu_and_mul_sparse_down_workspace_bytes(T, 16384, 2048) == want_ws
    p = _down_plan(1, 32768, 2048)
    assert (p.form, p.features_per_block, p.waves, p.grid) == (ga.GA_DOWN_DECODE, 4, 16, 512)
    for T, d in ((1, 32776), (2, 16392)):        # rows past the decode and staged forms' reach
        p = _down_plan(T, d, 2048)
        assert p.form == ga.GA_DOWN_TILED and p.k_step > 0, (T, d)
    # three tokens on: the measured table's plan (tests/planner_rule.py
    # states the lookup independently), or the staged form at three or four
    # tokens where the table found it faster and its row fits
    import planner_rule
    table = planner_rule.read_down_inc(os.path.join(os.path.dirname(ga.library_path), "csrc",
                                                    "planner_table_down.inc"))
    assert len(table) >= 91
    checked = staged = 0
    for T in (3, 4, 5, 9, 16, 17, 20, 31, 32, 33, 40, 64, 100, 128, 129, 150, 180, 200, 256):
        for d in (8, 1000, 4096, 6144, 8192, 8200, 12288, 16384, 24576, 32768, 65536):
            for H in (16, 1024, 2048, 3072, 4096, 8192, 65536):
                p = _down_plan(T, d, H)
                want = planner_rule.choose_down(table, T, d, H)
                if want == ("staged",) and d <= 16384:
                    assert (p.form, p.rows_per_block) == (ga.GA_DOWN_STAGED, 4), (T, d, H)
                    staged += 1
                    continue
                if want == ("staged",):                  # past the staged kernel's reach: the tiled plan
                    want = planner_rule.choose_down([e[:3] + (0,) + e[4:] for e in table], T, d, H)
                assert p.form == ga.GA_DOWN_TILED, (T, d, H)
                got = (p.rows_per_block, p.features_per_block, p.waves, p.k_step, p.depth, p.k_chunk)
                assert got == want, (T, d, H, got, want)
                assert p.grid == -(-T // p.rows_per_block) * -(-H // p.features_per_block) * p.splits
                checked += 1
    assert checked > 1000 and staged > 10
    # whole steps, at most 64 slices of d, for every d the kernels take
    for d in (8, 1024, 1032, 32768, 32776, 65536):
        for T in (1, 3, 20, 50, 200):
            for H in (16, 64, 2048, 65536):
                p = _down_plan(T, d, H)
                assert 1 <= p.splits <= 64 and p.splits == -(-d // p.k_chunk), (T, d, H)
                assert p.k_step == 0 or p.k_chunk % p.k_step == 0
                if p.form == ga.GA_DOWN_TILED and p.splits > 1:
                    assert p.grid // p.splits <= 16384, (T, d, H)        # output tiles with a counter
    assert ga.gelu_and_mul_sparse_down_workspace_bytes(1, 512, 16) == 0        # the decode form
    assert ga.gelu_and_mul_sparse_down_workspace_bytes(2, 520, 16) == ACT_OFFSET + 2 * 520 * 2 // 256 * 256 + 256
    # the tiled layout: counters, activation, partial tiles of every slice
    for T, d, H in ((5, 16384, 2048), (200, 3072, 64), (16, 512, 16)):
        p = _down_plan(T, d, H)
        tiles = -(-T // p.rows_per_block) * -(-H // p.features_per_block)
        part = tiles * p.splits * p.rows_per_block * p.features_per_block * 4 if p.splits > 1 else 0
        assert ga.gelu_and_mul_sparse_down_workspace_bytes(T, d, H) == \
            ACT_OFFSET + -(-T * d * 2 // 256) * 256 + part, (T, d, H)
    assert L.ga_plan_gelu_and_mul_sparse_down(300, 1024, 64, BF16, ctypes.byref(ga.DownPlan())) == EUNSUP
    assert L.ga_plan_gelu_and_mul_sparse_down(4, 1024, 64, F32, ctypes.byref(ga.DownPlan())) == EUNSUP
    assert L.ga_plan_gelu_and_mul_sparse_down(4, 1024, 64, BF16, None) == EINVAL


def test_down_with_plan_rejects_bad_geometry():
    T, d, H = 16, 4096, 512

    def run(**kw):
        p = _down_plan(T, d, H)
        for k, v in kw.items():
            setattr(p, k, v)
        return L.ga_gelu_and_mul_sparse_down_with_plan(IN, W_, Y_, T, d, H, BF16, Z, None, ctypes.byref(p),
                                                       WS, WS_BYTES, None)
    assert run(waves=3) == EINVAL                     # no kernel
    assert run(rows_per_block=8) == EINVAL
    assert run(features_per_block=48) == EINVAL
    assert run(k_step=384) == EINVAL
    assert run(depth=0) == EINVAL
    assert run(depth=4) == EINVAL
    assert run(k_chunk=1000) == EINVAL                # not a multiple of the step
    assert run(k_chunk=0) == EINVAL
    assert run(splits=3) == EINVAL                    # not ceil(d / k_chunk)
    assert run(grid=7) == EINVAL
    assert run(form=0) == EINVAL                      # no such form
    p = ga.DownPlan.tiled(16, 65536, 512, 16, 64, 4, 128, 512, 1)       # 128 slices
    assert L.ga_gelu_and_mul_sparse_down_with_plan(IN, W_, Y_, 16, 65536, 512, BF16, Z, None, ctypes.byref(p),
                                                   WS, WS_BYTES, None) == EUNSUP
    # the planner's widest launch keeps every output tile within the counters
    p = _down_plan(256, 1024, 65536)
    assert p.grid // p.splits <= 16384
    assert L.ga_gelu_and_mul_sparse_down_with_plan(IN, W_, Y_, T, d, H, BF16, Z, None, None, WS, WS_BYTES,
                                                   None) == EINVAL
    # the workspace: the tiled form's need, 256-byte aligned, not over gu, w or y
    need = ga.gelu_and_mul_sparse_down_workspace_bytes(T, d, H)
    p = _down_plan(T, d, H)
    assert L.ga_gelu_and_mul_sparse_down_with_plan(IN, W_, Y_, T, d, H, BF16, Z, None, ctypes.byref(p), WS, need - 1,
                                                   None) == EINVAL
    assert L.ga_gelu_and_mul_sparse_down_with_plan(IN, W_, Y_, T, d, H, BF16, Z, None, ctypes.byref(p), None, 0,
                                                   None) == EINVAL
    # decode plans
    def run_dec(T=2, d=4096, H=512, **kw):
        p = ga.DownPlan.decode(T, d, H, 2, 4, 8)
        for k, v in kw.items():
            setattr(p, k, v)
        return L.ga_gelu_and_mul_sparse_down_with_plan(IN, W_, Y_, T, d, H, BF16, Z, None, ctypes.byref(p),
                                                       None, 0, None)
    assert run_dec(T=3) == EINVAL                     # more tokens than the plan holds
    assert run_dec(d=32768) == EINVAL                 # row past the kernel's reach
    assert run_dec(rows_per_block=4) == EINVAL        # no such kernel
    assert run_dec(features_per_block=16) == EINVAL
    assert run_dec(features_per_block=8, grid=64) == EINVAL   # no 8-feature, 8-wave kernel for two tokens
    assert run_dec(waves=4) == EINVAL
    assert run_dec(form=7) == EINVAL                  # unknown form
    assert run_dec(k_step=128) == EINVAL
    # staged plans (two or four tokens, a workspace for the activation)
    ws_need = 4 * 4096 * 2

    def run_st(T=4, d=4096, H=512, ws=WS, ws_bytes=None, y=Y_, **kw):
        p = ga.DownPlan.staged(T, d, H, 4, 4, 16)
        for k, v in kw.items():
            setattr(p, k, v)
        return L.ga_gelu_and_mul_sparse_down_with_plan(IN, W_, y, T, d, H, BF16, Z, None, ctypes.byref(p),
                                                       ws, WS_BYTES if ws_bytes is None else ws_bytes, None)
    assert run_st(T=0) == OK
    assert run_st(T=5) == EINVAL                      # more tokens than the plan holds
    assert run_st(d=16392) == EINVAL                  # row past the kernel's reach
    assert run_st(waves=8) == EINVAL                  # no such kernel
    assert run_st(rows_per_block=8, T=0) == EINVAL
    assert run_st(grid=64) == EINVAL
    assert run_st(T=2, ws=None) == EINVAL             # the activation needs a workspace
    assert run_st(T=4, ws_bytes=ws_need - 256) == EINVAL
    assert run_st(T=4, ws=Y_) == EINVAL               # the workspace overlaps y
    assert run_st(T=4, ws=ctypes.c_void_p(IN.value + 256)) == EINVAL     # ... or gu
    assert run_dec(k_chunk=2048) == EINVAL
    assert run_dec(grid=3) == EINVAL
    assert run_dec(T=0) == OK                         # nothing to do
