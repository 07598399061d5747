"""The planner's measured tables (tests/planner_rule.py): the table writer
turns sweep lines into a table whose interpolation rule picks the measured
best geometry at the grid points and respects coverage between them, and the
committed tables are exactly what the committed sweep summaries give."""
import os

import planner_rule as mt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_activation_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def _body(path):
    return [ln for ln in open(path) if not ln.startswith("//")]


def test_committed_tables_regenerate_from_the_sweep_summaries(tmp_path):
    for inc, summary, flags in (("planner_table.inc", "planner_sweep_vector_bf16.csv", []),
                                ("planner_table_una.inc", "planner_sweep_unaligned_bf16.csv", ["--prefix", "kUna"]),
                                ("planner_table_split.inc", "planner_sweep_split_bf16.csv", ["--split"]),
                                ("planner_table_rep.inc", "planner_sweep_fewrows_bf16.csv", ["--rep"])):
        out = tmp_path / inc
        assert mt.main(["planner_rule.py"] + flags + [str(out), os.path.join(PROFILES, summary)]) == 0
        assert _body(str(out)) == _body(os.path.join(CSRC, inc)), inc


def test_committed_down_table_regenerates_from_its_sweep(tmp_path):
    out = tmp_path / "planner_table_down.inc"
    assert mt.main(["planner_rule.py", "--down", str(out),
                    os.path.join(PROFILES, "planner_sweep_down_bf16.csv")]) == 0
    assert open(out).read() == open(os.path.join(CSRC, "planner_table_down.inc")).read()


def test_down_lookup_on_a_synthetic_table():
    # two measured shapes at two token counts; a query takes the nearest
    # token count (T^2 against the neighbours' product), then the nearest
    # (d, H) in log2, and that point's workgroups over its own tiles
    table = [(4096, 1024, 4, 1, 16, 64, 4, 128, 3, 256), (16384, 4096, 4, 0, 16, 64, 4, 128, 1, 512),
             (4096, 1024, 64, 0, 64, 64, 4, 128, 2, 256), (16384, 4096, 64, 0, 64, 128, 8, 64, 3, 256)]
    assert mt.choose_down(table, 3, 4096, 1024) == ("staged",)
    assert mt.choose_down(table, 4, 8000, 2000) == ("staged",)          # nearer (4096, 1024)
    assert mt.choose_down(table, 4, 9000, 2100)[0] == 16                  # nearer (16384, 4096): tiled
    assert mt.choose_down(table, 16, 4096, 1024)[0] == 64                 # 16^2 = 4 * 64: the tie goes up
    assert mt.choose_down(table, 17, 4096, 1024)[0] == 64                 # 17^2 > 4 * 64: nearest is 64
    # (16384, 4096) at T = 64: 1 x 32 tiles, 256 workgroups -> 8 slices of 2048
    assert mt.choose_down(table, 64, 16384, 4096) == (64, 128, 8, 64, 3, 2048)
    # a wider H at the same point: 1 x 64 tiles -> 4 slices of 4096
    assert mt.choose_down(table, 64, 16384, 8192) == (64, 128, 8, 64, 3, 4096)
    # (16384, 2048) is nearer (16384, 4096): 1 x 16 tiles -> 16 slices of 1024
    assert mt.choose_down(table, 64, 16384, 2048) == (64, 128, 8, 64, 3, 1024)
    # slices capped at 64, and at ceil(d / k_step): (16384, 256) and (128, 128)
    # are nearer (4096, 1024), 256 workgroups over 1 x 4 and 1 x 2 tiles
    assert mt.choose_down(table, 64, 16384, 256) == (64, 64, 4, 128, 2, 256)
    assert mt.choose_down(table, 64, 128, 128) == (64, 64, 4, 128, 2, 128)


def test_table_builder_round_trip(tmp_path):
    # A synthetic sweep on a 2 x 2 grid: at every point one geometry is
    # fastest; a second one is 10 % slower everywhere.
    lines = []
    fast = {(100, 128): (1, 2, 0), (100, 512): (8, 1, 1), (400, 128): (2, 1, 1), (400, 512): (4, 2, 0)}
    for (T, n), g in fast.items():
        for geo in mt.GEOS:
            w, v, late = geo
            if w * 64 * v < n or w * 64 * v >= 8 * n:
                continue
            us = 10.0 if geo == g else 11.0 + 0.01 * mt.GEOS.index(geo)
            lines.append(f"{T},{n * 8},{n},{w},{v},{late},{us}")
    csv = tmp_path / "s.csv"
    csv.write_text("\n".join(lines) + "\ndone\n")
    inc = tmp_path / "t.inc"
    mt.main(["planner_rule.py", str(inc), str(csv)])
    table = mt.read_inc(str(inc))
    assert table[0] == [100, 400] and table[1] == [128, 512]
    for (T, n), g in fast.items():
        assert mt.choose(table, T, n) == g
        i = mt.GEOS.index(g)
        assert table[2][(T, n)][i] == 0
    # between grid points every choice still covers the row
    for T in (50, 150, 250, 1000):
        for n in (100, 200, 300, 511):
            w, v, late = mt.choose(table, T, n)
            assert w * 64 * v >= n
    # a geometry not run at a point is marked, not guessed
    assert table[2][(100, 128)][mt.GEOS.index((16, 8, 0))] == mt.NOT_RUN


def test_split_table_builder_round_trip(tmp_path):
    # Two row sizes x two row counts: at three points a chunk geometry wins,
    # at one the row path (no split) does.
    win = {(1, 4096): (8, 1), (1, 8192): (8, 2), (64, 4096): (4, 2), (64, 8192): None}
    lines = []
    for (T, n), g in win.items():
        for w, v in mt.SPLIT_CHUNKS:
            splits = -(-n // (w * 64 * v))
            if 2 <= splits <= 16:
                us = 5.0 if g == (w, v) else 6.0
                lines.append(f"{T},{n * 8},{n},{w},{v},0,{us},{splits}")
        lines.append(f"{T},{n * 8},{n},16,4,1,{5.0 if g is None else 7.0},1")
        lines.append(f"{T},{n * 8},{n},8,8,0,{9.0},1")
    csv = tmp_path / "split.csv"
    csv.write_text("\n".join(lines) + "\ndone\n")
    inc = tmp_path / "split.inc"
    mt.main(["planner_rule.py", "--split", str(inc), str(csv)])
    table = mt.read_inc(str(inc), "kSplit")
    for (T, n), g in win.items():
        c = mt.choose_split(table, T, n)
        if g is None:
            assert c is None
        else:
            assert c == (g[0], g[1], -(-n // (g[0] * 64 * g[1])))


def test_packed_check_reads_sweeps_and_asks_the_library(tmp_path, capsys):
    """The short-row check parses packed-mode sweep lines (eighth column:
    lanes per row, 0 for the row geometry) and rates the library's own
    choice (G = 8 lanes, one vector, for a row of 6 vectors; G = 32 for 24)
    against the fastest line of each shape."""
    csv = tmp_path / "packed.csv"
    csv.write_text("\n".join([
        "4096,48,6,0,1,0,2.00,8",      # the planner's G8 V1: the fastest
        "4096,48,6,0,1,0,2.20,4",      # G4 V2 would not be offered (spare half) but parses
        "4096,48,6,1,1,0,2.50,0",      # row geometry, up early
        "4096,192,24,0,1,0,3.15,32",   # the planner's G32 V1
        "4096,192,24,0,2,0,3.00,16",   # G16 V2: 5 % faster
        "4096,192,24,1,1,1,3.30,0",    # row geometry, up late
        "done",
    ]) + "\n")
    times = mt.read_packed_sweeps([str(csv)])
    assert times[(4096, 6)][("packed", 8, 1)] == 2.0
    assert times[(4096, 24)][("row", 1)] == 3.3
    assert mt.main(["planner_rule.py", "--packed", str(csv)]) == 0
    out = capsys.readouterr().out
    assert "nvec=  6 planner G8 V1" in out and "1.000 of the best (G8 V1" in out
    assert "nvec= 24 planner G32 V1" in out and "1.050 of the best (G16 V2" in out
    assert "2 shapes:" in out and "worst 1.0500" in out


def test_rep_table_builder_round_trip(tmp_path):
    """Few-rows sweep lines (ninth column: the path, 4 for replicated plans)
    become a table whose rule picks the fastest replicated geometry, or none
    where a row or split plan is faster; without a workspace a split plan is
    not a candidate."""
    lines = []
    # (T, nvec): (fastest replicated geometry or None, time of the best row plan, of the best split plan)
    cases = {(1, 1024): ((8, 2, 8), 3.0, 3.5), (1, 4096): (None, 7.0, 6.5), (64, 1024): ((8, 2, 4), 3.5, 4.0),
             (64, 4096): (None, 5.0, 6.0)}
    for (T, n), (g, row_us, split_us) in cases.items():
        lines.append(f"{T},{n * 8},{n},16,4,1,{row_us},1,0")
        lines.append(f"{T},{n * 8},{n},8,8,0,{row_us + 1},1,0")
        lines.append(f"{T},{n * 8},{n},4,2,0,{split_us},{-(-n // 512)},0")
        for w, v, r in mt.REP_GEOS:
            if n <= w * 64 * v < 8 * n:
                us = 2.5 if (w, v, r) == g else max(row_us, split_us) + 0.5
                lines.append(f"{T},{n * 8},{n},{w},{v},0,{us},{r},4")
    csv = tmp_path / "fewrows.csv"
    csv.write_text("\n".join(lines) + "\ndone\n")
    inc = tmp_path / "rep.inc"
    assert mt.main(["planner_rule.py", "--rep", str(inc), str(csv)]) == 0
    table = mt.read_inc(str(inc), "kRep")
    for (T, n), (g, row_us, split_us) in cases.items():
        assert mt.choose_rep(table, T, n) == g, (T, n)
    # (1, 4096): the split plan wins with a workspace; without one the row plan is
    # still faster than every replicated geometry there
    assert mt.choose_rep(table, 1, 4096, with_workspace=False) is None
    assert table[2][(1, 1024)][mt.REP_ROW] > 0 and table[2][(1, 4096)][mt.REP_SPLIT] == 0
