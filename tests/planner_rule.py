"""The planner's measured tables: an independent statement of the rule that
reads them, and the writer that turns geometry sweeps into them.

    python tests/planner_rule.py [--prefix kUna | --split] OUT.inc SWEEP.csv [SWEEP.csv ...]
    python tests/planner_rule.py --check [--prefix kUna | --split] TABLE.inc OFFGRID.csv
    python tests/planner_rule.py --packed PACKED.csv [PACKED.csv ...]
    python tests/planner_rule.py --summarize OUT.csv SWEEP.csv [SWEEP.csv ...]

A sweep line is "T,d,nvec,waves,vectors per lane,up_late,us[,splits | lanes
per row]": one MI355X's time per call of gelu_and_mul_sparse on T bf16 rows of
nvec 16-byte vectors with that geometry, forced through the library's
ga_gelu_and_mul_sparse_with_plan entry point (each geometry's best of 3
interleaved passes of back-to-back launches over buffer sets past 1 GiB).
The sweeps behind the committed tables are summarised under profiles/ as
planner_sweep_*.csv (--summarize: the runs averaged, one line per geometry
and shape), which the table writer reads like the raw sweeps, so
        python tests/planner_rule.py gated_activation_amd/csrc/planner_table.inc \
            profiles/planner_sweep_vector_bf16.csv
regenerates a table.

--packed checks the short-row planner (a rule, no table) against sweeps of
the packed-rows path: for every shape, the library's own choice (from
ga_plan_gelu_and_mul_sparse, host-only) against the fastest measured plan.

--down writes the fused down projection's table (csrc/planner_table_down.inc)
from a sweep of ga_gelu_and_mul_sparse_down_with_plan over (d, H, T): lines
"d,H,T,kind,form,tokens,features,waves,k_step,depth,splits,us" with kind
tiled, staged or unfused (the activation then a hipBLASLt GEMM, for
reference).  For every (d, H, T) point it keeps the fastest tiled plan as its
geometry and its workgroup count, and whether the staged form was faster
still.  choose_down() is the lookup the planner applies
(csrc/api.hip, pick_down_tiled): the measured token count nearest to T in
log2 (T^2 against the product of the two neighbours, in integers), then, among
that token count's points, the (d, H) nearest in log2 distance (the first in
table order on a tie); the geometry is that point's and the slices of d are
as many as bring the launch to its workgroup count, rounded, 1 to 64 and at
most ceil(d / k_step).

The prefix names the table's symbols: kPlan (default) for the vector path,
kUna for the unaligned path (its kernel also takes 3, 5, 6 or 7 vectors per
lane, but the table, and so the planner, keeps to 1, 2, 4, 8).

The table holds, for every (rows T, 16-byte vectors per row nvec) point of the
sweep's grid and every compiled geometry of the vector kernel (waves 1..16,
vectors per lane 1, 2, 4, 8, up early or late), that geometry's time over the
best geometry's time at that point (times averaged over the given sweeps),
as loss = round((ratio - 1) * 400), capped at 254; 255 marks a geometry the
sweep did not run there (it does not cover the row, or leaves more than 7/8
of its lanes idle).

choose() is the rule the planner applies to the table (csrc/api.hip,
pick_row_geometry): interpolate each geometry's loss over the four grid points
around (T, nvec), with weights linear in log2 T and log2 nvec, and take the
geometry that covers nvec with the least 0.5 * (weighted mean) + 0.5 *
(largest) loss over the points where it was measured (at least half of the
weight); ties go to the first geometry in table order.  It is written here
independently of the C code so that a test can compare the two.
"""
import collections
import math
import os
import re
import sys

WAVES = (1, 2, 4, 8, 16)
PER_LANE = (1, 2, 4, 8)
GEOS = [(w, v, late) for w in WAVES for v in PER_LANE for late in (0, 1)]
NOT_RUN = 255
# Split table (--split, sweeps run with GA_SWEEP_PATH=split): chunk geometries
# (waves, vectors per lane) of the split kernel, then the row path (no split)
# as the last candidate; a row takes ceil(nvec / chunk) splits, 2..16.
SPLIT_CHUNKS = [(w, v) for w in WAVES for v in (1, 2, 4)]
ROW = len(SPLIT_CHUNKS)


def read_sweeps(paths):
    acc = collections.defaultdict(list)
    for path in paths:
        for line in open(path):
            if not line[:1].isdigit():
                continue
            T, d, nvec, w, v, late, us = line.strip().split(",")[:7]
            acc[(int(T), int(nvec), (int(w), int(v), int(late)))].append(float(us))
    times = collections.defaultdict(dict)
    for (T, nvec, geo), ts in acc.items():
        times[(T, nvec)][geo] = sum(ts) / len(ts)
    return times


def read_split_sweeps(paths):
    """(T, nvec) -> {candidate index: mean time}: chunk candidates from the
    split plans, ROW from the fastest one-row-per-workgroup plan."""
    acc = collections.defaultdict(list)
    for path in paths:
        for line in open(path):
            if not line[:1].isdigit():
                continue
            f = line.strip().split(",")
            T, nvec, w, v, us, splits = int(f[0]), int(f[2]), int(f[3]), int(f[4]), float(f[6]), int(f[7])
            key = ROW if splits == 1 else SPLIT_CHUNKS.index((w, v))
            acc[(T, nvec, key, w, v, int(f[5]))].append(us)
    times = collections.defaultdict(dict)
    for (T, nvec, key, w, v, late), ts in acc.items():
        t = sum(ts) / len(ts)
        if key not in times[(T, nvec)] or t < times[(T, nvec)][key]:
            times[(T, nvec)][key] = t
    return times


def build_split(times):
    Ts = sorted({k[0] for k in times})
    Ns = sorted({k[1] for k in times})
    loss = {}
    for T in Ts:
        for n in Ns:
            g = times.get((T, n), {})
            row = [NOT_RUN] * (ROW + 1)
            if g:
                best = min(g.values())
                for c, t in g.items():
                    row[c] = min(254, int(round((t / best - 1.0) * 400.0)))
            loss[(T, n)] = row
    return Ts, Ns, loss


def split_valid(c, nvec):
    if c == ROW:
        return True
    w, v = SPLIT_CHUNKS[c]
    splits = -(-nvec // (w * 64 * v))
    return 2 <= splits <= 16


def choose_split(table, T, nvec):
    """None (do not split) or (waves, vectors per lane, splits)."""
    sc = scores(table, T, nvec, [c for c in range(ROW + 1) if split_valid(c, nvec)])
    best = None
    for c, x in enumerate(sc):
        if x is not None and (best is None or x < sc[best]):
            best = c
    if best is None or best == ROW:
        return None
    w, v = SPLIT_CHUNKS[best]
    return (w, v, -(-nvec // (w * 64 * v)))


# Replicated-statistics table (--rep, sweeps run in the few-rows mode: every
# row geometry, every split plan and every replicated plan of a shape):
# candidates c < 60 are replicated geometries, c = (waves index * 4 +
# vectors-per-lane index) * 3 + (log2 REP - 1) with REP 2, 4, 8; c = 60 is the
# fastest row geometry (no split), c = 61 the fastest split plan.
REP_FACTORS = (2, 4, 8)
REP_GEOS = [(w, v, r) for w in WAVES for v in PER_LANE for r in REP_FACTORS]
REP_ROW, REP_SPLIT = len(REP_GEOS), len(REP_GEOS) + 1


def read_fewrows_sweeps(paths):
    """(T, nvec) -> {candidate: time}; each plan's runs averaged first, then
    the row and split plans reduced to their fastest."""
    acc = collections.defaultdict(list)
    for path in paths:
        for line in open(path):
            if not line[:1].isdigit():
                continue
            f = line.strip().split(",")
            T, nvec, w, v, late, us, splits, kind = (int(f[0]), int(f[2]), int(f[3]), int(f[4]), int(f[5]),
                                                     float(f[6]), int(f[7]), int(f[8]))
            acc[(T, nvec, kind, w, v, late, splits)].append(us)
    times = collections.defaultdict(dict)
    for (T, nvec, kind, w, v, late, splits), ts in acc.items():
        t = sum(ts) / len(ts)
        if kind == 4:
            key = REP_GEOS.index((w, v, splits))
        else:
            key = REP_ROW if splits == 1 else REP_SPLIT
        if key not in times[(T, nvec)] or t < times[(T, nvec)][key]:
            times[(T, nvec)][key] = t
    return times


def build_rep(times):
    Ts = sorted({k[0] for k in times})
    Ns = sorted({k[1] for k in times})
    loss = {}
    for T in Ts:
        for n in Ns:
            g = times.get((T, n), {})
            row = [NOT_RUN] * (REP_SPLIT + 1)
            if g:
                best = min(g.values())
                for c, t in g.items():
                    row[c] = min(254, int(round((t / best - 1.0) * 400.0)))
            loss[(T, n)] = row
    return Ts, Ns, loss


def rep_valid(c, nvec, with_workspace=True):
    if c == REP_ROW:
        return True
    if c == REP_SPLIT:
        return with_workspace
    w, v, r = REP_GEOS[c]
    return w * 64 * v >= nvec


def choose_rep(table, T, nvec, with_workspace=True):
    """None (not a replicated plan) or (waves, vectors per lane, REP); outside
    the table's grid, None."""
    Ts, Ns = table[0], table[1]
    if T < 1 or T > Ts[-1] or nvec < Ns[0] or nvec > Ns[-1]:
        return None
    sc = scores(table, T, nvec, [c for c in range(REP_SPLIT + 1) if rep_valid(c, nvec, with_workspace)])
    best = None
    for c, x in enumerate(sc):
        if x is not None and (best is None or x < sc[best]):
            best = c
    if best is None or best >= REP_ROW:
        return None
    return REP_GEOS[best]


def build(times):
    Ts = sorted({k[0] for k in times})
    Ns = sorted({k[1] for k in times})
    loss = {}
    for T in Ts:
        for n in Ns:
            g = times.get((T, n))
            row = [NOT_RUN] * len(GEOS)
            if g:
                best = min(g.values())
                for i, geo in enumerate(GEOS):
                    if geo in g:
                        row[i] = min(254, int(round((g[geo] / best - 1.0) * 400.0)))
            loss[(T, n)] = row
    return Ts, Ns, loss


def write_inc(path, Ts, Ns, loss, sources, prefix="kPlan"):
    P = prefix
    kind = {"kUna": "the unaligned path", "kSplit": "few-row shapes (the split path)",
            "kRep": "few-row shapes (row, split and replicated-statistics plans)"}.get(P, "the vector path")
    if P == "kRep":
        cand = ["// candidate c < 60: replicated-statistics geometries, c = (waves index * 4 + vectors-per-lane",
                "// index) * 3 + (log2 REP - 1), waves 1, 2, 4, 8, 16, vectors per lane 1, 2, 4, 8, REP 2, 4, 8;",
                "// c = 60: the fastest one-row-per-workgroup geometry; c = 61: the fastest split plan."]
        ng = REP_SPLIT + 1
    elif P == "kSplit":
        cand = ["// candidate c < 15: split-kernel chunks of waves 1, 2, 4, 8, 16 (index c / 3) times",
                "// vectors per lane 1, 2, 4 (index c % 3), ceil(nvec / chunk) splits; c = 15: no split",
                "// (the fastest one-row-per-workgroup geometry)."]
        ng = ROW + 1
    else:
        cand = ["// Geometry g = ((waves index * 4 + vectors-per-lane index) * 2 + up_late), waves",
                "// 1, 2, 4, 8, 16, vectors per lane 1, 2, 4, 8."]
        ng = len(GEOS)
    out = ["// Generated by tests/planner_rule.py from geometry sweeps of " + kind,
           "// (bf16 rows, one MI355X): " + ", ".join(sources) + ".",
           f"// {P}Loss[t][n][g]: time of candidate g over the best candidate's time at",
           f"// ({P}T[t] rows, {P}N[n] vectors per row), as round((ratio - 1) * 400),",
           "// capped at 254; 255 = not run there."] + cand + [
           f"constexpr int {P}NT = {len(Ts)};",
           f"constexpr int {P}NN = {len(Ns)};",
           f"constexpr int {P}NG = {ng};",
           f"constexpr int {P}T[{P}NT] = {{" + ", ".join(map(str, Ts)) + "};",
           f"constexpr int {P}N[{P}NN] = {{" + ", ".join(map(str, Ns)) + "};",
           f"constexpr unsigned char {P}Loss[{P}NT][{P}NN][{P}NG] = {{"]
    for T in Ts:
        out.append("    {")
        for n in Ns:
            out.append("        {" + ",".join(map(str, loss[(T, n)])) + "},  // T=%d nvec=%d" % (T, n))
        out.append("    },")
    out.append("};")
    open(path, "w").write("\n".join(out) + "\n")


def read_inc(path, prefix="kPlan"):
    text = open(path).read()
    P = prefix
    Ts = [int(x) for x in re.search(P + r"T\[" + P + r"NT\] = \{([^}]*)\}", text).group(1).split(",")]
    Ns = [int(x) for x in re.search(P + r"N\[" + P + r"NN\] = \{([^}]*)\}", text).group(1).split(",")]
    rows = re.findall(r"^\s*\{([0-9,]+)\},\s*// T=(\d+) nvec=(\d+)", text, flags=re.M)
    loss = {(int(T), int(n)): [int(x) for x in r.split(",")] for r, T, n in rows}
    return Ts, Ns, loss


def _bracket(grid, x):
    if x <= grid[0]:
        return grid[0], grid[0], 1.0
    if x >= grid[-1]:
        return grid[-1], grid[-1], 1.0
    for lo, hi in zip(grid, grid[1:]):
        if lo <= x <= hi:
            return lo, hi, (math.log2(hi) - math.log2(x)) / (math.log2(hi) - math.log2(lo))
    raise AssertionError


def scores(table, T, nvec, valid=None):
    """Score of every candidate (None where not valid or not enough data).
    valid: candidate indices to score; default: the geometries covering nvec."""
    Ts, Ns, loss = table
    t0, t1, wt = _bracket(Ts, T)
    n0, n1, wn = _bracket(Ns, nvec)
    pts = [((t0, n0), wt * wn), ((t0, n1), wt * (1 - wn)), ((t1, n0), (1 - wt) * wn), ((t1, n1), (1 - wt) * (1 - wn))]
    if valid is None:
        valid = [i for i, (w, v, late) in enumerate(GEOS) if w * 64 * v >= nvec]
    out = []
    for i in range(len(next(iter(loss.values())))):
        if i not in valid:
            out.append(None)
            continue
        s = ws = mx = 0.0
        for p, wgt in pts:
            if wgt <= 0.0:
                continue
            l = loss[p][i]
            if l == NOT_RUN:
                continue
            s += wgt * l
            ws += wgt
            mx = max(mx, l)
        out.append(0.5 * s / ws + 0.5 * mx if ws >= 0.5 else None)
    return out


def choose(table, T, nvec):
    sc = scores(table, T, nvec)
    best = None
    for i, s in enumerate(sc):
        if s is not None and (best is None or s < sc[best]):
            best = i
    return None if best is None else GEOS[best]


def read_packed_sweeps(paths):
    """(T, nvec) -> {plan name: mean time}; packed plans are ('packed', lanes
    per row, vectors per lane), the row plan ('row', up_late)."""
    acc = collections.defaultdict(list)
    for path in paths:
        for line in open(path):
            if not line[:1].isdigit():
                continue
            f = line.strip().split(",")
            T, nvec, v, late, us, g = int(f[0]), int(f[2]), int(f[4]), int(f[5]), float(f[6]), int(f[7])
            acc[(T, nvec, ("packed", g, v) if g else ("row", late))].append(us)
    times = collections.defaultdict(dict)
    for (T, nvec, key), ts in acc.items():
        times[(T, nvec)][key] = sum(ts) / len(ts)
    return times


def plan_name(key):
    return "G%d V%d" % key[1:] if key[0] == "packed" else "row W1 V1%s" % (" late" if key[1] else "")


def check_packed(paths):
    # The repository root (this file is tests/planner_rule.py).
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import gated_activation_amd as ga
    times = read_packed_sweeps(paths)
    ratios = []
    for (T, n), g in sorted(times.items()):
        p = ga.plan_gelu_and_mul_sparse(T, 8 * n, ga.GA_BF16, aligned=True, with_workspace=False)
        key = ("packed", p.lanes_per_row, p.per_lane)
        best = min(g, key=g.get)
        r = g[key] / g[best] if key in g else float("nan")
        ratios.append(r)
        print(f"T={T:7d} nvec={n:3d} planner {plan_name(key):9s} {g.get(key, float('nan')):7.2f} us: {r:.3f} of the"
              f" best ({plan_name(best)}, {g[best]:.2f} us)")
    ok = sorted(x for x in ratios if x == x)
    print(f"{len(ok)} shapes: median {ok[len(ok) // 2]:.4f}, mean {sum(ok) / len(ok):.4f}, "
          f"90th percentile {ok[int(0.9 * len(ok))]:.4f}, worst {ok[-1]:.4f}, "
          f"> 3 % slower: {sum(x > 1.03 for x in ok)}, not measured: {len(ratios) - len(ok)}")
    return 0


def summarize(out, paths):
    """Average the runs of the given sweeps per (T, d, nvec, geometry[, extra
    column]) and write one line each, in the sweeps' own line format."""
    acc = collections.defaultdict(list)
    for path in paths:
        for line in open(path):
            if not line[:1].isdigit():
                continue
            f = line.strip().split(",")
            acc[tuple(f[:6]) + tuple(f[7:])].append(float(f[6]))
    lines = []
    for key in sorted(acc, key=lambda k: tuple(int(x) for x in k)):
        us = sum(acc[key]) / len(acc[key])
        lines.append(",".join(list(key[:6]) + [repr(us)] + list(key[6:])))
    head = ["# Geometry sweep summary (tests/planner_rule.py --summarize): " + ", ".join(
        os.path.basename(p) for p in paths) + " averaged.",
        "# T,d,nvec,waves,vectors per lane,up_late,us per call[,splits | lanes per row]"]
    open(out, "w").write("\n".join(head + lines) + "\n")
    return len(lines)


DOWN_MAX_SPLITS = 64


def read_down_sweep(paths):
    """{(d, H, T): {key: us}}, key ("staged",), ("unfused",) or
    (tokens, features, waves, k_step, depth, splits) of a tiled plan."""
    times = collections.defaultdict(dict)
    for path in paths:
        for line in open(path):
            if not line.strip() or line.startswith("#"):
                continue
            f = line.strip().split(",")
            d, H, T = int(f[0]), int(f[1]), int(f[2])
            us = float(f[11])
            if f[3] == "tiled":
                key = tuple(int(v) for v in f[5:11])
            elif f[3] in ("staged", "unfused"):
                key = (f[3],)
            else:
                continue
            times[(d, H, T)][key] = min(us, times[(d, H, T)].get(key, float("inf")))
    return times


def build_down(times):
    """Entries (d, H, T, staged, tokens, features, waves, k_step, depth,
    grid) sorted by (T, d, H): each point's fastest tiled plan, its
    workgroup count, and whether the staged form beat it."""
    entries = []
    for (d, H, T), g in times.items():
        tiled = {k: v for k, v in g.items() if len(k) == 6}
        (tm, bh, w, ks, pd, sp), us = min(tiled.items(), key=lambda kv: (kv[1], kv[0]))
        staged = int(g.get(("staged",), float("inf")) < us)
        grid = -(-T // tm) * -(-H // bh) * sp
        entries.append((d, H, T, staged, tm, bh, w, ks, pd, grid))
    return sorted(entries, key=lambda e: (e[2], e[0], e[1]))


def write_down_inc(path, entries, sources):
    out = ["// Generated by tests/planner_rule.py --down from a sweep of the fused down projection",
           "// (gelu_and_mul_sparse then y = a . w^T, bf16, one MI355X): " + ", ".join(sources) + ".",
           "// For each measured (d, H, T): the fastest tiled plan's geometry (tokens, features,",
           "// waves, k step, steps of loads in flight) and workgroups, and whether the staged form",
           "// was faster still.  Sorted by T, then d, then H.",
           "struct DownTableEntry {",
           "    int d, H, T, staged, tm, bh, waves, kstep, depth, grid;",
           "};",
           f"constexpr int kDownTableN = {len(entries)};",
           "constexpr DownTableEntry kDownTable[kDownTableN] = {"]
    for e in entries:
        out.append("    {" + ", ".join(map(str, e)) + "},")
    out.append("};")
    open(path, "w").write("\n".join(out) + "\n")


def read_down_inc(path):
    text = open(path).read()
    rows = re.findall(r"^\s*\{([0-9, ]+)\},\s*$", text, flags=re.M)
    return [tuple(int(x) for x in r.split(",")) for r in rows]


def choose_down(entries, T, d, H):
    """The table lookup for T >= 1 tokens: ("staged",) or the tiled plan
    (tokens, features, waves, k_step, depth, k_chunk)."""
    Ts = sorted({e[2] for e in entries})
    if T <= Ts[0]:
        Tn = Ts[0]
    elif T >= Ts[-1]:
        Tn = Ts[-1]
    else:
        hi = next(t for t in Ts if t >= T)
        lo = max(t for t in Ts if t <= T)
        Tn = lo if T * T < lo * hi else hi
    best = None
    for e in entries:
        if e[2] != Tn:
            continue
        dist = (math.log2(d / e[0])) ** 2 + (math.log2(H / e[1])) ** 2
        if best is None or dist < best[0]:
            best = (dist, e)
    _, (_, _, _, staged, tm, bh, w, ks, pd, grid) = best
    if staged and T <= 4:
        return ("staged",)
    tiles = -(-T // tm) * -(-H // bh)
    slices = (grid + tiles // 2) // tiles
    slices = min(max(slices, 1), DOWN_MAX_SPLITS, -(-d // ks))
    kc = -(-(-(-d // slices)) // ks) * ks
    return (tm, bh, w, ks, pd, kc)


def main(argv):
    argv = list(argv)
    if "--down" in argv:
        argv.remove("--down")
        out, sources = argv[1], argv[2:]
        entries = build_down(read_down_sweep(sources))
        write_down_inc(out, entries, [p.split("/")[-1] for p in sources])
        print(f"{out}: {len(entries)} points")
        return 0
    if "--summarize" in argv:
        argv.remove("--summarize")
        print(f"{argv[1]}: {summarize(argv[1], argv[2:])} lines")
        return 0
    if "--packed" in argv:
        argv.remove("--packed")
        return check_packed(argv[1:])
    check = "--check" in argv
    if check:
        argv.remove("--check")
    prefix = "kPlan"
    if "--prefix" in argv:
        i = argv.index("--prefix")
        prefix = argv[i + 1]
        del argv[i:i + 2]
    rep = "--rep" in argv
    if rep:
        argv.remove("--rep")
        prefix = "kRep"
        if check:
            table = read_inc(argv[1], prefix)
            times = read_fewrows_sweeps(argv[2:])
            ratios = []
            for (T, n), g in sorted(times.items()):
                c = choose_rep(table, T, n)
                key = REP_GEOS.index(c) if c is not None else None
                if key is None:
                    # not replicated: the row or split choice (the other tables'); rated by the better of the two
                    t = min(g.get(REP_ROW, float("inf")), g.get(REP_SPLIT, float("inf")))
                else:
                    t = g.get(key, float("nan"))
                ratios.append(t / min(g.values()))
                print(f"T={T:4d} nvec={n:5d} choice {'row/split' if c is None else 'W%d V%d REP%d' % c}:"
                      f" {ratios[-1]:.3f} of the best")
            ok = sorted(x for x in ratios if x == x)
            print(f"{len(ok)} shapes: median {ok[len(ok) // 2]:.4f}, mean {sum(ok) / len(ok):.4f}, "
                  f"90th percentile {ok[int(0.9 * len(ok))]:.4f}, worst {ok[-1]:.4f}, "
                  f"> 3 % slower: {sum(x > 1.03 for x in ok)}, not measured: {len(ratios) - len(ok)}")
            return 0
        out, sources = argv[1], argv[2:]
        Ts, Ns, loss = build_rep(read_fewrows_sweeps(sources))
        write_inc(out, Ts, Ns, loss, [p.split("/")[-1] for p in sources], prefix)
        print(f"{out}: {len(Ts)} row counts x {len(Ns)} row sizes x {REP_SPLIT + 1} candidates")
        return 0
    split = "--split" in argv
    if split:
        argv.remove("--split")
        prefix = "kSplit"
    if check and split:
        table = read_inc(argv[1], prefix)
        times = read_split_sweeps(argv[2:])
        ratios = []
        for (T, n), g in sorted(times.items()):
            c = choose_split(table, T, n)
            key = ROW if c is None else SPLIT_CHUNKS.index((c[0], c[1]))
            ratios.append(g[key] / min(g.values()) if key in g else float("nan"))
            print(f"T={T:4d} nvec={n:5d} choice {'no split' if c is None else 'S%d W%d V%d' % (c[2], c[0], c[1])}:"
                  f" {ratios[-1]:.3f} of the best")
        ok = sorted(x for x in ratios if x == x)
        print(f"{len(ok)} shapes: median {ok[len(ok) // 2]:.4f}, mean {sum(ok) / len(ok):.4f}, "
              f"90th percentile {ok[int(0.9 * len(ok))]:.4f}, worst {ok[-1]:.4f}, "
              f"> 3 % slower: {sum(x > 1.03 for x in ok)}, not measured: {len(ratios) - len(ok)}")
        return 0
    if split:
        out, sources = argv[1], argv[2:]
        Ts, Ns, loss = build_split(read_split_sweeps(sources))
        write_inc(out, Ts, Ns, loss, [p.split("/")[-1] for p in sources], prefix)
        print(f"{out}: {len(Ts)} row counts x {len(Ns)} row sizes x {ROW + 1} candidates")
        return 0
    if check:
        table = read_inc(argv[1], prefix)
        times = read_sweeps(argv[2:])
        ratios = []
        for (T, n), g in sorted(times.items()):
            c = choose(table, T, n)
            best = min(g.values())
            r = g[c] / best if c in g else float("nan")
            ratios.append(r)
            print(f"T={T:6d} nvec={n:5d} choice W{c[0]} V{c[1]}{' late' if c[2] else ''}: {r:.3f} of the best")
        ok = sorted(x for x in ratios if x == x)
        print(f"{len(ok)} shapes: median {ok[len(ok) // 2]:.4f}, mean {sum(ok) / len(ok):.4f}, "
              f"90th percentile {ok[int(0.9 * len(ok))]:.4f}, worst {ok[-1]:.4f}, "
              f"> 3 % slower: {sum(x > 1.03 for x in ok)}, not measured: {len(ratios) - len(ok)}")
        return 0
    out, sources = argv[1], argv[2:]
    Ts, Ns, loss = build(read_sweeps(sources))
    write_inc(out, Ts, Ns, loss, [p.split("/")[-1] for p in sources], prefix)
    print(f"{out}: {len(Ts)} row counts x {len(Ns)} row sizes x {len(GEOS)} geometries")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
