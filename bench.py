"""Benchmark: achieved HBM bandwidth of gelu_and_mul_sparse, T=2048, d=16384, bf16.

One step is one gelu_and_mul_sparse call over the whole [2048, 32768] bf16
input (gate N(0,2) | up N(0,1), seed 2048016, z = Phi^-1(0.95)), inputs
already resident in HBM.  Algorithmic bytes per call: read 2d + write d
elements per row = 2048 * 3 * 16384 * 2 B = 201,326,592 B.  Input/output sets
rotate so the working set (>= 1 GiB) is several times the 256 MB Infinity
Cache.  The K timed steps are recorded into one HIP graph and replayed once
between HIP events on the stream they run on (the same steps launched one by
one from the host are reported beside it).

Also measured in the same run: a streaming kernel with the same access
pattern (the ceiling), silu_and_mul_bounded on the MoE decode buffer
(M = 16384, d = 768, live 16384, 2048 and 64; its own roofline object, and
the fp64 oracle's silu timed on the host beside it), the activation fused
with the down projection at decode token counts against the unfused pair
(its own roofline object and oracle timing), and the fp64 CPU oracle on a
bounded sample of the headline workload (the CPU baseline).

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints one JSON line.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s and % of peak, gelu_and_mul_sparse T=2048 d=16384 bf16"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, AMD published peak
T, D = 2048, 16384
Z = 1.6448536
ROTATE_BYTES = 1 << 30
SILU_M, SILU_D = 16384, 768
# Calls moving less than this finish in about the launch latency: % of peak is
# not meaningful for them.
LATENCY_BOUND_BYTES = 16 << 20
CSRC = os.path.join(ROOT, "gated_activation_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gelu_and_mul_sparse_T2048_d16384_bf16.traffic.txt")
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("gelu_sparse.hip", "ga_device.h")]
SILU_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "silu_and_mul_bounded_M16384_d768_bf16.traffic.txt")
SILU_SOURCES = [os.path.join(CSRC, f) for f in ("elementwise.hip", "ga_device.h")]
DOWN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gelu_and_mul_sparse_down_d16384_H2048_bf16.traffic.txt")
DOWN_SOURCES = [os.path.join(CSRC, f) for f in ("gelu_sparse_decode.hip", "ga_device.h")]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="approximate CPU time spent on the oracle baseline, half on one thread "
                        "and half over the host cores (0 = skip)")
    p.add_argument("--no-side", action="store_true", help="skip the ceiling, silu and sweep measurements")
    p.add_argument("--clock-warm-ms", type=float, default=300.0,
                   help="untimed headline launches for about this long before the warmup steps, so the "
                        "timed steps run at steady-state clocks (0 = none)")
    p.add_argument("--markers", action="store_true",
                   help="wrap each measured item in a roctx range (for a rocprofv3 --marker-trace run)")
    p.add_argument("--no-sweep", action="store_true", help="skip the sweep and the sibling ops")
    p.add_argument("--profile-cases", type=int, default=0, metavar="N",
                   help="instead of the benchmark: launch each of the counter cases N times (and the "
                        "same-pattern streaming kernel N times where it applies), printing one 'D <label>' "
                        "line per launch, for rocprofv3 counter runs joined by dispatch order")
    p.add_argument("--down-only", action="store_true",
                   help="instead of the benchmark: only the fused down-projection measurements")
    p.add_argument("--down-geometries", action="store_true",
                   help="instead of the benchmark: time every fused down-projection geometry at each "
                        "token count of the planner's sweep (CSV lines in the JSON)")
    p.add_argument("--down-calls", type=int, default=0, metavar="N",
                   help="instead of the benchmark: N fused down-projection calls at each --down-ts token count "
                        "(default 1) on rotating weights, untimed, one 'D <label>' line per call (for rocprofv3 "
                        "counter runs)")
    p.add_argument("--down-ts", default="", metavar="T1,T2,...",
                   help="token counts of the fused down-projection measurements (default 1,4,16,64,256)")
    p.add_argument("--down-shapes", default="", metavar="DxH,...",
                   help="with --down-only or --down-geometries: the (d, H) shapes to measure, one result per "
                        "shape (default: d = 16384, H = 2048 only)")
    return p.parse_args()


class Markers:
    """roctx ranges around the measured items, so a rocprofv3 kernel trace
    taken with --marker-trace can be split per item; no-ops unless enabled."""

    def __init__(self, enabled):
        self.lib = None
        if not enabled:
            return
        import ctypes
        path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "librocprofiler-sdk-roctx.so")
        self.lib = ctypes.CDLL(path)
        self.lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
        self.lib.roctxRangePushA.restype = ctypes.c_int
        self.lib.roctxRangePop.argtypes = []
        self.lib.roctxRangePop.restype = ctypes.c_int

    def push(self, label):
        if self.lib is not None:
            self.lib.roctxRangePushA(label.encode())

    def pop(self):
        if self.lib is not None:
            self.lib.roctxRangePop()


# The pages' own figures, quoted beside the measurement for context; none of
# them is a target (another machine, another workload).
CONTEXT = {
    "note": "figures printed on the source pages, for context only: not targets",
    "megatron_silu_and_mul_bounded_gb200": {
        "source": "Megatron-LM PR 6328, What changed and why / Measured gain / Where the time went",
        "bytes_per_layer_MB": 9.44,
        "us_per_layer_old_grid": 15.8,
        "us_per_launch_old_to_new": [17.158, 7.644],
        "bandwidth_floor_us_as_printed": 1.57,
        "bandwidth_floor_us_recomputed": 1.552,
        "measured_streaming_ceiling_TBps": 6.081,
        "peer_elementwise_kernels_us": [1.26, 2.60],
        "final_multiple_of_floor": 4.9,
        "here": "silu_and_mul_bounded at live=2048 (9.44 MB) below",
    },
    "vllm_gelu_and_mul_sparse": {
        "source": "vLLM PR 48498, Test Result (BF16 kernel performance)",
        "published": "speed-ups over the compiled native path only (A100 geomean 2.59x over 42 shapes, "
                     "B200 1.11-4.06x); no microseconds or GB/s",
    },
}


def kernel_source_digest(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in sources:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def recorded_traffic(path=TRAFFIC_FILE, sources=KERNEL_SOURCES, key="hbm_bytes_per_launch"):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    if not os.path.exists(path):
        return None
    fields = {}
    for ln in open(path):
        if "=" in ln and not ln.lstrip().startswith("#"):
            k, v = ln.split("=", 1)
            fields[k.strip()] = v.split()[0] if v.split() else ""
    if fields.get("kernel_source_sha256") != kernel_source_digest(sources):
        return None
    try:
        return int(float(fields[key]))
    except (KeyError, ValueError):
        return None


def time_graph(fn, n_sets, steps, warmup, stream, per_graph=64):
    """Per-call time with the launches recorded once into a HIP graph and
    replayed, so host-side launch cost does not hide short kernels."""
    import torch
    for i in range(warmup):
        fn(i % n_sets)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(per_graph):
            fn(i % n_sets)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // per_graph)
    cur = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(cur)
    for _ in range(reps):
        graph.replay()
    end.record(cur)
    torch.cuda.synchronize()
    del graph
    return start.elapsed_time(end) / (reps * per_graph)


def time_graph_steps(fn, n_sets, steps, warmup, stream):
    """ms per step over exactly `steps` calls recorded into one HIP graph and
    replayed once between events, after `warmup` eager calls and one untimed
    replay; synchronised on both sides."""
    import torch
    for i in range(warmup):
        fn(i % n_sets)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            fn(i % n_sets)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        graph.replay()
        end.record(stream)
    torch.cuda.synchronize()
    del graph
    return start.elapsed_time(end) / steps


def time_calls(fn, n_sets, steps, warmup, stream, segments=1):
    """ms per call over exactly `steps` calls launched back to back on the
    stream, bracketed by synchronisations.  With segments > 1, events are also
    recorded at segment boundaries inside the same timed region (no
    synchronisation between them) and the per-segment ms per call are
    returned as well."""
    import torch
    for i in range(warmup):
        fn(i % n_sets)
    torch.cuda.synchronize()
    bounds = [round(k * steps / segments) for k in range(segments + 1)]
    events = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    events[0].record(stream)
    for k in range(segments):
        for i in range(bounds[k], bounds[k + 1]):
            fn(i % n_sets)
        events[k + 1].record(stream)
    torch.cuda.synchronize()
    total = events[0].elapsed_time(events[-1]) / steps      # ms per call
    if segments == 1:
        return total
    seg = [events[k].elapsed_time(events[k + 1]) / max(1, bounds[k + 1] - bounds[k]) for k in range(segments)]
    return total, seg


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the kernels are per-row and need no "
              "cross-GPU exchange; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import gated_activation_amd as ga
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.profile_cases > 0:
        profile_cases(args.profile_cases)
        return
    if args.down_calls > 0:
        down_calls(args.down_calls, tuple(int(t) for t in (args.down_ts or "1").split(",")))
        return
    if args.down_only or args.down_geometries:
        dev = torch.device("cuda", 0)
        torch.cuda.set_device(dev)
        ts = tuple(int(t) for t in args.down_ts.split(",")) if args.down_ts else None
        shapes = [tuple(int(v) for v in sh.split("x")) for sh in args.down_shapes.split(",")] \
            if args.down_shapes else [(DOWN_D, DOWN_H)]
        res = [down_projection(dev, Markers(args.markers), geometries=args.down_geometries,
                               cpu_seconds=0.0 if args.down_geometries else args.cpu_seconds, token_counts=ts,
                               shape=sh) for sh in shapes]
        print(json.dumps({"down_projection": res[0] if not args.down_shapes else res}), flush=True)
        return
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    props = torch.cuda.get_device_properties(dev)

    # ---- inputs: one seeded set, replicated on the device past 1 GiB ----
    seed = synth.large_row_seed(T, D)
    xb = synth.gelu_large(T, D)
    bytes_call = T * 3 * D * 2
    n_sets = max(2, math.ceil(ROTATE_BYTES / bytes_call))
    x0 = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    xs = [x0] + [x0.clone() for _ in range(n_sets - 1)]
    outs = [torch.empty(T, D, dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]
    plan = ga.plan_gelu_and_mul_sparse(T, D, ga.GA_BF16, True, props.multi_processor_count)

    def gelu(i):
        ga.gelu_and_mul_sparse(xs[i], Z, out=outs[i])

    # The timed calls go straight to the C entry point with their arguments
    # marshalled once, so the host issues a launch in about 2 us and the
    # stream never waits for it (the binding's checks cost about 10 us per
    # call, which a short timed region would see at its start).
    # They run on a stream of their own (default priority), which the graph
    # capture below needs (the device's default stream cannot be captured).
    import ctypes
    hs = torch.cuda.Stream(device=dev)
    c_args = [(ctypes.c_void_p(xs[i].data_ptr()), ctypes.c_void_p(outs[i].data_ptr()), T, D, ga.GA_BF16,
               ctypes.c_float(Z), None, ctypes.c_void_p(hs.cuda_stream)) for i in range(n_sets)]
    statuses = []

    def gelu_c(i):
        statuses.append(ga.lib.ga_gelu_and_mul_sparse(*c_args[i]))

    markers = Markers(args.markers)
    # Steady-state clocks: the device ramps its clocks under load, and a short
    # timed region would otherwise include the ramp.
    warm_calls = 0
    if args.clock_warm_ms > 0:
        t_end = time.perf_counter() + args.clock_warm_ms * 1e-3
        while time.perf_counter() < t_end:
            for i in range(16):
                gelu_c((warm_calls + i) % n_sets)
            warm_calls += 16
            torch.cuda.synchronize()
    # The timed region: the K steps recorded into one HIP graph and replayed
    # once (after the W warmup steps and one untimed replay), bracketed by
    # synchronisations, so consecutive kernels start without a host launch
    # between them and the per-step time is the kernel's own (it agrees with
    # the rocprofv3 kernel trace).  The same K steps launched one by one from
    # the host are timed as well (stream_steps_us_per_call): each launch adds
    # a dispatch gap of about 0.5-1 us there.
    markers.push(f"headline T={T} d={D}")
    with torch.cuda.stream(hs):
        ms = time_graph_steps(gelu_c, n_sets, args.steps, args.warmup, hs)
        ms_stream, seg_ms = time_calls(gelu_c, n_sets, args.steps, args.warmup, hs, segments=5)
    markers.pop()
    assert statuses and all(st == ga.GA_OK for st in statuses), "gelu_and_mul_sparse returned an error"
    gbps = bytes_call / (ms * 1e-3) / 1e9
    gelu_out = outs[0].clone()      # kept for the parity check of the CPU leg

    result = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "gelu_and_mul_sparse T=2048 d=16384 bf16 in/out, gate N(0,2) up N(0,1), "
                        "z=1.6448536 (95% sparsity)",
            "T": T, "d": D, "io_dtype": "bf16", "seed": seed, "z": Z,
            "bytes_per_call": bytes_call, "rotation_sets": n_sets,
            "plan": plan.as_dict(),
            "device": f"{props.name} ({getattr(props, 'gcnArchName', '?')}, {props.multi_processor_count} CUs)",
        },
        "us_per_call": round(ms * 1e3, 3),
        "timing": "HIP events on the launch stream around one replay of a HIP graph of the K steps, after W "
                  "warmup steps and one untimed replay",
        "clock_warm": {"ms": args.clock_warm_ms, "untimed_calls": warm_calls},
        # the same K steps launched one by one from the host, and in five
        # consecutive segments of that region (events only)
        "stream_steps_us_per_call": round(ms_stream * 1e3, 3),
        "stream_segments_us_per_call": [round(x * 1e3, 3) for x in seg_ms],
        "pct_of_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "traffic": recorded_traffic(),
            "kernel": "gelu_sparse_vec_kernel<bf16, %d, %d>" % (plan.waves_per_row, plan.per_lane),
        },
        "context": CONTEXT,
    }

    if not args.no_side:
        # ---- streaming ceiling: same access pattern, no arithmetic ----
        def xor(i):
            ga.stream_xor_rows(xs[i], out=outs[i])
        markers.push(f"ceiling T={T} d={D}")
        ms_c = time_calls(xor, n_sets, args.steps, args.warmup, stream)
        markers.pop()
        ceil_gbps = bytes_call / (ms_c * 1e-3) / 1e9
        result["copy_ceiling"] = {"GBps": round(ceil_gbps, 1), "us_per_call": round(ms_c * 1e3, 3),
                                  "pct_of_peak": round(100 * ceil_gbps / PEAK_HBM_GBPS, 2)}
        result["pct_of_copy_ceiling"] = round(100.0 * gbps / ceil_gbps, 2)

        # ---- silu_and_mul_bounded on the MoE decode buffer ----
        sb = synth.moe_buffer(SILU_M, SILU_D)
        sx0 = torch.from_numpy(sb.view(np.int16)).to(dev).view(torch.bfloat16)
        s_sets = max(2, math.ceil(ROTATE_BYTES / (SILU_M * 3 * SILU_D * 2)))
        sxs = [sx0] + [sx0.clone() for _ in range(s_sets - 1)]
        souts = [torch.empty(SILU_M, SILU_D, dtype=torch.bfloat16, device=dev) for _ in range(s_sets)]
        live = torch.zeros(1, dtype=torch.int32, device=dev)
        silu_res = {"M": SILU_M, "d": SILU_D, "io_dtype": "bf16",
                    "plan": ga.plan_silu_and_mul_bounded(SILU_M, SILU_D, ga.GA_BF16, True,
                                                         props.multi_processor_count).as_dict()}
        for n_live in (SILU_M, 2048, 64):
            live.fill_(n_live)

            def silu(i):
                ga.silu_and_mul_bounded(sxs[i], live, out=souts[i])
            # Short kernels: replayed from a graph (the decode setting the
            # op is built for), so Python launch cost is not measured.
            markers.push(f"silu live={n_live}")
            ms_s = time_graph(silu, s_sets, args.steps, args.warmup, stream)
            markers.pop()
            b = n_live * 3 * SILU_D * 2 + 4
            silu_res[f"live{n_live}"] = {"us_per_call": round(ms_s * 1e3, 3),
                                         "GBps": round(b / (ms_s * 1e-3) / 1e9, 1),
                                         "pct_of_peak": round(100 * b / (ms_s * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
                                         "bytes": b, "timing": "graph replay"}
        # The same-pattern streaming kernel over only the live rows, replayed
        # the same way: what a decode-size call allows at its size.
        for n_live in (2048, 64):
            def live_ceiling(i, n_live=n_live):
                ga.stream_xor_rows(sxs[i][:n_live], out=souts[i][:n_live])
            markers.push(f"silu ceiling live={n_live}")
            ms_c = time_graph(live_ceiling, s_sets, args.steps, args.warmup, stream)
            markers.pop()
            rec = silu_res[f"live{n_live}"]
            rec["ceiling_us_per_call"] = round(ms_c * 1e3, 3)
            rec["pct_of_ceiling"] = round(100.0 * ms_c / (rec["us_per_call"] * 1e-3), 2)
        # The full buffer (live = M) moves 75 MB per call: the HBM-bound case.
        full = silu_res[f"live{SILU_M}"]

        # The same-pattern streaming kernel (read [M, 2d], write [M, d]) on
        # the same buffers, replayed the same way: what this shape allows.
        def silu_ceiling(i):
            ga.stream_xor_rows(sxs[i], out=souts[i])
        markers.push(f"silu ceiling live={SILU_M}")
        ms_c = time_graph(silu_ceiling, s_sets, args.steps, args.warmup, stream)
        markers.pop()
        full["ceiling_us_per_call"] = round(ms_c * 1e3, 3)
        full["pct_of_ceiling"] = round(100.0 * ms_c / (full["us_per_call"] * 1e-3), 2)
        silu_res["roofline"] = {
            "bound": "hbm", "achieved": full["GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(full["GBps"] / PEAK_HBM_GBPS, 4),
            "traffic": recorded_traffic(SILU_TRAFFIC_FILE, SILU_SOURCES, f"live{SILU_M}_hbm_bytes_per_launch"),
            "kernel": "act_vec_kernel<bf16, 1 item per lane, silu>", "live": SILU_M}
        if args.cpu_seconds > 0:
            live.fill_(2048)
            souts[0].zero_()
            ga.silu_and_mul_bounded(sxs[0], live, out=souts[0])
            silu_res["cpu_baseline"], silu_res["parity_sample"] = silu_cpu_baseline(
                sb, souts[0], min(3.0, args.cpu_seconds / 4))
        result["silu_and_mul_bounded"] = silu_res
        # The headline kernel replayed from a graph as well, for comparison
        # with the stream-launched figure above.
        markers.push(f"headline graph T={T} d={D}")
        ms_g = time_graph(gelu, n_sets, min(args.steps, 640), 10, stream)
        markers.pop()
        result["graph_replay_us_per_call"] = round(ms_g * 1e3, 3)

        if not args.no_sweep:
            result["down_projection"] = down_projection(dev, markers, cpu_seconds=args.cpu_seconds)
            result["sweep"] = sweep(dev, stream, props.multi_processor_count, markers)
            markers.push("siblings")
            result["siblings"] = siblings(dev, stream)
            markers.pop()

    if args.cpu_seconds > 0:
        result["cpu_baseline"], result["parity_sample"] = cpu_baseline(xb, gelu_out, args.cpu_seconds)

    print(json.dumps(result), flush=True)


# The token sweep (d = 8192), the large rows (d = 16384, 32768) and, within
# them, the whole target region T in {512, 1024, 2048, 4096} x d in {8192,
# 16384, 32768}; then short rows at T = 65536 (the packed-rows path).
SWEEP = [(T, 8192) for T in (1, 2, 8, 32, 128, 512, 1024, 2048, 4096)] + \
        [(T, d) for d in (16384, 32768) for T in (1, 64, 512, 1024, 2048, 4096)] + \
        [(65536, d) for d in (64, 128, 256)]


def sweep(dev, stream, num_cus, markers):
    """gelu_and_mul_sparse over the token sweep (d = 8192, gate N(0,1) plus a
    per-row offset), the large-row shapes (gate N(0,2)) and short rows at
    T = 65536 (gate N(0,2); the packed-rows path), bf16, each timed
    by replaying a graph of 64 launches over distinct buffers (a split-row
    workspace passed explicitly so few-row shapes take the split path), and
    by the same launches issued one by one on the stream; the same-pattern
    streaming kernel is graph-replayed on the same buffers beside each
    shape (ceiling_us_per_call, pct_of_ceiling).  Shapes under
    ~256 MB in total may be served from the Infinity Cache; shapes that move
    under 16 MiB are bound by launch latency (about 2 us per call), not by
    HBM, and are marked latency_bound: their % of peak is not meaningful."""
    import numpy as np
    import torch
    import gated_activation_amd as ga
    import synth
    out = []
    per_graph = 64
    for T, d in SWEEP:
        xb = synth.gelu_offset_rows(T, d) if d == 8192 else synth.gelu_large(T, d)
        x0 = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        bytes_call = T * 3 * d * 2
        n_sets = int(min(per_graph, max(2, math.ceil(ROTATE_BYTES / bytes_call))))
        xs = [x0] + [x0.clone() for _ in range(n_sets - 1)]
        outs = [torch.empty(T, d, dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]
        ws = torch.zeros(max(1, ga.lib.ga_gelu_and_mul_sparse_workspace_bytes(T)), dtype=torch.uint8,
                         device=dev)

        def call(i):
            ga.gelu_and_mul_sparse(xs[i], Z, out=outs[i], workspace=ws)
        reps = 4 if bytes_call > (64 << 20) else 16
        markers.push(f"sweep gelu T={T} d={d}")
        ms = time_graph(call, n_sets, reps * per_graph, 10, stream, per_graph=per_graph)
        # The same calls launched one by one on the stream: for kernels longer
        # than the host's launch cost this avoids the per-node cost of graph
        # replay; for short ones it measures the host instead.
        ms_s = time_calls(call, n_sets, reps * per_graph, 10, stream)
        markers.pop()

        def ceiling(i):
            ga.stream_xor_rows(xs[i], out=outs[i])
        # The same-pattern streaming kernel on the same buffers, replayed the
        # same way: what the shape allows without statistics or arithmetic.
        markers.push(f"sweep ceiling T={T} d={d}")
        ms_c = time_graph(ceiling, n_sets, reps * per_graph, 10, stream, per_graph=per_graph)
        markers.pop()
        plan = ga.plan_gelu_and_mul_sparse(T, d, ga.GA_BF16, True, num_cus, True)
        gbps = bytes_call / (ms * 1e-3) / 1e9
        gbps_s = bytes_call / (ms_s * 1e-3) / 1e9
        if plan.path == 3:
            geom = f"packed lanes_per_row={plan.lanes_per_row} per_lane={plan.per_lane}"
        elif plan.path == 4:
            geom = f"replicated statistics rep={plan.splits} waves={plan.waves_per_row} per_lane={plan.per_lane}"
        elif plan.splits > 1:
            geom = f"split rows splits={plan.splits} waves={plan.waves_per_row} per_lane={plan.per_lane}"
        else:
            geom = f"row waves={plan.waves_per_row} per_lane={plan.per_lane} up_late={plan.up_late}"
        out.append({"T": T, "d": d, "us_per_call": round(ms * 1e3, 3), "GBps": round(gbps, 1),
                    "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
                    "us_per_call_stream": round(ms_s * 1e3, 3),
                    "pct_of_peak_stream": round(100 * gbps_s / PEAK_HBM_GBPS, 2),
                    "ceiling_us_per_call": round(ms_c * 1e3, 3),
                    "pct_of_ceiling": round(100 * ms_c / ms, 2),
                    "latency_bound": bytes_call < LATENCY_BOUND_BYTES,
                    "bytes": bytes_call,
                    "working_set_MB": round(n_sets * bytes_call / 1e6, 1), "plan": geom})
        del xs, outs, ws
    return out


# The activation fused with the down projection: decode and small-batch
# token counts at d = 16384 (the headline rows' width) into H = 2048 output
# features (the pages give d, not the model width; 2048 is a synthetic choice).
DOWN_D, DOWN_H = 16384, 2048
DOWN_TS = (1, 2, 4, 16, 64, 128, 256)
DOWN_ROOFLINE_T = 1
DOWN_SWEEP_TS = (1, 2, 3, 4, 5, 8, 16, 32, 64, 128, 256)
# (tokens, features, waves, k step, depth) of every instantiated tiled kernel;
# the geometry sweep times each at 4 to 32 slices of d.
DOWN_TILED = [(16, 64, 4, 128, 1), (16, 64, 4, 256, 1), (16, 64, 4, 64, 3), (16, 128, 8, 128, 2),
              (32, 64, 4, 128, 1), (32, 64, 4, 64, 3),
              (64, 128, 8, 128, 1), (64, 128, 8, 64, 3), (64, 128, 4, 64, 2),
              (128, 128, 8, 64, 1), (128, 128, 8, 64, 2), (128, 256, 8, 64, 2)]
# Decode kernels (most tokens, features per workgroup, wavefronts) and the
# longest row each reaches.
DOWN_DECODE_REACH = {(1, 4, 8): 16384, (1, 4, 16): 32768, (1, 4, 4): 16384, (1, 2, 8): 16384,
                     (1, 2, 16): 32768, (1, 8, 16): 16384, (2, 4, 16): 16384, (2, 4, 8): 16384,
                     (2, 2, 16): 16384}
DOWN_DECODE = list(DOWN_DECODE_REACH)
# Staged-form product kernels (most tokens, features per workgroup, wavefronts) and their reach.
DOWN_STAGED_REACH = {(2, 4, 16): 16384, (4, 4, 16): 16384}


def time_graph_on(fn, n_sets, reps, per_graph, s, warmup=8):
    """ms per call: `per_graph` calls recorded into a HIP graph on stream s
    and replayed `reps` times between events on s (after eager warmup calls
    and one untimed replay)."""
    import torch
    with torch.cuda.stream(s):
        for i in range(warmup):
            fn(i % n_sets)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(per_graph):
            fn(i % n_sets)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        g.replay()
        start.record(s)
        for _ in range(reps):
            g.replay()
        end.record(s)
    torch.cuda.synchronize()
    del g
    return start.elapsed_time(end) / (reps * per_graph)


def down_projection(dev, markers, geometries=False, cpu_seconds=0.0, token_counts=None, shape=(DOWN_D, DOWN_H)):
    """gelu_and_mul_sparse_down (the activation fused with the down
    projection y = a . w^T) against the unfused pair on the same stream: the
    activation stored by ga_gelu_and_mul_sparse, then torch.mm with the
    weights (hipBLASLt).  Both are graph-replayed (64 launches per graph)
    over rotating (gu, w, y) sets whose weights total 1 GiB, so each call's
    64 MB of weights comes from HBM, as when a model's layers take turns.
    Algorithmic bytes per fused call: w (H*d*2) + gu (T*2d*2) + y (T*H*2);
    flops 2*T*d*H.  geometries: also time every instantiated geometry at
    each of DOWN_SWEEP_TS (the planner's measurements).  shape: (d, H); the
    roofline object and the CPU baseline are taken at d = 16384, H = 2048
    only.  One progress line per token count goes to stderr."""
    import ctypes
    import numpy as np
    import torch
    import gated_activation_amd as ga
    import synth
    d, H = shape
    w_bytes = H * d * 2
    n_sets = max(2, math.ceil(ROTATE_BYTES / w_bytes))
    w0 = torch.from_numpy(synth.down_weight(H, d, seed=1).view(np.int16)).to(dev).view(torch.bfloat16)
    wts = [w0] + [w0.clone() for _ in range(n_sets - 1)]
    s = torch.cuda.Stream(device=dev)
    hs = ctypes.c_void_p(s.cuda_stream)
    zc = ctypes.c_float(Z)
    res = {"d": d, "H": H, "io_dtype": "bf16", "weight_sets": n_sets,
           "workload": "gelu_and_mul_sparse then y = a . w^T, gate and up N(0,1) seed T, w N(0,1/d) seed 1, "
                       "z=1.6448536", "rows": []}
    sweep_rows = []
    for T in token_counts or (DOWN_SWEEP_TS if geometries else DOWN_TS):
        x0 = torch.from_numpy(synth.gelu_iid(T, d, seed=T).view(np.int16)).to(dev).view(torch.bfloat16)
        xs = [x0] + [x0.clone() for _ in range(n_sets - 1)]
        ys = [torch.empty(T, H, dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]
        acts = [torch.empty(T, d, dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]
        plan = ga.plan_gelu_and_mul_sparse_down(T, d, H)
        plans = [plan]
        if geometries:
            for tm, bh, wv, step, depth in DOWN_TILED:        # the tiled form
                if T < 3 or (tm > 16 and tm >= 2 * T):
                    continue
                for sp in (4, 8, 16, 32):
                    ks = -(-(-(-d // sp)) // step) * step
                    plans.append(ga.DownPlan.tiled(T, d, H, tm, bh, wv, step, ks, depth))
            for tmax, f, wv in DOWN_DECODE:         # the decode form
                if T <= tmax and d <= DOWN_DECODE_REACH[(tmax, f, wv)]:
                    plans.append(ga.DownPlan.decode(T, d, H, tmax, f, wv))
            for (tmax, f, wv), reach in DOWN_STAGED_REACH.items():   # the staged form
                if T <= tmax and d <= reach:
                    plans.append(ga.DownPlan.staged(T, d, H, tmax, f, wv))
        need = max(ga.gelu_and_mul_sparse_down_workspace_bytes(T, d, H, p) for p in plans)
        wsp = ga.reserve_down_workspace(need, dev, s)
        statuses = []
        bytes_call = w_bytes + T * 2 * d * 2 + T * H * 2
        flops = 2 * T * d * H

        def fused_for(p):
            args = [(ctypes.c_void_p(xs[i].data_ptr()), ctypes.c_void_p(wts[i].data_ptr()),
                     ctypes.c_void_p(ys[i].data_ptr()), T, d, H, ga.GA_BF16, zc, None, ctypes.byref(p),
                     ctypes.c_void_p(wsp.data_ptr()), wsp.numel(), hs) for i in range(n_sets)]

            def call(i):
                statuses.append(ga.lib.ga_gelu_and_mul_sparse_down_with_plan(*args[i]))
            return call
        act_args = [(ctypes.c_void_p(xs[i].data_ptr()), ctypes.c_void_p(acts[i].data_ptr()), T, d, ga.GA_BF16,
                     zc, None, hs) for i in range(n_sets)]

        def act(i):
            statuses.append(ga.lib.ga_gelu_and_mul_sparse(*act_args[i]))

        def unfused(i):
            act(i)
            torch.mm(acts[i], wts[i].t(), out=ys[i])

        def mm_only(i):
            torch.mm(acts[i], wts[i].t(), out=ys[i])
        reps = 8
        markers.push(f"down fused T={T}")
        ms_f = time_graph_on(fused_for(plan), n_sets, reps, 64, s)
        markers.pop()
        if geometries:
            for p in plans[1:]:
                markers.push(f"down geometry T={T} form={p.form} tm={p.rows_per_block} bh={p.features_per_block} "
                             f"waves={p.waves} step={p.k_step} depth={p.depth} chunk={p.k_chunk}")
                ms_p = time_graph_on(fused_for(p), n_sets, reps, 64, s)
                markers.pop()
                sweep_rows.append(f"{T},{d},{H},{p.form},{p.rows_per_block},{p.features_per_block},{p.waves},"
                                  f"{p.k_step},{p.depth},{p.k_chunk},{ms_p * 1e3!r}")
                print(sweep_rows[-1], file=sys.stderr, flush=True)
            continue
        with torch.cuda.stream(s):
            fused_for(plan)(0)
        torch.cuda.synchronize()
        y_fused = ys[0].float().clone()
        markers.push(f"down unfused T={T}")
        ms_u = time_graph_on(unfused, n_sets, reps, 64, s)
        markers.pop()
        markers.push(f"down activation T={T}")
        ms_a = time_graph_on(act, n_sets, reps, 64, s)
        markers.pop()
        markers.push(f"down mm T={T}")
        ms_m = time_graph_on(mm_only, n_sets, reps, 64, s)
        markers.pop()
        with torch.cuda.stream(s):
            unfused(0)
        torch.cuda.synchronize()
        y_unf = ys[0].float()
        rel = float((y_fused - y_unf).abs().max() / y_unf.abs().max().clamp_min(1e-30))
        gbps = bytes_call / (ms_f * 1e-3) / 1e9
        res["rows"].append({
            "T": T, "plan": plan.as_dict(), "bytes": bytes_call, "flops": flops,
            "fused_us": round(ms_f * 1e3, 3), "unfused_us": round(ms_u * 1e3, 3),
            "activation_us": round(ms_a * 1e3, 3), "mm_us": round(ms_m * 1e3, 3),
            "speedup_vs_unfused": round(ms_u / ms_f, 3),
            "GBps": round(gbps, 1), "pct_of_peak_hbm": round(100 * gbps / PEAK_HBM_GBPS, 2),
            "TFLOPs": round(flops / (ms_f * 1e-3) / 1e12, 2),
            "max_rel_diff_vs_unfused": rel})
        assert all(st == ga.GA_OK for st in statuses), "a fused or activation call returned an error"
        print(f"down d={d} H={H} T={T}: fused {ms_f * 1e3:.2f} us, unfused {ms_u * 1e3:.2f} us", file=sys.stderr,
              flush=True)
        if T == DOWN_ROOFLINE_T and (d, H) == (DOWN_D, DOWN_H):
            if plan.form == ga.GA_DOWN_DECODE:
                kname = "down_decode_kernel<bf16, tokens %d, features %d, waves %d>" % (
                    plan.rows_per_block, plan.features_per_block, plan.waves)
            elif plan.form == ga.GA_DOWN_STAGED:
                kname = "gelu_and_mul_sparse row kernel, then down_staged_kernel<bf16, tokens %d, features %d, " \
                        "waves %d>" % (plan.rows_per_block, plan.features_per_block, plan.waves)
            else:
                kname = "gelu_and_mul_sparse row kernel, then down_tiled_kernel<bf16, tokens %d, features %d, " \
                        "waves %d, step %d, depth %d> k_chunk %d" % (plan.rows_per_block, plan.features_per_block,
                                                                    plan.waves, plan.k_step, plan.depth, plan.k_chunk)
            res["roofline"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                               "frac": round(gbps / PEAK_HBM_GBPS, 4),
                               "traffic": recorded_traffic(DOWN_TRAFFIC_FILE, DOWN_SOURCES,
                                                           f"T{T}_hbm_bytes_per_call"),
                               "kernel": kname, "launches_per_call": 1 if plan.form == ga.GA_DOWN_DECODE else 2,
                               "T": T}
            if cpu_seconds > 0:
                res["cpu_baseline"], res["parity_sample"] = down_cpu_baseline(
                    synth.gelu_iid(T, d, seed=T), synth.down_weight(H, d, seed=1), ys, xs, wts, fused_for(plan), s)
        del xs, ys, acts
    if geometries:
        res["geometry_sweep_csv"] = sweep_rows
    return res


def down_calls(n, token_counts):
    """n eager calls of the fused op per token count (d = 16384, H = 2048,
    weights rotating over 1 GiB), for counter runs: each call is one
    dispatch in the decode form, two otherwise (the activation or the
    cutoffs, then the product)."""
    import numpy as np
    import torch
    import gated_activation_amd as ga
    import synth
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    d, H = DOWN_D, DOWN_H
    n_sets = max(2, math.ceil(ROTATE_BYTES / (H * d * 2)))
    w0 = torch.from_numpy(synth.down_weight(H, d, seed=1).view(np.int16)).to(dev).view(torch.bfloat16)
    wts = [w0] + [w0.clone() for _ in range(n_sets - 1)]
    for T in token_counts:
        x = torch.from_numpy(synth.gelu_iid(T, d, seed=T).view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        for i in range(n):
            ga.gelu_and_mul_sparse_down(x, wts[i % n_sets], Z, out=y)
            torch.cuda.synchronize()
            print(f"D down T={T} d={d} H={H} call {i}", flush=True)


def down_cpu_baseline(xb, wb, ys, xs, wts, fused, s):
    """The oracle's fused composition (fp64, one thread) on the roofline
    call, timed on the host, and the GPU output of that call checked against
    it (the parity tests' tolerance: ulp + 2^-13 of the absolute sum)."""
    import numpy as np
    import torch
    import oracle
    o = oracle.get()
    t0 = time.perf_counter()
    y_bits, f64, mag = o.gelu_and_mul_sparse_down(xb, wb, oracle.BF16, Z, want_f64=True)
    dt = time.perf_counter() - t0
    with torch.cuda.stream(s):
        fused(0)
    torch.cuda.synchronize()
    g = ys[0].float().cpu().numpy().astype(np.float64)
    a = np.abs(f64)
    _, e = np.frexp(a)
    ulp = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    tol = ulp + 2.0 ** -13 * mag + 1e-6
    err = np.abs(g - f64)
    T, H = f64.shape
    bytes_call = wb.size * 2 + xb.size * 2 + T * H * 2
    return ({"value": round(bytes_call / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
             "sample": f"one whole call, T={T} d={wb.shape[1]} H={H}: {dt:.2f} s"},
            {"outputs": int(g.size), "max_err_over_tol": float((err / tol).max()),
             "bitexact_frac": float((ys[0].view(torch.int16).cpu().numpy().view(np.uint16) == y_bits).mean())})


def siblings(dev, stream):
    """The other ops of the family, graph-replayed over rotating buffers:
    gelu_and_mul (tanh and erf), gelu_and_mul_sparse in fp16 and fp32, the
    round-trip form of gelu_and_mul_sparse
    and its unaligned path (a base one element off 16-byte alignment, and
    d = 16383) on the headline shape, and the bounded
    squared ReLU (not gated: read d, write d per row) on an MoE buffer."""
    import numpy as np
    import torch
    import gated_activation_amd as ga
    import synth
    res = {}
    xb = synth.gelu_large(T, D)
    x0 = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    bytes_call = T * 3 * D * 2
    n_sets = max(2, math.ceil(ROTATE_BYTES / bytes_call))
    xs = [x0] + [x0.clone() for _ in range(n_sets - 1)]
    outs = [torch.empty(T, D, dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]
    for mode in ("tanh", "none"):
        def call(i, mode=mode):
            ga.gelu_and_mul(xs[i], mode, out=outs[i])
        ms = time_graph(call, n_sets, 256, 10, stream)
        res[f"gelu_and_mul_{mode}_T{T}_d{D}"] = {
            "us_per_call": round(ms * 1e3, 3), "GBps": round(bytes_call / (ms * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * bytes_call / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2)}

    # The headline op in fp16 (same bytes as bf16) and fp32 (twice the bytes).
    for name, dt, tdt in (("fp16", synth.F16, torch.float16), ("fp32", synth.F32, torch.float32)):
        xt = synth.gelu_large(T, D, dtype=dt)
        npdt = np.int16 if dt == synth.F16 else np.int32
        t0 = torch.from_numpy(xt.view(npdt)).to(dev).view(tdt)
        b = T * 3 * D * t0.element_size()
        k_sets = max(2, math.ceil(ROTATE_BYTES / b))
        ts = [t0] + [t0.clone() for _ in range(k_sets - 1)]
        touts = [torch.empty(T, D, dtype=tdt, device=dev) for _ in range(k_sets)]

        def call(i, ts=ts, touts=touts):
            ga.gelu_and_mul_sparse(ts[i], Z, out=touts[i])
        ms = time_graph(call, k_sets, 256, 10, stream)
        res[f"gelu_and_mul_sparse_{name}_T{T}_d{D}"] = {
            "us_per_call": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2), "bytes": b}
        del ts, touts, t0

    # The round-trip form of the headline op (intermediates rounded to bf16).
    def call(i):
        ga.gelu_and_mul_sparse(xs[i], Z, out=outs[i], round_intermediates=True)
    ms = time_graph(call, n_sets, 256, 10, stream)
    res[f"gelu_and_mul_sparse_round_trip_T{T}_d{D}"] = {
        "us_per_call": round(ms * 1e3, 3), "GBps": round(bytes_call / (ms * 1e-3) / 1e9, 1),
        "pct_of_peak": round(100 * bytes_call / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2)}

    # Rows off 16-byte alignment (the unaligned path): the headline input
    # viewed one element past a 16-byte boundary, and an odd d.
    bases = [torch.empty(x0.numel() + 8, dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]
    shifted = [b[1:1 + x0.numel()].view(T, 2 * D) for b in bases]
    for a in shifted:
        a.copy_(x0)

    def call(i):
        ga.gelu_and_mul_sparse(shifted[i], Z, out=outs[i])
    ms = time_graph(call, n_sets, 256, 10, stream)
    res[f"gelu_and_mul_sparse_shifted_base_T{T}_d{D}"] = {
        "us_per_call": round(ms * 1e3, 3), "GBps": round(bytes_call / (ms * 1e-3) / 1e9, 1),
        "pct_of_peak": round(100 * bytes_call / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2)}
    del shifted, bases
    d_odd = D - 1
    odd = [torch.from_numpy(synth.gelu_large(T, d_odd).view(np.int16)).to(dev).view(torch.bfloat16)]
    odd += [odd[0].clone() for _ in range(n_sets - 1)]
    odd_out = [torch.empty(T, d_odd, dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]

    def call(i):
        ga.gelu_and_mul_sparse(odd[i], Z, out=odd_out[i])
    ms = time_graph(call, n_sets, 256, 10, stream)
    b_odd = T * 3 * d_odd * 2
    res[f"gelu_and_mul_sparse_T{T}_d{d_odd}"] = {
        "us_per_call": round(ms * 1e3, 3), "GBps": round(b_odd / (ms * 1e-3) / 1e9, 1),
        "pct_of_peak": round(100 * b_odd / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2)}
    del odd, odd_out, xs, outs
    M, d = SILU_M, 2 * SILU_D
    q0 = torch.from_numpy(synth.moe_buffer(M, SILU_D).view(np.int16)).to(dev).view(torch.bfloat16).view(M, d)
    q_sets = max(2, math.ceil(ROTATE_BYTES / (M * 2 * d * 2)))
    qs = [q0] + [q0.clone() for _ in range(q_sets - 1)]
    qouts = [torch.empty(M, d, dtype=torch.bfloat16, device=dev) for _ in range(q_sets)]
    live = torch.zeros(1, dtype=torch.int32, device=dev)
    for n_live in (M, 2048):
        live.fill_(n_live)

        def call(i):
            ga.squared_relu_bounded(qs[i], live, out=qouts[i])
        ms = time_graph(call, q_sets, 640, 10, stream)
        b = n_live * 2 * d * 2 + 4
        res[f"squared_relu_bounded_M{M}_d{d}_live{n_live}"] = {
            "us_per_call": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2)}
    return res


# Counter cases: (label, T, d, input shift, output shift, explicit plan or None
# for the planner's, with the streaming kernel beside it).
PROFILE_CASES = [
    ("headline", 2048, 16384, 0, 0, None, True),
    ("2048x32768 planner", 2048, 32768, 0, 0, None, True),
    ("2048x32768 W8V8 early", 2048, 32768, 0, 0, (8, 8, 0, 0), False),
    ("2048x32768 W16V4 early", 2048, 32768, 0, 0, (16, 4, 0, 0), False),
    ("4096x32768 planner", 4096, 32768, 0, 0, None, True),
    ("1024x32768 planner", 1024, 32768, 0, 0, None, True),
    ("512x32768 planner", 512, 32768, 0, 0, None, True),
    ("512x8192 planner", 512, 8192, 0, 0, None, True),
    ("1024x8192 planner", 1024, 8192, 0, 0, None, True),
    ("2048x8192 planner", 2048, 8192, 0, 0, None, True),
    ("4096x8192 planner", 4096, 8192, 0, 0, None, True),
    ("512x16384 planner", 512, 16384, 0, 0, None, True),
    ("1024x16384 planner", 1024, 16384, 0, 0, None, True),
    ("4096x16384 planner", 4096, 16384, 0, 0, None, True),
    ("unaligned in+1 out+1", 2048, 16384, 1, 1, None, False),
    ("unaligned in+1", 2048, 16384, 1, 0, None, False),
    ("unaligned out+1", 2048, 16384, 0, 1, None, False),
    ("unaligned kernel aligned rows", 2048, 16384, 0, 0, (8, 4, 1, 2), False),
    ("d=16383", 2048, 16383, 0, 0, None, False),
    ("T1 d8192", 1, 8192, 0, 0, None, True),
    ("T64 d8192", 64, 8192, 0, 0, None, True),
    ("T128 d8192", 128, 8192, 0, 0, None, True),
    ("T1 d32768 split", 1, 32768, 0, 0, None, True),
    ("T64 d32768 split", 64, 32768, 0, 0, None, True),
]


def profile_cases(reps):
    """Each counter case `reps` times (distinct buffer sets, gate N(0,2) and
    up N(0,1) rows tiled from a seeded block), then the same-pattern streaming
    kernel `reps` times where the rows are 16-byte aligned; one 'D <label>'
    line per launch, in launch order."""
    import numpy as np
    import torch
    import gated_activation_amd as ga
    import synth
    dev = torch.device("cuda", 0)
    block = synth.gelu_large(64, 32768)
    for label, T, d, ish, osh, plan, ceiling in PROFILE_CASES:
        rows = np.concatenate([block[:, :d], block[:, 32768:32768 + d]], axis=1)
        x0 = torch.from_numpy(rows.view(np.int16)).to(dev).view(torch.bfloat16)
        x0 = x0.repeat((T + 63) // 64, 1)[:T].contiguous()
        sets = []
        for _ in range(min(reps, 4)):
            xbuf = torch.empty(T * 2 * d + 8, dtype=torch.bfloat16, device=dev)
            x = xbuf[ish:ish + T * 2 * d].view(T, 2 * d)
            x.copy_(x0)
            obuf = torch.empty(T * d + 8, dtype=torch.bfloat16, device=dev)
            sets.append((x, obuf[osh:osh + T * d].view(T, d)))
        p = None
        if plan is not None:
            w, v, late, path = plan
            p = ga.Plan(path=path, waves_per_row=w, per_lane=v, up_late=late, block=64 * w)
        torch.cuda.synchronize()
        for k in range(reps):
            x, out = sets[k % len(sets)]
            ga.gelu_and_mul_sparse(x, Z, out=out, plan=p)
            torch.cuda.synchronize()
            print(f"D gelu {label}", flush=True)
        if ceiling:
            for k in range(reps):
                x, out = sets[k % len(sets)]
                ga.stream_xor_rows(x, out=out)
                torch.cuda.synchronize()
                print(f"D ceiling {label}", flush=True)
        del sets, x0
    print("done", flush=True)


def silu_cpu_baseline(sb, gpu_out, seconds):
    """The fp64 oracle's silu_and_mul_bounded, as it stands, on one thread,
    over 2048-row blocks of the MoE buffer (each call with all 2048 rows
    live) for about `seconds`; its first block is compared with the GPU's
    output at live = 2048."""
    import numpy as np
    import torch
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import BF16, bits_of, compare
    o = oracle.get()
    block = 2048
    ref = o.silu_and_mul_bounded(sb[:block], oracle.BF16, block)
    got = bits_of(gpu_out, BF16)
    torch.cuda.synchronize()
    parity = compare(got[:block], ref, BF16, label="bench silu sample")
    parity["rows"] = f"0..{block - 1} (live {block})"
    assert not got[block:].any(), "silu wrote rows beyond the live count"
    done, b, t0 = 0, 0, time.perf_counter()
    n_blocks = sb.shape[0] // block
    while True:
        r0 = (b % n_blocks) * block
        o.silu_and_mul_bounded(sb[r0:r0 + block], oracle.BF16, block)
        done += block
        b += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    row_bytes = 3 * SILU_D * 2
    del np
    return ({"value": round(done * row_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
             "sample": f"{done} live rows of the M=16384 d=768 bf16 buffer (2048-row blocks, 1 thread, "
                       f"{el:.1f} s, fp64)",
             "us_per_call_equiv_live2048": round(el / done * block * 1e6, 1)},
            parity)


def cpu_baseline(xb, gpu_out, seconds):
    """The fp64 oracle, as it stands, on bounded samples of the same workload
    (blocks of 64 rows in order): first on one thread for about seconds / 2,
    then on every host core the process may use (at most 16, the host share
    of one GPU), one thread per core, for about seconds / 2 of CPU time in
    total.  The oracle's C routine runs without Python's lock, so the threads
    run in parallel.  Every row of the GPU's output is also compared with
    the oracle."""
    import concurrent.futures
    import numpy as np
    import torch
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import BF16, bits_of, compare, decode

    o = oracle.get()
    block = 64
    row_bytes = 3 * D * 2

    # parity of the GPU's output against the oracle on every row
    ref, st = o.gelu_and_mul_sparse(xb, oracle.BF16, Z, want_stats=True)
    got = bits_of(gpu_out, BF16)
    torch.cuda.synchronize()
    parity = compare(got, ref, BF16, gate=decode(xb[:, :D], BF16), stats=st, label="bench output")
    parity["rows"] = f"0..{T - 1} (all)"

    def run(first_block, stride, budget):
        done, b, t0 = 0, first_block, time.perf_counter()
        while True:
            r0 = (b * block) % T
            o.gelu_and_mul_sparse(xb[r0:r0 + block], oracle.BF16, Z)
            done += block
            b += stride
            if time.perf_counter() - t0 >= budget:
                return done, time.perf_counter() - t0

    one_rows, one_s = run(0, 1, seconds / 2)
    one_gbps = one_rows * row_bytes / one_s / 1e9
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    n = max(1, min(16, n))
    wall = seconds / 2 / n
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(n) as pool:
        parts = list(pool.map(lambda i: run(i, n, wall), range(n)))
    elapsed = time.perf_counter() - t0
    all_rows = sum(p[0] for p in parts)
    gbps = all_rows * row_bytes / elapsed / 1e9
    del np
    return ({"value": round(gbps, 4), "unit": "GB/s", "cores": n, "kind": "oracle",
             "sample": f"{all_rows} rows of the T=2048 d=16384 bf16 workload (64-row blocks, {n} threads "
                       f"over {elapsed:.2f} s wall, fp64)",
             "us_per_call_equiv": round(elapsed / all_rows * T * 1e6, 1),
             "one_thread": {"value": round(one_gbps, 4), "unit": "GB/s", "cores": 1,
                            "sample": f"{one_rows} rows, {one_s:.1f} s",
                            "us_per_call_equiv": round(one_s / one_rows * T * 1e6, 1)}},
            parity)


if __name__ == "__main__":
    main()
