#!/usr/bin/env python3
"""Benchmark of the FP8 quantization library on one MI355X.

Headline (one JSON line on stdout): MXFP8 dual quantization of a 16384x4096 BF16 gradient tensor
(Laplace(0, 1e-3) with 0.01% outliers x1e4), rowwise and columnwise 1x32 blocks with E8M0
scales. One step = the four variants the workload names: {E4M3, E5M2} x {OCP round-down,
round-up}, each on its own device-resident copy of the input and its own outputs, so that no
variant finds the previous variant's data in the 256 MB last-level cache.

  effective GB/s = algorithmic bytes (2N read + N + N written + 2 * N/32 scale bytes per
                   variant = 272,629,760 B) * 4 variants * steps / wall time of the timed steps
  roofline.achieved = 272,629,760 B / average duration of one dual-quantization kernel launch:
                   a HIP event pair on the launch stream brackets the timed region, whose
                   4 * steps launches run back to back (no event between them);
                   peak = 8000 GB/s (MI355X HBM3E). A separate, untimed pass with an event
                   pair around every launch gives the per-variant split (those events add a
                   few microseconds of gap per launch, so they stay out of the timed region).
  config.cold_median_ms_per_variant = median of single launches each preceded by a 1 GiB
                   scratch fill that evicts L2 and the last-level cache (also outside `value`).
  roofline.traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE counters (in
                   profiles/), scaled by the same counters' reading for a plain copy of known
                   size; null when the kernel sources changed since the counters were taken.
  config.per_tensor_8192x8192 = per-tensor current scaling of the 8192x8192 BF16 activation, E4M3
                   and E5M2, the average launch of back-to-back launches (algorithmic bytes
                   2N + N + 8 = 201,326,600), with its % of HBM peak; the two formats are timed
                   in alternating chunks of 40 launches after a long warm-up (time_per_tensor).
  cpu_baseline   = the CPU oracle (plain C) on the whole input, all four variants, on 1 thread and on
                   T threads over row bands (T = the usable CPUs, at most 16), with the CPU model.

--suite also times every other operation on its workload (per-tensor, delayed with its variants,
1x128, 128x128, re-grouping, MXFP4, NVFP4, de-scaling and error statistics, MX rowwise on the small
tensor, a plain copy): one JSON line per operation on stderr, and the list to --suite-out if given.
"""
import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective GB/s (bytes in+out) & % of HBM peak, MXFP8 dual quantize 16384x4096"
PEAK_GBPS = 8000.0
ROWS, COLS = 16384, 4096
DUAL_BYTES = 2 * ROWS * COLS + 2 * ROWS * COLS + 2 * (ROWS * COLS // 32)   # 272,629,760
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mx_dual_16384x4096_traffic.json")
KERNEL_SOURCES = ["mx_block_scaled_amax_amd/csrc/qf8_mx.hip", "mx_block_scaled_amax_amd/csrc/qf8_device.h"]


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per dual launch from the committed counter summary, if it matches the sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sources_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--suite", action="store_true", help="also time every other operation")
    ap.add_argument("--suite-out", default=None, help="also write the suite's lines to this JSON file")
    ap.add_argument("--only-dual", action="store_true",
                    help="launch only the dual kernel (E4M3 round-up) --steps times, for counter runs")
    ap.add_argument("--only-per-tensor", action="store_true",
                    help="launch only per-tensor E4M3 on the 8192x8192 activation --steps times, for counter runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="launch only a plain 256 MiB device copy --steps times, for counter runs")
    return ap.parse_args()


def to_dev(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class DualCall:
    """Pre-marshalled quantize_mx_dual call (keeps Python overhead out of the timed loop)."""

    def __init__(self, qf8, x, fmt, rnd, stream):
        import torch
        self.out = [torch.empty((ROWS, COLS), dtype=torch.uint8, device="cuda"),
                    torch.empty((ROWS, COLS // 32), dtype=torch.uint8, device="cuda"),
                    torch.empty((COLS, ROWS), dtype=torch.uint8, device="cuda"),
                    torch.empty((COLS, ROWS // 32), dtype=torch.uint8, device="cuda")]
        self.x = x
        vp = ctypes.c_void_p
        self.fn = qf8._load().quantize_mx_dual
        self.args = (vp(x.data_ptr()), 0, ROWS, COLS, fmt, rnd) + tuple(vp(t.data_ptr()) for t in self.out) + \
                    (None, vp(stream.cuda_stream))

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"quantize_mx_dual failed with status {st}")


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(xb):
    """The CPU oracle (plain single-threaded C, test infrastructure) on the whole 16384x4096
    workload, all four dual variants: once on one thread, once with the rows cut into T bands of
    a multiple of 32 rows run on T threads (ctypes releases the GIL, so the bands run in parallel;
    each band's columnwise blocks lie inside it). T = the CPUs this process may use, at most 16 (a
    GPU's share of the host). The T-thread rate is the reported value."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle as O
    variants = [(f, r) for f in (O.E4M3, O.E5M2) for r in (O.ROUND_DOWN, O.ROUND_UP)]
    nbytes = len(variants) * DUAL_BYTES
    nproc = os.cpu_count() or 1
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = nproc
    threads = max(1, min(16, usable))
    t0 = time.perf_counter()
    for fmt, rnd in variants:
        O.quantize_mx(xb, fmt, rnd)
    one = time.perf_counter() - t0
    band = -(-ROWS // threads)
    band = -(-band // 32) * 32
    bounds = [(r, min(r + band, ROWS)) for r in range(0, ROWS, band)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        for fmt, rnd in variants:
            list(ex.map(lambda b: O.quantize_mx(xb[b[0]:b[1]], fmt, rnd), bounds))
    par = time.perf_counter() - t0
    return {"value": round(nbytes / par / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole 16384x4096 input, all four dual variants ({nbytes} algorithmic bytes): "
                      f"{par:.2f} s on {threads} threads (row bands of {band}), {one:.2f} s on 1 thread",
            "one_thread_GBps": round(nbytes / one / 1e9, 4), "cpu_model": cpu_model(), "nproc": nproc,
            "usable_cpus": usable}


def time_per_tensor(args, qf8, stream):
    """Per-tensor current scaling of the 8192x8192 BF16 activation (N(0,1), 0.1% entries x1000,
    seed 2), E4M3 and E5M2: a round is one launch on each of four device-resident input copies.
    After at least 100 untimed rounds of each format (this leg follows the cold launches, whose
    cache flushes leave the GPU idle between launches), args.steps rounds per format are timed in
    chunks of up to 10 rounds, the two formats alternating chunk by chunk so that both see the same
    conditions; each chunk's launches run back to back under one HIP event pair on the launch
    stream. Algorithmic bytes 2N read + N written + the fp32 amax and scale = 201,326,600 per launch."""
    import torch
    from synthetic import per_tensor_activation
    xb = per_tensor_activation()
    xs = [to_dev(xb) for _ in range(4)]
    n = xb.size
    nbytes = 3 * n + 8
    q = torch.empty(xb.shape, dtype=torch.uint8, device="cuda")
    am = torch.empty(1, dtype=torch.float32, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = qf8.workspace(xs[0])
    lib = qf8._load()
    vp = ctypes.c_void_p
    sp = vp(stream.cuda_stream)
    out = {"workload": "per_tensor_current_8192x8192", "values": "N(0,1), 0.1% entries x1000, seed 2",
           "algorithmic_bytes": nbytes}
    runs = {}
    for fmt, name in ((qf8.E4M3, "e4m3"), (qf8.E5M2, "e5m2")):
        args_of = [(vp(x.data_ptr()), 0, xb.shape[0], xb.shape[1], fmt, vp(q.data_ptr()), vp(am.data_ptr()),
                    vp(sc.data_ptr()), None, vp(ws.data_ptr()), ws.numel(), sp) for x in xs]

        def run(args_of=args_of):
            for a in args_of:
                st = lib.quantize_per_tensor(*a)
                if st != 0:
                    raise RuntimeError(f"quantize_per_tensor failed with status {st}")
        runs[name] = run
    for _ in range(max(args.warmup, 100)):
        for run in runs.values():
            run()
    torch.cuda.synchronize()
    spans = {name: [] for name in runs}
    done = 0
    while done < args.steps:
        rounds = min(10, args.steps - done)
        for name, run in runs.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(rounds):
                run()
            e1.record(stream)
            spans[name].append((e0, e1))
        done += rounds
    torch.cuda.synchronize()
    for name in runs:
        ms = sum(e0.elapsed_time(e1) for e0, e1 in spans[name]) / (4 * args.steps)
        gbps = nbytes / (ms / 1e3) / 1e9
        out[name] = {"avg_launch_ms": round(ms, 5), "GBps": round(gbps, 1),
                     "pct_of_hbm_peak": round(100 * gbps / PEAK_GBPS, 2)}
    del xs
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this quantization path has no multi-GPU leg here "
              "; use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mx_block_scaled_amax_amd as qf8
    from synthetic import mx_gradient

    torch.cuda.init()
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        n = 256 << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": args.steps}))
        return

    if args.only_per_tensor:
        from synthetic import per_tensor_activation
        xa = to_dev(per_tensor_activation())
        q = torch.empty(xa.shape, dtype=torch.uint8, device="cuda")
        am = torch.empty(1, dtype=torch.float32, device="cuda")
        sc = torch.empty(1, dtype=torch.float32, device="cuda")
        ws = qf8.workspace(xa)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            qf8.quantize_per_tensor(xa, qf8.E4M3, q=q, amax=am, scale=sc, ws=ws)
        torch.cuda.synchronize()
        print(json.dumps({"per_tensor_launches": args.steps, "bytes_per_launch": 3 * xa.numel() + 8}))
        return

    xb = mx_gradient(ROWS, COLS, seed=4)
    variants = [(f, r) for f in (qf8.E4M3, qf8.E5M2) for r in (qf8.ROUND_DOWN, qf8.ROUND_UP)]

    if args.only_dual:
        call = DualCall(qf8, to_dev(xb), qf8.E4M3, qf8.ROUND_UP, stream)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
        print(json.dumps({"dual_launches": args.steps, "bytes_per_launch": DUAL_BYTES}))
        return

    calls = [DualCall(qf8, to_dev(xb), f, r, stream) for f, r in variants]
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()

    ev_begin, ev_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_begin.record(stream)
    for _ in range(args.steps):
        for c in calls:
            c()
    ev_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_launch_s = ev_begin.elapsed_time(ev_end) / 1e3 / (args.steps * len(calls))
    achieved = DUAL_BYTES / avg_launch_s / 1e9

    # per-variant split (untimed pass, one event pair per launch)
    split_steps = min(args.steps, 20)
    starts = [[torch.cuda.Event(enable_timing=True) for _ in calls] for _ in range(split_steps)]
    ends = [[torch.cuda.Event(enable_timing=True) for _ in calls] for _ in range(split_steps)]
    for k in range(split_steps):
        for j, c in enumerate(calls):
            starts[k][j].record(stream)
            c()
            ends[k][j].record(stream)
    torch.cuda.synchronize()
    kms = np.array([[starts[k][j].elapsed_time(ends[k][j]) for j in range(len(calls))] for k in range(split_steps)])
    # cold launches (untimed for `value`): a 1 GiB scratch fill before each one evicts L2 and the
    # last-level cache, then one event pair around the launch; median over the reps
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cold = [[] for _ in calls]
    for k in range(min(args.steps, 20)):
        for j, c in enumerate(calls):
            flush.fill_(k & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            c()
            e1.record(stream)
            torch.cuda.synchronize()
            cold[j].append(e0.elapsed_time(e1))
    del flush
    cold_med = [float(np.median(v)) for v in cold]
    cold_all = np.concatenate([np.array(v) for v in cold])
    per_tensor = time_per_tensor(args, qf8, stream)
    value = len(calls) * DUAL_BYTES * args.steps / wall / 1e9
    traffic = stored_traffic()
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mxfp8_dual_16384x4096", "rows": ROWS, "cols": COLS, "input": "bf16",
                   "values": "Laplace(0, 1e-3), 0.01% entries x1e4, seed 4",
                   "variants": ["e4m3-round_down", "e4m3-round_up", "e5m2-round_down", "e5m2-round_up"],
                   "bytes_per_variant": DUAL_BYTES, "pct_of_hbm_peak": round(100 * value / PEAK_GBPS, 2),
                   "avg_launch_ms": round(avg_launch_s * 1e3, 5),
                   "launch_ms_per_variant_event_bracketed": {v: round(float(kms[:, j].mean()), 5) for j, v in enumerate(
                       ["e4m3-round_down", "e4m3-round_up", "e5m2-round_down", "e5m2-round_up"])},
                   "cold_median_ms_per_variant": {v: round(cold_med[j], 5) for j, v in enumerate(
                       ["e4m3-round_down", "e4m3-round_up", "e5m2-round_down", "e5m2-round_up"])},
                   "cold_pct_of_hbm_peak": round(100 * DUAL_BYTES / (float(np.mean(cold_med)) / 1e3) / 1e9 / PEAK_GBPS, 2),
                   "cold_ms_all_variants": {"median": round(float(np.median(cold_all)), 5),
                                            "min": round(float(cold_all.min()), 5),
                                            "p90": round(float(np.percentile(cold_all, 90)), 5)},
                   "per_tensor_8192x8192": per_tensor},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(xb)
    print(json.dumps(line), flush=True)

    if args.suite:
        del calls
        torch.cuda.empty_cache()
        run_suite(args)


# ---------------------------------------------------------------------------------------------
# --suite: every other operation on its own workload (one JSON line each on stderr)
# ---------------------------------------------------------------------------------------------
class PreCall:
    """A library entry point with its ctypes arguments marshalled once, so that back-to-back
    launches are not limited by Python."""

    def __init__(self, fn, *args):
        self.fn, self.args = fn, args

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"{self.fn.__name__} failed with status {st}")


def _timed(torch, stream, fns, reps, warmup):
    """Run fns round-robin (each on its own buffers). Returns (per-call ms with an event pair
    around each call, mean ms per call of reps calls back to back under one event pair)."""
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record(stream)
        fns[i % len(fns)]()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_call = [a.elapsed_time(b) for a, b in ev]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        fns[i % len(fns)]()
    e1.record(stream)
    torch.cuda.synchronize()
    return per_call, e0.elapsed_time(e1) / reps


def _summ(name, nbytes, timing, extra=None):
    """One suite line: back-to-back mean (the throughput figure) and the per-call distribution."""
    import numpy as np
    ms, b2b = timing
    ms = np.array(ms)
    med = float(np.median(ms))
    d = {"op": name, "algorithmic_bytes": int(nbytes), "mean_ms_back_to_back": round(b2b, 5),
         "GBps": round(nbytes / b2b / 1e6, 1), "pct_of_8TBps": round(100 * nbytes / b2b / 1e6 / PEAK_GBPS, 2),
         "per_call_event_median_ms": round(med, 5), "per_call_event_min_ms": round(float(ms.min()), 5),
         "per_call_event_p90_ms": round(float(np.percentile(ms, 90)), 5)}
    if extra:
        d.update(extra)
    print(json.dumps(d), file=sys.stderr, flush=True)
    return d


def run_suite(args):
    import numpy as np
    import torch

    import mx_block_scaled_amax_amd as qf8
    from synthetic import (block_weight, delayed_base, delayed_sigmas, mx_gradient, per_tensor_activation,
                           per_tensor_small, token_activation)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    L = qf8._load()
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    reps, warm = 40, 5
    res = []

    # plain copy: the achievable streaming ceiling (read 2N + write 2N of a 16384x4096 BF16 tensor)
    src = [torch.empty(2 * ROWS * COLS, dtype=torch.uint8, device="cuda").fill_(1) for _ in range(4)]
    dst = [torch.empty_like(t) for t in src]
    fns = [lambda a=a, b=b: b.copy_(a) for a, b in zip(src, dst)]
    res.append(_summ("copy 128 MiB -> 128 MiB (torch)", 4 * ROWS * COLS, _timed(torch, stream, fns, reps, warm)))
    del src, dst

    # per-tensor current scaling, 8192x8192 BF16, E4M3 and E5M2 (4 input copies in rotation)
    xb = per_tensor_activation()
    xs = [to_dev(xb) for _ in range(4)]
    n = xb.size
    q = torch.empty(xb.shape, dtype=torch.uint8, device="cuda")
    am = torch.empty(1, dtype=torch.float32, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = qf8.workspace(xs[0])
    for fmt, name in ((qf8.E4M3, "e4m3"), (qf8.E5M2, "e5m2")):
        fns = [PreCall(L.quantize_per_tensor, vp(x), 0, xb.shape[0], xb.shape[1], fmt, vp(q), vp(am), vp(sc), None,
                       vp(ws), ws.numel(), sp) for x in xs]
        res.append(_summ(f"per_tensor 8192x8192 {name}", 3 * n + 8, _timed(torch, stream, fns, reps, warm),
                         {"note": "one kernel, x read from HBM once (held on chip across a grid barrier)"}))
    del xs

    # per-tensor and MX rowwise on the 256x512 tensor (latency-bound)
    xsm = to_dev(per_tensor_small())
    qs = torch.empty(xsm.shape, dtype=torch.uint8, device="cuda")
    ssm = torch.empty((xsm.shape[0], xsm.shape[1] // 32), dtype=torch.uint8, device="cuda")
    res.append(_summ("per_tensor 256x512 e4m3", 3 * xsm.numel() + 8,
                     _timed(torch, stream, [PreCall(L.quantize_per_tensor, vp(xsm), 0, xsm.shape[0], xsm.shape[1], qf8.E4M3,
                                                    vp(qs), vp(am), vp(sc), None, vp(ws), ws.numel(), sp)], reps, warm)))
    res.append(_summ("mx rowwise 256x512 e4m3 round-up", 3 * xsm.numel() + xsm.numel() // 32,
                     _timed(torch, stream, [PreCall(L.quantize_mx_dual, vp(xsm), 0, xsm.shape[0], xsm.shape[1], qf8.E4M3,
                                                    qf8.ROUND_UP, vp(qs), vp(ssm), None, None, None, sp)], reps, warm)))

    # delayed scaling: 100 iterations of 4096x14336 (history 16, Interval 5, N 3, E4M3)
    z = torch.from_numpy(delayed_base()).cuda()
    sig = delayed_sigmas()
    xsd = [(z * float(s)).to(torch.bfloat16) for s in sig]
    del z
    qd = torch.empty(xsd[0].shape, dtype=torch.uint8, device="cuda")
    wsd = qf8.workspace(xsd[0])
    R, C = xsd[0].shape

    def steps_of(state, amax_out=None):
        return [PreCall(L.quantize_delayed, vp(x), 0, R, C, state.struct.fmt, ctypes.byref(state.struct), vp(qd), None,
                        None if amax_out is None else vp(amax_out), None, vp(wsd), wsd.numel(), sp) for x in xsd]
    for c in steps_of(qf8.DelayedState(16, 5, 3, qf8.E4M3))[:3]:     # warm the code paths on a throwaway state
        c()
    torch.cuda.synchronize()
    # pass 1: an event pair around every step (distribution, step 0 alone)
    calls = steps_of(qf8.DelayedState(16, 5, 3, qf8.E4M3))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
    for t, c in enumerate(calls):
        ev[t][0].record(stream)
        c()
        ev[t][1].record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    # pass 2: a fresh state, steps 1..99 back to back under one event pair
    calls = steps_of(qf8.DelayedState(16, 5, 3, qf8.E4M3))
    calls[0]()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for c in calls[1:]:
        c()
    e1.record(stream)
    torch.cuda.synchronize()
    nd = xsd[0].numel()
    res.append(_summ("delayed 4096x14336 e4m3, steps 1..99", 3 * nd, (ms[1:], e0.elapsed_time(e1) / (len(calls) - 1)),
                     {"step0_ms": round(ms[0], 5), "total_100_steps_ms_event_per_step": round(sum(ms), 4),
                      "note": "step 0 is current scaling (single-pass kernel + finalize); update steps one fused "
                              "cast pass + a one-workgroup finalize; reuse steps, asked for no amax, the cast alone"}))
    # the same 99 steps with the amax split over the Interval, and with the mean estimator
    amax_every = torch.empty(1, dtype=torch.float32, device="cuda")
    for label, kw, ao in (("amax_out every step", {}, amax_every), ("split amax", {"split": True}, None),
                          ("mean estimator", {"estimator": qf8.EST_MEAN}, None)):
        calls = steps_of(qf8.DelayedState(16, 5, 3, qf8.E4M3, **kw), ao)
        calls[0]()
        e0.record(stream)
        for c in calls[1:]:
            c()
        e1.record(stream)
        torch.cuda.synchronize()
        b2b = e0.elapsed_time(e1) / (len(calls) - 1)
        res.append(_summ(f"delayed 4096x14336 e4m3 {label}, steps 1..99", 3 * nd, ([b2b], b2b)))
    del xsd

    # fine-grained: 1x128 activations 8192x7168 and 128x128 weights 7168x18432 (E4M3)
    xa = token_activation()
    xas = [to_dev(xa) for _ in range(4)]
    qa = torch.empty(xa.shape, dtype=torch.uint8, device="cuda")
    sa = torch.empty((xa.shape[0], xa.shape[1] // 128), dtype=torch.float32, device="cuda")
    res.append(_summ("block 1x128 8192x7168 e4m3", 3 * xa.size + 4 * sa.numel(),
                     _timed(torch, stream, [PreCall(L.quantize_block, vp(x), 0, xa.shape[0], xa.shape[1], 1, 128, qf8.E4M3,
                                                    vp(qa), vp(sa), None, None, sp) for x in xas], reps, warm)))
    del xas
    xw = block_weight()
    xws = [to_dev(xw) for _ in range(2)]
    qw = torch.empty(xw.shape, dtype=torch.uint8, device="cuda")
    sw = torch.empty((xw.shape[0] // 128, xw.shape[1] // 128), dtype=torch.float32, device="cuda")
    res.append(_summ("block 128x128 7168x18432 e4m3", 3 * xw.size + 4 * sw.numel(),
                     _timed(torch, stream, [PreCall(L.quantize_block, vp(x), 0, xw.shape[0], xw.shape[1], 128, 128, qf8.E4M3,
                                                    vp(qw), vp(sw), None, None, sp) for x in xws], reps, warm)))
    del xws

    # power-of-two 1x128 groups and the 1x128 -> 128x1 transposed re-grouping, 8192x7168 E4M3
    xa = token_activation()
    xads = [to_dev(xa) for _ in range(4)]
    na = xa.size
    gsz = xa.shape[0] * (xa.shape[1] // 128)
    qa2 = torch.empty(xa.shape, dtype=torch.uint8, device="cuda")
    sa2 = torch.empty((xa.shape[0], xa.shape[1] // 128), dtype=torch.float32, device="cuda")
    res.append(_summ("block 1x128 pow2 scales 8192x7168 e4m3", 3 * na + 4 * gsz,
                     _timed(torch, stream, [PreCall(L.quantize_block_ex, vp(x), 0, xa.shape[0], xa.shape[1], 1, 128,
                                                    qf8.E4M3, qf8.FLAG_POW2_SCALES, vp(qa2), vp(sa2), None, None, sp)
                                            for x in xads], reps, warm)))
    qT2 = torch.empty((xa.shape[1], xa.shape[0]), dtype=torch.uint8, device="cuda")
    sT2 = torch.empty((xa.shape[1], xa.shape[0] // 128), dtype=torch.float32, device="cuda")
    res.append(_summ("requant 1x128 -> 128x1 transposed 8192x7168 e4m3 pow2", na + 4 * gsz + na + 4 * (na // 128),
                     _timed(torch, stream, [PreCall(L.requantize_1x128_to_128x1, vp(qa2), vp(sa2), xa.shape[0], xa.shape[1],
                                                    qf8.E4M3, qf8.E4M3, qf8.FLAG_POW2_SCALES, vp(qT2), vp(sT2), None, sp)],
                            reps, warm)))
    del xads, qa2, qT2

    # FP4 on the same gradient workload: MXFP4 dual / rowwise, NVFP4 (amax pass + cast, or a
    # caller-given amax and one read). Algorithmic bytes count x once.
    xg = to_dev(mx_gradient(ROWS, COLS, seed=4))
    N = ROWS * COLS
    f4r = torch.empty((ROWS, COLS // 2), dtype=torch.uint8, device="cuda")
    f4rs = torch.empty((ROWS, COLS // 32), dtype=torch.uint8, device="cuda")
    f4c = torch.empty((COLS, ROWS // 2), dtype=torch.uint8, device="cuda")
    f4cs = torch.empty((COLS, ROWS // 32), dtype=torch.uint8, device="cuda")
    for rnd, rname in ((qf8.ROUND_DOWN, "round-down"), (qf8.ROUND_UP, "round-up")):
        res.append(_summ(f"mxfp4 dual 16384x4096 bf16 {rname}", 2 * N + N + N // 16,
                         _timed(torch, stream, [PreCall(L.quantize_mxfp4_dual, vp(xg), 0, ROWS, COLS, rnd, vp(f4r),
                                                        vp(f4rs), vp(f4c), vp(f4cs), None, sp)], reps, warm)))
    res.append(_summ("mxfp4 rowwise 16384x4096 bf16 round-down", 2 * N + N // 2 + N // 32,
                     _timed(torch, stream, [PreCall(L.quantize_mxfp4_dual, vp(xg), 0, ROWS, COLS, qf8.ROUND_DOWN, vp(f4r),
                                                    vp(f4rs), None, None, None, sp)], reps, warm)))
    del f4c, f4cs
    nvs = torch.empty((ROWS, COLS // 16), dtype=torch.uint8, device="cuda")
    nvt = torch.empty(1, dtype=torch.float32, device="cuda")
    nva = torch.empty(1, dtype=torch.float32, device="cuda")
    wsn = qf8.workspace(xg)
    res.append(_summ("nvfp4 16384x4096 bf16 (measured amax, single pass)", 2 * N + N // 2 + N // 16,
                     _timed(torch, stream, [PreCall(L.quantize_nvfp4, vp(xg), 0, ROWS, COLS, None, vp(f4r), vp(nvs),
                                                    vp(nvt), vp(nva), None, vp(wsn), wsn.numel(), sp)], reps, warm)))
    res.append(_summ("nvfp4 16384x4096 bf16 (caller amax, one read)", 2 * N + N // 2 + N // 16,
                     _timed(torch, stream, [PreCall(L.quantize_nvfp4, vp(xg), 0, ROWS, COLS, vp(nva), vp(f4r), vp(nvs),
                                                    vp(nvt), None, None, None, 0, sp)], reps, warm)))
    o16f = torch.empty((ROWS, COLS), dtype=torch.bfloat16, device="cuda")
    L.quantize_mxfp4_dual(vp(xg), 0, ROWS, COLS, qf8.ROUND_DOWN, vp(f4r), vp(f4rs), None, None, None, sp)
    res.append(_summ("dequant mxfp4 rowwise 16384x4096 -> bf16", N // 2 + N // 32 + 2 * N,
                     _timed(torch, stream, [PreCall(L.dequantize_mxfp4, vp(f4r), vp(f4rs), ROWS, COLS, vp(o16f), 0, sp)],
                            reps, warm)))
    L.quantize_nvfp4(vp(xg), 0, ROWS, COLS, vp(nva), vp(f4r), vp(nvs), vp(nvt), None, None, None, 0, sp)
    res.append(_summ("dequant nvfp4 16384x4096 -> bf16", N // 2 + N // 16 + 2 * N,
                     _timed(torch, stream, [PreCall(L.dequantize_nvfp4, vp(f4r), vp(nvs), vp(nvt), ROWS, COLS, vp(o16f), 0,
                                                    sp)], reps, warm)))
    del f4r, f4rs, nvs, o16f

    # dequantization (and fused error statistics) of the MX dual result and the per-tensor result
    q_row, s_row, q_colT, s_colT = qf8.quantize_mx_dual(xg, qf8.E4M3, qf8.ROUND_DOWN)
    o16 = torch.empty((ROWS, COLS), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(8, dtype=torch.int64, device="cuda")
    wsg = qf8.workspace(xg)
    res.append(_summ("dequant mx rowwise 16384x4096 -> bf16", N + N // 32 + 2 * N,
                     _timed(torch, stream, [PreCall(L.dequantize_mx, vp(q_row), vp(s_row), ROWS, COLS, qf8.E4M3, vp(o16), 0,
                                                    None, 0, None, None, 0, sp)], reps, warm)))
    res.append(_summ("dequant mx rowwise + stats 16384x4096 -> bf16", N + N // 32 + 2 * N + 2 * N,
                     _timed(torch, stream, [PreCall(L.dequantize_mx, vp(q_row), vp(s_row), ROWS, COLS, qf8.E4M3, vp(o16), 0,
                                                    vp(xg), 0, vp(st), vp(wsg), wsg.numel(), sp)], reps, warm)))
    res.append(_summ("stats only, mx rowwise 16384x4096", N + N // 32 + 2 * N,
                     _timed(torch, stream, [PreCall(L.dequantize_mx, vp(q_row), vp(s_row), ROWS, COLS, qf8.E4M3, None, 0,
                                                    vp(xg), 0, vp(st), vp(wsg), wsg.numel(), sp)], reps, warm)))
    del q_row, s_row, q_colT, s_colT
    qp, amp, scp = qf8.quantize_per_tensor(xg, qf8.E4M3)
    res.append(_summ("dequant per-tensor 16384x4096 -> bf16", N + 2 * N + 4,
                     _timed(torch, stream, [PreCall(L.dequantize_scaled, vp(qp), N, qf8.E4M3, vp(scp), vp(o16), 0,
                                                    None, 0, None, None, 0, sp)], reps, warm)))
    del xg, o16, qp
    if args.suite_out:
        d = os.path.dirname(os.path.abspath(args.suite_out))
        os.makedirs(d, exist_ok=True)
        with open(args.suite_out, "w") as f:
            json.dump(res, f, indent=1)


if __name__ == "__main__":
    main()
