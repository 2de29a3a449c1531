"""Benchmark: GiB/s written by the counter-based bulk fills on one MI355X.

One step runs every fill of the hot path once at 2^28 elements (tandem-cuda,
"Performance", §GPU: 2^28 elements into device memory): the uniform fills (u8, u16,
f16 bits, u32, u64, f32, f64, bool; key and start draw cycle through 1..3 and 0, 1, 3
from step to step), the bounded fills (u32/u64 below 1000 and below 2^W - 2, int32 and
int64 with a low bound), the f64 ziggurat and f32 Box-Muller normals, fused dropout over
X = f32[2^20, 256] (p = 0.1), the choice fill through a 1000-way Zipf(1.1) alias table,
and the Philox4x32-10 u32 fill.  Inputs are resident in device memory before timing.

The JSON line reports the whole step's bytes written per second (`value`), each fill's
median rate, the roofline of the dominant kernel (algorithmic bytes per launch over its
HIP-event-timed average duration, against the 8 TB/s HBM peak), and the CPU oracle timed
on a bounded sample of the same step on this host.
"""
import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

GIB = float(1 << 30)
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=2.0,
                    help="keep warming up for at least this long (the pages warm each row for 2 s)")
    ap.add_argument("--cpu-sample-log2", type=int, default=27,
                    help="elements per fill in the oracle's CPU sample (0 disables it)")
    ap.add_argument("--only", default="",
                    help="comma-separated fill names to run (profiling); 'calib_copy' adds a plain 1 GiB "
                         "device copy used to calibrate the HBM byte counters")
    return ap.parse_args()


def build_step(tk, torch, n):
    """Returns a list of (name, bytes_written, bytes_read, kernels, fn(step_index))."""
    import tk_inputs as ti
    dev = torch.device("cuda")
    out = torch.empty(8 * n, dtype=torch.uint8, device=dev)   # 2 GiB, reused by every fill
    x = torch.empty(n, dtype=torch.float32, device=dev)       # dropout input
    tk.tk_fill_normal_f32(ti.DROPOUT_X_KEY, 0, n, x)          # X ~ N(0, 1), seed 7
    table = tk.tk_alias_create(ti.zipf_weights())
    optr = out.data_ptr()
    # the library finishes ziggurat misses inside the table pass unless told otherwise
    zig_kernels = 3 if os.environ.get("TK_ZIG_MODE") == "split" else 1
    ks = lambda s: ti.KEYS[s % 3]
    st = lambda s: ti.STARTS[s % 3]
    fills = [
        ("u32", 4 * n, 0, 1, lambda s: tk.tk_fill_u32(ks(s), st(s), n, optr)),
        ("u64", 8 * n, 0, 1, lambda s: tk.tk_fill_u64(ks(s), st(s), n, optr)),
        ("f32", 4 * n, 0, 1, lambda s: tk.tk_fill_f32(ks(s), st(s), n, optr)),
        ("f64", 8 * n, 0, 1, lambda s: tk.tk_fill_f64(ks(s), st(s), n, optr)),
        ("u16", 2 * n, 0, 1, lambda s: tk.tk_fill_u16(ks(s), st(s), n, optr)),
        ("f16_bits", 2 * n, 0, 1, lambda s: tk.tk_fill_f16_bits(ks(s), st(s), n, optr)),
        ("u8", n, 0, 1, lambda s: tk.tk_fill_u8(ks(s), st(s), n, optr)),
        ("bool", n, 0, 1, lambda s: tk.tk_fill_bool(ks(s), st(s), n, optr)),
        ("u32_below_1000", 4 * n, 0, 1, lambda s: tk.tk_fill_u32_below(1, 0, n, 1000, optr)),
        ("u32_below_2^32-2", 4 * n, 0, 1, lambda s: tk.tk_fill_u32_below(1, 0, n, (1 << 32) - 2, optr)),
        ("u64_below_1000", 8 * n, 0, 1, lambda s: tk.tk_fill_u64_below(1, 0, n, 1000, optr)),
        ("u64_below_2^64-2", 8 * n, 0, 1, lambda s: tk.tk_fill_u64_below(1, 0, n, (1 << 64) - 2, optr)),
        ("i32_below_low", 4 * n, 0, 1, lambda s: tk.tk_fill_i32_below(1, 0, n, ti.LOW, ti.LOW_BOUND, optr)),
        ("i64_below32_low", 8 * n, 0, 1, lambda s: tk.tk_fill_i64_below32(1, 0, n, ti.LOW, ti.LOW_BOUND, optr)),
        ("normal_f64", 8 * n, 0, zig_kernels, lambda s: tk.tk_fill_normal_f64(1, st(s), n, optr)),
        ("normal_f32", 4 * n, 0, 1, lambda s: tk.tk_fill_normal_f32(1, 0, n, optr)),
        ("dropout_f32", 4 * n, 4 * n, 1,
         lambda s: tk.tk_dropout_f32(ti.DROPOUT_KEY, 0, n, ti.DROPOUT_P, x.data_ptr(), optr)),
        ("choice_u32", 4 * n, 0, 1, lambda s: tk.tk_fill_choice_u32(1, 0, n, table, optr)),
        ("philox_u32", 4 * n, 0, 1, lambda s: tk.tk_philox_fill_u32(1, st(s), n, optr)),
    ]
    # rows beyond the hot path, timed after it and not counted in `value`
    m20, m24 = 1 << 20, 1 << 24
    mis_n = n - m20
    next_rows = [
        ("exponential_f64", 8 * n, 0, 1, lambda s: tk.tk_fill_exponential_f64(ks(s), st(s), n, optr)),
        ("exponential_f32", 4 * n, 0, 1, lambda s: tk.tk_fill_exponential_f32(ks(s), st(s), n, optr)),
        ("dropout_backward_f32", 4 * n, 4 * n, 1,
         lambda s: tk.tk_dropout_backward_f32(ti.DROPOUT_KEY, 0, n, ti.DROPOUT_P, x.data_ptr(), optr)),
        # generator and normal variants
        ("philox_u32_below_1000", 4 * n, 0, 1, lambda s: tk.tk_philox_fill_u32_below(1, st(s), n, 1000, optr)),
        ("philox_u64_below_1000", 8 * n, 0, 1, lambda s: tk.tk_philox_fill_u64_below(1, st(s), n, 1000, optr)),
        ("philox_choice_u32", 4 * n, 0, 1, lambda s: tk.tk_philox_fill_choice_u32(1, 0, n, table, optr)),
        ("philox_normal_f32", 4 * n, 0, 1, lambda s: tk.tk_philox_fill_normal_f32(1, st(s), n, optr)),
        ("philox_normal_f64", 8 * n, 0, zig_kernels, lambda s: tk.tk_philox_fill_normal_f64(1, st(s), n, optr)),
        ("normal_f32_half_turn", 4 * n, 0, 1, lambda s: tk.tk_fill_normal_f32_half_turn(1, st(s), n, optr)),
        ("randn_f32", 4 * n, 0, 1, lambda s: tk.tk_fill_randn_f32(1, 0, n, optr)),
        # outputs 8 bytes past a 4 KiB boundary: the vector grid starts at the next boundary
        # and the head is written element by element (2^28 - 2^20 elements, so that these
        # launches differ in grid size from the step's in a kernel trace)
        ("u32_out+8B", 4 * mis_n, 0, 1, lambda s: tk.tk_fill_u32(1, 0, mis_n, optr + 8)),
        ("normal_f64_out+8B", 8 * mis_n, 0, 2 if zig_kernels == 1 else zig_kernels,
         lambda s: tk.tk_fill_normal_f64(1, 0, mis_n, optr + 8)),
        # short fills (latency rows: 4 MiB and 8 MiB sit in the caches)
        ("u32_2^20", 4 * m20, 0, 1, lambda s: tk.tk_fill_u32(1, 0, m20, optr)),
        ("normal_f64_2^20", 8 * m20, 0, zig_kernels, lambda s: tk.tk_fill_normal_f64(1, st(s), m20, optr)),
        ("normal_f64_2^24", 8 * m24, 0, zig_kernels, lambda s: tk.tk_fill_normal_f64(1, st(s), m24, optr)),
    ]
    # not a fill: a plain copy of a known size, only when named with --only
    xc = x.view(torch.uint8)
    calib = ("calib_copy", 4 * n, 4 * n, 1, lambda s: out[:4 * n].copy_(xc))
    return fills, next_rows, calib, (out, x, table)


class FenceFreeEvent:
    """A HIP timing event created with hipEventDisableSystemFence and recorded on torch's
    current stream (the stream the fills are launched on).  torch's own events perform a
    system-scope fence when they are recorded, a cache writeback and invalidation between
    two kernels; these mark the same point in the stream without it, so the time between a
    pair is the launch's own.  The HIP runtime is the one libtk.so is linked against, the
    runtime torch loaded, reached through the library's handle."""
    FLAG = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)

    def __init__(self, hip):
        import ctypes as C
        self.C, self.hip = C, hip
        hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        hip.hipEventSynchronize.argtypes = [C.c_void_p]
        hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.e = C.c_void_p()
        self._check(hip.hipEventCreateWithFlags(C.byref(self.e), self.FLAG), "hipEventCreateWithFlags")

    @staticmethod
    def _check(code, what):
        if code != 0:
            raise RuntimeError(f"{what} failed: hipError {code}")

    def record(self):
        import torch
        self._check(self.hip.hipEventRecord(self.e, self.C.c_void_p(torch.cuda.current_stream().cuda_stream)),
                    "hipEventRecord")

    def elapsed_time(self, end):
        self._check(self.hip.hipEventSynchronize(end.e), "hipEventSynchronize")
        ms = self.C.c_float()
        self._check(self.hip.hipEventElapsedTime(self.C.byref(ms), self.e, end.e), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        if self.e:
            self.hip.hipEventDestroy(self.e)


def measured_traffic(fill):
    """HBM bytes per launch of `fill`'s kernel from the committed rocprofv3 counter record
    (FETCH_SIZE and WRITE_SIZE scaled by a copy-kernel calibration), or None when there is
    no record or the kernel's sources changed since the counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("kernels", {}).get(fill)
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:  # paths relative to the repository root
        path = os.path.join(here, f)
        if not os.path.exists(path):
            return None
        h.update(open(path, "rb").read())
    return rec["traffic_bytes"] if h.hexdigest() == rec["source_sha256"] else None


def cpu_baseline(n_sample):
    """The oracle (single-threaded C) over the same fills at n_sample elements each."""
    import oracle
    import tk_inputs as ti
    x = ti.normal_x(n_sample)
    q, a, _ = oracle.alias_build(ti.zipf_weights())
    m = n_sample
    jobs = [
        (4 * m, lambda: oracle.fill_u32(1, 0, m)), (8 * m, lambda: oracle.fill_u64(1, 0, m)),
        (4 * m, lambda: oracle.fill_f32(1, 0, m)), (8 * m, lambda: oracle.fill_f64(1, 0, m)),
        (2 * m, lambda: oracle.fill_u16(1, 0, m)), (2 * m, lambda: oracle.fill_f16_bits(1, 0, m)),
        (m, lambda: oracle.fill_u8(1, 0, m)), (m, lambda: oracle.fill_bool(1, 0, m)),
        (4 * m, lambda: oracle.fill_u32_below(1, 0, m, 1000)),
        (4 * m, lambda: oracle.fill_u32_below(1, 0, m, (1 << 32) - 2)),
        (8 * m, lambda: oracle.fill_u64_below(1, 0, m, 1000)),
        (8 * m, lambda: oracle.fill_u64_below(1, 0, m, (1 << 64) - 2)),
        (4 * m, lambda: oracle.fill_i32_below(1, 0, m, ti.LOW, ti.LOW_BOUND)),
        (8 * m, lambda: oracle.fill_i64_below32(1, 0, m, ti.LOW, ti.LOW_BOUND)),
        (8 * m, lambda: oracle.fill_normal_f64(1, 0, m)), (4 * m, lambda: oracle.fill_normal_f32(1, 0, m)),
        (4 * m, lambda: oracle.dropout_f32(ti.DROPOUT_KEY, 0, x, ti.DROPOUT_P, with_mask=False)),
        (4 * m, lambda: oracle.fill_choice_u32(1, 0, m, q, a)), (4 * m, lambda: oracle.philox_fill_u32(1, 0, m)),
    ]
    total_bytes, total_s = 0, 0.0
    for nbytes, fn in jobs:
        t0 = time.perf_counter()
        fn()
        total_s += time.perf_counter() - t0
        total_bytes += nbytes
    return {"value": total_bytes / total_s / GIB, "unit": "GiB/s", "cores": 1, "kind": "oracle",
            "sample": f"every fill of one step at 2^{int(np.log2(n_sample))} elements instead of 2^28 "
                      f"(single-threaded C oracle, {total_s:.1f} s)"}


def device_info():
    """What the numbers were measured on: device, architecture, compute units, HBM, HIP runtime."""
    import ctypes as C
    import torch
    import bulk_fills_amd as tk
    props = torch.cuda.get_device_properties(0)
    ver = C.c_int(0)
    tk.lib.hipRuntimeGetVersion.argtypes = [C.POINTER(C.c_int)]
    hip_rt = ver.value if tk.lib.hipRuntimeGetVersion(C.byref(ver)) == 0 else None
    return {"name": props.name, "gfx_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hbm_gib": round(props.total_memory / GIB, 1),
            "hip_runtime_version": hip_rt, "torch": torch.__version__, "torch_hip": torch.version.hip}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the fills shard with no communication, so only "
              "--gpus 1 is supported here", file=sys.stderr)
        sys.exit(2)
    import torch
    import bulk_fills_amd as tk
    import tk_inputs as ti

    n = ti.FULL_N
    fills, next_rows, calib, keep = build_step(tk, torch, n)
    if args.only:
        wanted = set(args.only.split(","))
        fills = [f for f in fills + next_rows + [calib] if f[0] in wanted]
        next_rows = []
    torch.cuda.synchronize()

    def step(s, events=None):
        # events: {fill index: (start, end)}; every other fill runs without instrumentation
        for j, (_, _, _, _, fn) in enumerate(fills):
            ev = events.get(j) if events is not None else None
            if ev is not None:
                ev[0].record()
            fn(s)
            if ev is not None:
                ev[1].record()

    t_end = time.perf_counter() + args.warmup_seconds
    w = 0
    while w < args.warmup or time.perf_counter() < t_end:
        step(w)
        w += 1
        if w % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    K = args.steps
    bytes_step = sum(f[1] for f in fills)

    def pairs():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    # per-fill pass, outside the timed region: an event pair around every fill of K steps
    evs = [{j: pairs() for j in range(len(fills))} for _ in range(K)]
    for s in range(K):
        step(s, evs[s])
    torch.cuda.synchronize()
    # and each fill K times back to back between one event pair (no event records between
    # its launches): the sustained time per fill, the figure its GiB/s is quoted on
    batch = []
    for j, f in enumerate(fills):
        a, b = pairs()
        a.record()
        for s in range(K):
            f[4](s)
        b.record()
        batch.append((a, b))
    torch.cuda.synchronize()
    per_fill = {}
    for j, (name, wbytes, rbytes, nk, _) in enumerate(fills):
        ms = [evs[s][j][0].elapsed_time(evs[s][j][1]) for s in range(K)]
        per_launch = batch[j][0].elapsed_time(batch[j][1]) / K
        per_fill[name] = {"median_ms": statistics.median(ms), "mean_ms": statistics.fmean(ms),
                          "batched_ms": per_launch, "GiB_per_s": wbytes / (per_launch / 1e3) / GIB,
                          "bytes_written": wbytes, "bytes_read": rbytes, "kernels": nk}
    # dominant single-kernel fill: the largest share of the step's device time
    single = {k: v for k, v in per_fill.items() if v["kernels"] == 1 and k != "calib_copy"}
    dom = max(single, key=lambda k: single[k]["mean_ms"])
    dj = [f[0] for f in fills].index(dom)

    # timed region: K steps; the only instrumentation is an event pair around the dominant
    # fill's launch, on the stream it is launched on (torch's current stream), without the
    # system-scope fence torch's events would add
    dev = [{dj: (FenceFreeEvent(tk.lib), FenceFreeEvent(tk.lib))} for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step(s, dev[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    elapsed = t1 - t0
    value = bytes_step * K / elapsed / GIB
    d = per_fill[dom]
    dom_ms = statistics.fmean(dev[s][dj][0].elapsed_time(dev[s][dj][1]) for s in range(K))
    algo_bytes = d["bytes_written"] + d["bytes_read"]
    achieved = algo_bytes / (dom_ms / 1e3) / 1e9
    traffic = measured_traffic(dom)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": round(traffic) if traffic is not None else None,
                "bytes_per_launch": algo_bytes, "avg_launch_ms": round(dom_ms, 5)}
    # rows beyond the hot path: same protocol, separate loop
    # (back to back as in the step: an event pair around each launch, one sync at the end)
    nxt = {}
    for name, wbytes, _, _, fn in next_rows:
        for s in range(3):
            fn(s)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for s in range(K):
            ev[s][0].record()
            fn(s)
            ev[s][1].record()
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        med = statistics.median(ms)
        nxt[name] = {"GiB_per_s": round(wbytes / (med / 1e3) / GIB, 1), "median_ms": round(med, 4),
                     "median_us": round(med * 1e3, 1)}
    cpu = cpu_baseline(1 << args.cpu_sample_log2) if args.cpu_sample_log2 > 0 else None

    rec = {
        "metric": "GiB/s written per fill (2^28 elems) on 1 MI355X; % of HBM write peak",
        "value": round(value, 2), "unit": "GiB/s", "n_gpus": 1, "steps": K, "warmup": w,
        "ms_per_step": round(elapsed / K * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": {"workload": "every hot-path fill once per step at 2^28 elements: uniform u8/u16/f16/u32/u64/"
                               "f32/f64/bool, bounded (Lemire) x6, ziggurat f64 normal, Box-Muller f32 normal, "
                               "dropout over f32[2^20,256], Zipf(1.1)x1000 choice, Philox u32",
                   "elements_per_fill": n, "fills_per_step": len(fills), "bytes_written_per_step": bytes_step},
        "pct_of_hbm_peak": round(100 * value * GIB / 1e9 / HBM_PEAK_GBS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fills": {k: {"GiB_per_s": round(v["GiB_per_s"], 1), "batched_ms": round(v["batched_ms"], 4),
                      "event_pair_median_ms": round(v["median_ms"], 4)} for k, v in per_fill.items()},
        "next_rows": nxt,
        "device": device_info(),
    }
    print(json.dumps(rec), flush=True)
    del keep


if __name__ == "__main__":
    main()
