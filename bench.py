"""Benchmark: GiB/s written by the counter-based bulk fills on one MI355X.

One step runs every fill of the hot path once at 2^28 elements (tandem-cuda,
"Performance", §GPU: 2^28 elements into device memory): the uniform fills (u8, u16,
f16 bits, u32, u64, f32, f64, bool; key and start draw cycle through 1..3 and 0, 1, 3
from step to step), the bounded fills (u32/u64 below 1000 and below 2^W - 2, int32 and
int64 with a low bound), the f64 ziggurat and f32 Box-Muller normals, fused dropout over
X = f32[2^20, 256] (p = 0.1), the choice fill through a 1000-way Zipf(1.1) alias table,
and the Philox4x32-10 u32 fill.  Inputs are resident in device memory before timing.

The JSON line reports the whole step's bytes written per second (`value`); each fill's
median and fastest of 21 event-timed launches after 2 s of warm-up per row (tandem-cuda,
"Performance", §GPU: 2 s of warm-up, the median of 21 fills, the fastest within a few
percent), as GiB/s and as a fraction of the 8 TB/s HBM peak and of the measured store
ceiling (the library's constant fill, which has the fills' store path and no generator,
and hipMemsetAsync, at each output size); per-start rows; the roofline of the dominant
kernel (algorithmic bytes per launch over its HIP-event-timed average duration); and the
CPU oracle timed on this host's cores over the same step.
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
# dependent integer steps per lane before each store of the constant fill, swept for the
# store ceiling (stores spaced by some arithmetic, as in the fills, can go faster than
# stores issued back to back), and dynamic LDS per work-group (fewer groups in flight per
# compute unit can also write faster)
CONST_WORK = (0, 12, 24, 32)
CONST_LDS = (0, 32768, 49152)
# a constant fill of MARKER_N words (one work-group, a grid no other launch has) right before
# and right after the timed steps, so that a kernel trace can pick out the timed region
TIMED_MARKER, MARKER_N = 0x7E57AB1E, 64


# ---- summaries of rocprofv3 output (run on the GPU host after a profiled bench) --------
# The kernel behind each fill's 2^28-element launch, by a prefix of its name in the
# profiler's records (the fill's launch is its kernel's largest grid).
FILL_KERNELS = {
    "normal_f64": "void tk::k_zig_table_pass<256, 4, true, false, true, false>",
    "dropout_f32": "void tk::k_vec_fill<tk::OpDropout, 1, true>",
    "u64": "void tk::k_vec_fill<tk::OpWord64<false>, 1, false>",
    "f64": "void tk::k_vec_fill<tk::OpWord64<true>, 1, false>",
    "u32": "void tk::k_vec_fill<tk::OpWord32<false>, 1, false>",
    "f16_bits": "void tk::k_vec_fill<tk::OpSub16<true>, 1, false>",
    "normal_f32": "void tk::k_vec_line<tk::OpNormalF32<false>, false>",
    "choice_u32": "void tk::k_choice<2, true, false, false>",
    "philox_u32": "void tk::k_philox_tile<tk::OpPhilox32<false>, false>",
    "exponential_f64": "void tk::k_exp_fill<tk::OpExpF64, 2, false>",
    "exponential_f32": "void tk::k_exp_fill<tk::OpExpF32, 2, false>",
    "calib_copy": "__amd_rocclr_copyBuffer",
    # store-only references, only when named with --only (2 GiB, one or four tiles per group)
    "constant_fill": "void tk::k_vec_fill<tk::OpConst, 1, false>",
    "constant_fill_tiles4": "void tk::k_vec_fill<tk::OpConst, 4, false>",
}
# Algorithmic bytes of each fill's 2^28-element launch (written + read) and the sources its
# kernel is built from (a traffic record holds only while they are unchanged).
_FILLS_SRC = ["bulk_fills_amd/csrc/tk_fills.hip", "bulk_fills_amd/csrc/tk_device.h", "bulk_fills_amd/csrc/tk_log.h",
              "bulk_fills_amd/csrc/logf256.inc", "bulk_fills_amd/csrc/log256.inc", "include/tk_device_api.h"]
FILL_SOURCES = {k: _FILLS_SRC for k in FILL_KERNELS}
FILL_SOURCES["normal_f64"] = ["bulk_fills_amd/csrc/tk_ziggurat.hip", "bulk_fills_amd/csrc/zig1024.inc",
                              "bulk_fills_amd/csrc/tk_device.h", "include/tk_device_api.h"]
FILL_SOURCES["choice_u32"] = ["bulk_fills_amd/csrc/tk_choice.hip", "bulk_fills_amd/csrc/tk_device.h",
                              "include/tk_device_api.h"]
_N28 = 1 << 28
FILL_BYTES = {"normal_f64": 8 * _N28, "dropout_f32": 8 * _N28, "u64": 8 * _N28, "f64": 8 * _N28, "u32": 4 * _N28,
              "f16_bits": 2 * _N28, "normal_f32": 4 * _N28, "choice_u32": 4 * _N28, "philox_u32": 4 * _N28,
              "exponential_f64": 8 * _N28, "exponential_f32": 4 * _N28, "calib_copy": 8 * _N28,
              "constant_fill": 8 * _N28, "constant_fill_tiles4": 8 * _N28}


def _csv_rows(d, suffix):
    import csv
    import glob
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def _sources_sha(files):
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(here, f), "rb").read())
    return h.hexdigest()


def trace_summary(d, min_share=0.0005, timed_only=False):
    """Markdown table of a --kernel-trace run: per kernel and grid size, calls and the
    duration statistics of its dispatches (End - Start timestamps).  With timed_only, only
    the dispatches between the two marker launches (the timed steps)."""
    rows = sorted(_csv_rows(d, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    if timed_only:
        marks = [i for i, r in enumerate(rows) if "OpConst" in r["Kernel_Name"] and int(r["Grid_Size_X"]) == 256]
        rows = rows[marks[-2] + 1:marks[-1]] if len(marks) >= 2 else []
    groups = {}
    for r in rows:
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        g = groups.setdefault((r["Kernel_Name"], grid), {"d": [], "vgpr": r["VGPR_Count"], "lds": r["LDS_Block_Size"]})
        g["d"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(g["d"]) for g in groups.values()) or 1.0
    out = ["| kernel | grid (threads) | calls | avg us | median us | min us | max us | VGPRs | LDS B | share |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for (name, grid), g in sorted(groups.items(), key=lambda kv: -sum(kv[1]["d"])):
        share = sum(g["d"]) / total
        if share < min_share:
            continue
        d_ = g["d"]
        out.append(f"| `{name[:110]}` | {grid} | {len(d_)} | {statistics.fmean(d_):.2f} | {statistics.median(d_):.2f} | "
                   f"{min(d_):.2f} | {max(d_):.2f} | {g['vgpr']} | {g['lds']} | {100 * share:.1f}% |")
    return "\n".join(out)


def _counter_medians(d):
    """{(kernel, grid): {counter: median value over the dispatches}} from a --pmc run."""
    vals = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        key = (r["Kernel_Name"], int(r["Grid_Size"]))
        vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: {c: statistics.median(v) for c, v in cs.items()} for k, cs in vals.items()}


def _fill_launch(meds, fill):
    """The counters of a fill's 2^28-element launch: its kernel's largest grid."""
    keys = [k for k in meds if k[0].startswith(FILL_KERNELS[fill])]
    return meds[max(keys, key=lambda k: k[1])] if keys else None


def pmc_summary(fetch_dir, write_dir, out_json):
    """HBM bytes per launch from a FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch),
    scaled by what the same counters read for a plain 1 GiB device copy; writes the record
    bench.py takes `traffic` from and returns a markdown table."""
    fetch, write = _counter_medians(fetch_dir), _counter_medians(write_dir)
    cf, cw = _fill_launch(fetch, "calib_copy"), _fill_launch(write, "calib_copy")
    copy_kib = float(FILL_BYTES["calib_copy"] // 2 // 1024)  # 1 GiB read and 1 GiB written
    ff, wf = copy_kib / cf["FETCH_SIZE"], copy_kib / cw["WRITE_SIZE"]
    rec = {"fetch_factor": ff, "write_factor": wf, "calibration": "1 GiB device copy (__amd_rocclr_copyBuffer)",
           "kernels": {}}
    out = [f"Calibration: a 1 GiB device copy reads FETCH_SIZE {cf['FETCH_SIZE']:.1f} KiB and WRITE_SIZE "
           f"{cw['WRITE_SIZE']:.1f} KiB per dispatch: fetch factor {ff:.4f}, write factor {wf:.4f}.", "",
           "| fill | kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM bytes | algorithmic bytes | ratio |",
           "|---|---|---|---|---|---|---|"]
    for fill in FILL_KERNELS:
        if fill == "calib_copy":
            continue
        f_, w_ = _fill_launch(fetch, fill), _fill_launch(write, fill)
        if not f_ or not w_:
            continue
        traffic = f_["FETCH_SIZE"] * 1024 * ff + w_["WRITE_SIZE"] * 1024 * wf
        algo = FILL_BYTES[fill]
        rec["kernels"][fill] = {"kernel": FILL_KERNELS[fill], "fetch_kib": f_["FETCH_SIZE"], "write_kib": w_["WRITE_SIZE"],
                                "traffic_bytes": traffic, "algorithmic_bytes": algo, "sources": FILL_SOURCES[fill],
                                "source_sha256": _sources_sha(FILL_SOURCES[fill])}
        out.append(f"| {fill} | `{FILL_KERNELS[fill]}` | {f_['FETCH_SIZE']:.1f} | {w_['WRITE_SIZE']:.1f} | "
                   f"{traffic:.4g} | {algo:.4g} | {traffic / algo:.4f} |")
    with open(out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
    return "\n".join(out)


def counter_summary(d):
    """Markdown table of the per-dispatch counters of a --pmc run, per fill (median over the
    fill's 2^28-element dispatches; SQ_* per wave where SQ_WAVES was collected)."""
    meds = _counter_medians(d)
    rows = [(f, _fill_launch(meds, f)) for f in FILL_KERNELS if f != "calib_copy"]
    rows = [(f, c) for f, c in rows if c]
    names = sorted({k for _, c in rows for k in c})
    out = ["| fill | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    for f, c in rows:
        waves = c.get("SQ_WAVES")
        cells = []
        for k in names:
            v = c.get(k)
            if v is None:
                cells.append("")
            elif waves and k.startswith("SQ_INSTS"):
                cells.append(f"{v / waves:.1f} / wave")
            else:
                cells.append(f"{v:.4g}")
        out.append(f"| {f} | " + " | ".join(cells) + " |")
    return "\n".join(out)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5, help="untimed steps before the timed ones")
    ap.add_argument("--row-warmup-seconds", type=float, default=2.0,
                    help="warm-up of each hot-path row before its 21 timed launches (the pages warm each "
                         "row for 2 s); rows outside the step get a quarter of it")
    ap.add_argument("--row-launches", type=int, default=21, help="timed launches per row")
    ap.add_argument("--cpu-single-log2", type=int, default=26,
                    help="elements per fill in the one-core oracle sample (0: skip it)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print the kernel-trace summary of a rocprofv3 --kernel-trace output directory and exit")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_JSON"),
                    help="HBM bytes per launch from FETCH_SIZE and WRITE_SIZE rocprofv3 runs: write the traffic "
                         "record and print its table, then exit")
    ap.add_argument("--counter-summary", metavar="DIR",
                    help="print the per-fill counters of a rocprofv3 --pmc output directory and exit")
    ap.add_argument("--only", default="",
                    help="comma-separated fill names to run (profiling); 'calib_copy' adds a plain 1 GiB "
                         "device copy used to calibrate the HBM byte counters, 'constant_fill' and "
                         "'constant_fill_tiles4' the 2 GiB store-only fill at one and four tiles per group")
    return ap.parse_args()


def build_step(tk, torch, n):
    """Returns the step's fills and the rows outside it, each (name, bytes_written,
    bytes_read, kernels, fn(step_index)); the per-start rows and the store-ceiling rows;
    and the buffers they use."""
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
    # not fills: a plain copy of a known size and the store-only constant fill at one and four
    # tiles per group, only when named with --only
    xc = x.view(torch.uint8)
    def const_tiles4(s):
        tk.tk_debug_set_tunable("unroll", 4)
        try:
            tk.tk_fill_constant_u32(0, 2 * n, optr)
        finally:
            tk.tk_debug_set_tunable("unroll", -1)
    calib = [("calib_copy", 4 * n, 4 * n, 1, lambda s: out[:4 * n].copy_(xc)),
             ("constant_fill", 8 * n, 0, 1, lambda s: tk.tk_fill_constant_u32(0, 2 * n, optr)),
             ("constant_fill_tiles4", 8 * n, 0, 1, const_tiles4)]

    # one row per start draw: (fill, start, bytes written, fn)
    def at(fill, nb, f):
        return [(fill, s0, nb, (lambda s0: lambda s: f(s0))(s0)) for s0 in starts[fill]]
    starts = {"normal_f64": (0, 1, 3), "normal_f64_2^24": (0, 1, 3), "philox_u32": (0, 1, 2, 3),
              "normal_f32": (0, 1, 3), "normal_f32_half_turn": (0, 1), "u16": (0, 1), "f16_bits": (0, 1),
              "u8": (0, 1, 3), "philox_normal_f32": (0, 1, 2, 3)}
    start_rows = (at("normal_f64", 8 * n, lambda s0: tk.tk_fill_normal_f64(1, s0, n, optr))
                  + at("normal_f64_2^24", 8 * m24, lambda s0: tk.tk_fill_normal_f64(1, s0, m24, optr))
                  + at("philox_u32", 4 * n, lambda s0: tk.tk_philox_fill_u32(1, s0, n, optr))
                  + at("normal_f32", 4 * n, lambda s0: tk.tk_fill_normal_f32(1, s0, n, optr))
                  + at("normal_f32_half_turn", 4 * n, lambda s0: tk.tk_fill_normal_f32_half_turn(1, s0, n, optr))
                  + at("u16", 2 * n, lambda s0: tk.tk_fill_u16(1, s0, n, optr))
                  + at("f16_bits", 2 * n, lambda s0: tk.tk_fill_f16_bits(1, s0, n, optr))
                  + at("u8", n, lambda s0: tk.tk_fill_u8(1, s0, n, optr))
                  + at("philox_normal_f32", 4 * n, lambda s0: tk.tk_philox_fill_normal_f32(1, s0, n, optr)))

    # the store ceiling at every output size of the step: the library's constant fill (the
    # fills' own store path, no generator) and the runtime's hipMemsetAsync
    import ctypes as C
    hip = tk.lib
    hip.hipMemsetAsync.argtypes = [C.c_void_p, C.c_int, C.c_size_t, C.c_void_p]
    hip.hipMemsetAsync.restype = C.c_int

    def memset(nb):
        rc = hip.hipMemsetAsync(optr, 0, nb, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipMemsetAsync failed: hipError {rc}")
    def const_fill(nb, work, lds):
        def f(s):
            tk.tk_debug_set_tunable("const_work", work)
            tk.tk_debug_set_tunable("lds_pad", lds)
            try:
                tk.tk_fill_constant_u32(0, nb // 4, optr)
            finally:
                tk.tk_debug_set_tunable("const_work", -1)
                tk.tk_debug_set_tunable("lds_pad", -1)
        return f
    ceil_rows = []
    for nb in (n, 2 * n, 4 * n, 8 * n):
        for work in CONST_WORK:
            for lds in CONST_LDS:
                ceil_rows.append((f"constant_fill_work{work}_lds{lds >> 10}k", nb, const_fill(nb, work, lds)))
        ceil_rows.append(("hipMemsetAsync", nb, (lambda nb: lambda s: memset(nb))(nb)))
    # the store pattern, 2 GiB: consecutive 4 KiB tiles per work-group (one, two or four),
    # a capped grid whose groups stride over the output, for the constant fill, the f64
    # fill and the ziggurat (whose table pass runs four tiles per group)
    def tuned(fn, **tunables):
        def f(s):
            for k, v in tunables.items():
                tk.tk_debug_set_tunable(k, v)
            try:
                fn(s)
            finally:
                for k in tunables:
                    tk.tk_debug_set_tunable(k, -1)
        return f
    c2 = lambda s: tk.tk_fill_constant_u32(0, 2 * n, optr)
    f64 = lambda s: tk.tk_fill_f64(1, 0, n, optr)
    zig = lambda s: tk.tk_fill_normal_f64(1, 0, n, optr)
    pattern_rows = [("constant_fill", 8 * n, c2), ("constant_fill tiles=2", 8 * n, tuned(c2, unroll=2)),
                    ("constant_fill tiles=4", 8 * n, tuned(c2, unroll=4)),
                    ("constant_fill grid=8192", 8 * n, tuned(c2, max_blocks=8192)),
                    ("f64", 8 * n, f64), ("f64 tiles=4", 8 * n, tuned(f64, unroll=4)),
                    # the integer fills' LDS cap on resident groups against none
                    ("u64", 8 * n, lambda s: tk.tk_fill_u64(1, 0, n, optr)),
                    ("u64 uncapped", 8 * n, tuned(lambda s: tk.tk_fill_u64(1, 0, n, optr), lds_pad=0)),
                    ("u32", 4 * n, lambda s: tk.tk_fill_u32(1, 0, n, optr)),
                    ("u32 uncapped", 4 * n, tuned(lambda s: tk.tk_fill_u32(1, 0, n, optr), lds_pad=0)),
                    ("normal_f64 tiles=2", 8 * n, tuned(zig, zig_tiles=2)),
                    ("normal_f64 tiles=4", 8 * n, tuned(zig, zig_tiles=4)),
                    ("normal_f64 tiles=8", 8 * n, tuned(zig, zig_tiles=8)),
                    # Philox at word offsets 1..3: the LDS tile kernel (default) against the
                    # overlapping-wave kernel; start 0 is the direct kernel
                    ("philox_u32 start 0 direct", 4 * n, lambda s: tk.tk_philox_fill_u32(1, 0, n, optr)),
                    ("philox_u32 start 1 tile", 4 * n, lambda s: tk.tk_philox_fill_u32(1, 1, n, optr)),
                    ("philox_u32 start 1 overlap", 4 * n,
                     tuned(lambda s: tk.tk_philox_fill_u32(1, 1, n, optr), philox_lds=0)),
                    ("philox_u64_below_1000 start 1 tile", 8 * n,
                     lambda s: tk.tk_philox_fill_u64_below(1, 1, n, 1000, optr)),
                    ("philox_u64_below_1000 start 1 overlap", 8 * n,
                     tuned(lambda s: tk.tk_philox_fill_u64_below(1, 1, n, 1000, optr), philox_lds=0))]
    return fills, next_rows, calib, start_rows, ceil_rows, pattern_rows, (out, x, table)


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


def _oracle_jobs(x):
    """(fill name, bytes written per element, fn(start, n)) for every fill of one step, over
    the oracle.
    x: the dropout input of at least as many elements as the largest call."""
    import oracle
    import tk_inputs as ti
    q, a, _ = oracle.alias_build(ti.zipf_weights())
    L, LB = ti.LOW, ti.LOW_BOUND
    return [
        ("u32", 4, lambda s, m: oracle.fill_u32(1, s, m)), ("u64", 8, lambda s, m: oracle.fill_u64(1, s, m)),
        ("f32", 4, lambda s, m: oracle.fill_f32(1, s, m)), ("f64", 8, lambda s, m: oracle.fill_f64(1, s, m)),
        ("u16", 2, lambda s, m: oracle.fill_u16(1, s, m)),
        ("f16_bits", 2, lambda s, m: oracle.fill_f16_bits(1, s, m)),
        ("u8", 1, lambda s, m: oracle.fill_u8(1, s, m)), ("bool", 1, lambda s, m: oracle.fill_bool(1, s, m)),
        ("u32_below_1000", 4, lambda s, m: oracle.fill_u32_below(1, s, m, 1000)),
        ("u32_below_2^32-2", 4, lambda s, m: oracle.fill_u32_below(1, s, m, (1 << 32) - 2)),
        ("u64_below_1000", 8, lambda s, m: oracle.fill_u64_below(1, s, m, 1000)),
        ("u64_below_2^64-2", 8, lambda s, m: oracle.fill_u64_below(1, s, m, (1 << 64) - 2)),
        ("i32_below_low", 4, lambda s, m: oracle.fill_i32_below(1, s, m, L, LB)),
        ("i64_below32_low", 8, lambda s, m: oracle.fill_i64_below32(1, s, m, L, LB)),
        ("normal_f64", 8, lambda s, m: oracle.fill_normal_f64(1, s, m)),
        ("normal_f32", 4, lambda s, m: oracle.fill_normal_f32(1, s, m)),
        ("dropout_f32", 4,
         lambda s, m: oracle.dropout_f32(ti.DROPOUT_KEY, s, x[s:s + m], ti.DROPOUT_P, with_mask=False)),
        ("choice_u32", 4, lambda s, m: oracle.fill_choice_u32(1, s, m, q, a)),
        ("philox_u32", 4, lambda s, m: oracle.philox_fill_u32(1, s, m)),
    ]


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_threads():
    """Threads for the all-core oracle run: the CPUs this process may use, at most 16 (one
    GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(n_full, single_log2):
    """The oracle (plain single-threaded C, untouched) over every fill of one step.
    All cores: each fill at the full n_full elements, cut into P contiguous ranges run on P
    threads at once (a fill cut at any element equals the whole fill; ctypes releases the
    GIL during each call).  One core: each fill at 2^single_log2 elements, one call."""
    import tk_inputs as ti
    from concurrent.futures import ThreadPoolExecutor
    P = host_threads()
    x = ti.normal_x(n_full)
    jobs = _oracle_jobs(x)
    cut = [(n_full * j) // P for j in range(P + 1)]
    total_bytes, total_s = 0, 0.0
    per_fill = {}
    with ThreadPoolExecutor(P) as pool:
        for name, nb, fn in jobs:
            t0 = time.perf_counter()
            list(pool.map(lambda j: fn(cut[j], cut[j + 1] - cut[j]) is None, range(P)))
            dt = time.perf_counter() - t0
            per_fill[name] = {"all_cores_s": round(dt, 4)}
            total_s += dt
            total_bytes += nb * n_full
    rec = {"value": round(total_bytes / total_s / GIB, 3), "unit": "GiB/s", "cores": P, "kind": "oracle",
           "sample": f"every fill of one step at the full 2^{int(np.log2(n_full))} elements, each cut into {P} "
                     f"contiguous ranges on {P} threads ({total_s:.1f} s wall)",
           "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
    if single_log2 > 0:
        m = 1 << single_log2
        b1, s1 = 0, 0.0
        for name, nb, fn in jobs:
            t0 = time.perf_counter()
            fn(0, m)
            dt = time.perf_counter() - t0
            # one core's time for the whole 2^n_full fill, scaled from the sample
            per_fill[name]["single_core_s_scaled"] = round(dt * n_full / m, 3)
            s1 += dt
            b1 += nb * m
        rec["single_core"] = {"value": round(b1 / s1 / GIB, 3), "unit": "GiB/s", "cores": 1,
                              "sample": f"every fill of one step at 2^{single_log2} elements, one thread "
                                        f"({s1:.1f} s)"}
    rec["per_fill"] = per_fill
    return rec


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


class ClockSampler:
    """Samples the GPU's shader and memory clocks every `period` seconds while the per-fill
    rows run, so the line records the clocks the fills ran at.  Reads the driver's
    pp_dpm_sclk / pp_dpm_mclk files under /sys/class/drm (the line marked '*' is the current
    level; file reads only, no child process).  Leaves `result` None when they are absent."""

    def __init__(self, period=0.25):
        import glob
        import threading
        self.period, self.samples, self.result = period, {"sclk": [], "mclk": []}, None
        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.dev = os.path.dirname(cards[0]) if cards else None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _sample(self):
        import re
        for clk in ("sclk", "mclk"):
            try:
                lines = open(os.path.join(self.dev, f"pp_dpm_{clk}")).read().splitlines()
            except OSError:
                return False
            for line in lines:
                m = re.search(r"(\d+)\s*mhz\s*\*", line, re.I)
                if m:
                    self.samples[clk].append(int(m.group(1)))
        return True

    def _run(self):
        while self.dev and not self._stop.is_set():
            if not self._sample():
                return
            self._stop.wait(self.period)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=5)
        res = {}
        for clk, v in self.samples.items():
            if v:
                res[f"{clk}_mhz"] = {"min": min(v), "median": statistics.median(v), "max": max(v), "samples": len(v)}
        self.result = res or None
        return False


class RowTimer:
    """Times launches of one row: a warm-up of at least `warm_s` seconds, then `k` launches
    each between a pair of fence-free events recorded on the launch stream (back to back:
    no synchronisation between them), then the same k launches between a single pair."""

    def __init__(self, tk, torch, k):
        self.tk, self.torch, self.k = tk, torch, k
        self.ev = [(FenceFreeEvent(tk.lib), FenceFreeEvent(tk.lib)) for _ in range(k)]
        self.batch = (FenceFreeEvent(tk.lib), FenceFreeEvent(tk.lib))

    def time(self, fn, warm_s):
        torch = self.torch
        t_end = time.perf_counter() + warm_s
        w = 0
        while True:
            fn(w)
            w += 1
            if w % 8 == 0:
                torch.cuda.synchronize()
                if time.perf_counter() >= t_end:
                    break
        for s, (a, b) in enumerate(self.ev):
            a.record()
            fn(s)
            b.record()
        self.batch[0].record()
        for s in range(self.k):
            fn(s)
        self.batch[1].record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in self.ev)
        return {"median_ms": statistics.median(ms), "min_ms": ms[0], "max_ms": ms[-1],
                "batched_ms": self.batch[0].elapsed_time(self.batch[1]) / self.k, "warmup_launches": w}


def progress(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def rate(nbytes, ms):
    return nbytes / (ms / 1e3) / GIB


def main():
    args = parse()
    if args.trace_summary:
        print("All dispatches:\n")
        print(trace_summary(args.trace_summary))
        print("\nThe timed steps only (between the two marker launches):\n")
        print(trace_summary(args.trace_summary, min_share=0.0, timed_only=True))
        return
    if args.pmc_summary:
        print(pmc_summary(*args.pmc_summary))
        return
    if args.counter_summary:
        print(counter_summary(args.counter_summary))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the fills shard with no communication, so only "
              "--gpus 1 is supported here", file=sys.stderr)
        sys.exit(2)
    import torch
    import bulk_fills_amd as tk
    import tk_inputs as ti

    n = ti.FULL_N
    fills, next_rows, calib, start_rows, ceil_rows, pattern_rows, keep = build_step(tk, torch, n)
    if args.only:
        wanted = set(args.only.split(","))
        fills = [f for f in fills + next_rows + calib if f[0] in wanted]
        next_rows, start_rows, ceil_rows, pattern_rows = [], [], [], []
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

    # warm-up: exactly W untimed steps
    for w in range(args.warmup):
        step(w)
    torch.cuda.synchronize()

    K = args.steps
    R = args.row_launches
    bytes_step = sum(f[1] for f in fills)
    rt = RowTimer(tk, torch, R)
    warm = args.row_warmup_seconds

    # store ceiling first, so that every fill can be set against it
    ceiling = {}
    for name, nb, fn in ceil_rows:
        t = rt.time(fn, warm / 4)
        progress(f"ceiling {name} {nb >> 20} MiB: {t['median_ms'] * 1e3:.1f} us")
        ceiling.setdefault(name, {})[str(nb)] = {
            "GiB_per_s": round(rate(nb, t["median_ms"]), 1), "GiB_per_s_fastest": round(rate(nb, t["min_ms"]), 1),
            "median_us": round(t["median_ms"] * 1e3, 2), "min_us": round(t["min_ms"] * 1e3, 2)}

    def ceiling_at(nb):
        c = [ceiling[k][str(nb)]["GiB_per_s"] for k in ceiling if str(nb) in ceiling[k]]
        return max(c) if c else None

    # per output size: the fastest store-only kernel (median of its launches) and which it was
    ceiling_best = {}
    for k, per in ceiling.items():
        for nb, r in per.items():
            if nb not in ceiling_best or r["GiB_per_s"] > ceiling_best[nb]["GiB_per_s"]:
                ceiling_best[nb] = {"GiB_per_s": r["GiB_per_s"], "kernel": k,
                                    "pct_of_hbm_peak": round(100 * r["GiB_per_s"] * GIB / 1e9 / HBM_PEAK_GBS, 2)}

    def row_record(nb, rbytes, t):
        rec = {"GiB_per_s": round(rate(nb, t["median_ms"]), 1),
               "GiB_per_s_fastest": round(rate(nb, t["min_ms"]), 1),
               "median_us": round(t["median_ms"] * 1e3, 2), "min_us": round(t["min_ms"] * 1e3, 2),
               "batched_us": round(t["batched_ms"] * 1e3, 2),
               "pct_of_hbm_peak": round(100 * (nb + rbytes) / (t["median_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 2)}
        c = ceiling_at(nb)
        if c and not rbytes:
            rec["pct_of_store_ceiling"] = round(100 * rec["GiB_per_s"] / c, 2)
        return rec

    # per-fill pass, outside the timed region: warm-up, then 21 event-timed launches per row
    # (the clocks are sampled meanwhile)
    per_fill = {}
    with ClockSampler() as clocks:
        for name, wbytes, rbytes, nk, fn in fills:
            t = rt.time(fn, warm)
            progress(f"{name}: {t['median_ms'] * 1e3:.1f} us")
            per_fill[name] = dict(row_record(wbytes, rbytes, t), bytes_written=wbytes, bytes_read=rbytes, kernels=nk,
                                  _median_ms=t["median_ms"])
    # dominant single-kernel fill: the largest share of the step's device time
    single = {k: v for k, v in per_fill.items() if v["kernels"] == 1 and k != "calib_copy"}
    dom = max(single, key=lambda k: single[k]["_median_ms"])
    dj = [f[0] for f in fills].index(dom)

    # timed region: K steps; the only instrumentation is an event pair around the dominant
    # fill's launch, on the stream it is launched on (torch's current stream), without the
    # system-scope fence torch's events would add
    dev = [{dj: (FenceFreeEvent(tk.lib), FenceFreeEvent(tk.lib))} for _ in range(K)]
    marker = keep[0].data_ptr()
    tk.tk_fill_constant_u32(TIMED_MARKER, MARKER_N, marker)  # marks the timed region in a kernel trace
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step(s, dev[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tk.tk_fill_constant_u32(TIMED_MARKER, MARKER_N, marker)
    torch.cuda.synchronize()

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
    c_dom = ceiling_at(d["bytes_written"])
    if c_dom:
        roofline["frac_of_store_ceiling"] = round(algo_bytes / (dom_ms / 1e3) / GIB / c_dom, 4)

    # rows beyond the hot path and per-start rows: same protocol, a shorter warm-up
    progress(f"timed steps: {elapsed / K * 1e3:.3f} ms per step")
    nxt = {}
    for name, wbytes, rbytes, _, fn in next_rows:
        nxt[name] = row_record(wbytes, rbytes, rt.time(fn, warm / 4))
        progress(f"{name}: {nxt[name]['median_us']} us")
    per_start = {}
    for fill, s0, nb, fn in start_rows:
        per_start.setdefault(fill, {})[str(s0)] = r = row_record(nb, 0, rt.time(fn, warm / 4))
        progress(f"{fill} start {s0}: {r['median_us']} us")

    store_pattern = {}
    for name, nb, fn in pattern_rows:
        r = rt.time(fn, warm / 4)
        store_pattern[name] = {"GiB_per_s": round(rate(nb, r["median_ms"]), 1),
                               "median_us": round(r["median_ms"] * 1e3, 2), "min_us": round(r["min_ms"] * 1e3, 2)}
        progress(f"store pattern {name}: {store_pattern[name]['median_us']} us")

    cpu = None
    if not args.no_cpu:
        progress("CPU oracle baseline")
        cpu = cpu_baseline(n, args.cpu_single_log2)

    for v in per_fill.values():
        del v["_median_ms"]
    rec = {
        "metric": "GiB/s written per fill (2^28 elems) on 1 MI355X; % of HBM write peak",
        "value": round(value, 2), "unit": "GiB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(elapsed / K * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "per fill: u8/u16/u32/u64 integers, f16/f32/f64", "data": "synthetic",
        "config": {"workload": "every hot-path fill once per step at 2^28 elements: uniform u8/u16/f16/u32/u64/"
                               "f32/f64/bool, bounded (Lemire) x6, ziggurat f64 normal, Box-Muller f32 normal, "
                               "dropout over f32[2^20,256], Zipf(1.1)x1000 choice, Philox u32",
                   "elements_per_fill": n, "fills_per_step": len(fills), "bytes_written_per_step": bytes_step},
        "pct_of_hbm_peak": round(100 * value * GIB / 1e9 / HBM_PEAK_GBS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "protocol": {"warmup_steps": args.warmup, "row_warmup_s": warm, "row_warmup_s_outside_step": warm / 4,
                     "row_launches": R, "row_statistic": "median and fastest of the row launches, each between "
                     "fence-free HIP events; batched_us = the same launches back to back between one pair"},
        "store_ceiling": {"best": ceiling_best, "rows": ceiling},
        "fills": per_fill,
        "per_start": per_start,
        "store_pattern": store_pattern,
        "next_rows": nxt,
        "device": dict(device_info(), clocks_during_fill_rows=clocks.result),
    }
    print(json.dumps(rec), flush=True)
    del keep


if __name__ == "__main__":
    main()
