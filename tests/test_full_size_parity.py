"""Every element of each fill family at the measured size (2^28 elements, the benchmark's
launch configuration and an aligned output) compared with the oracle.

The device fills the whole output in one call.  The oracle computes it in 256 MiB pieces,
each one call with its own start draw and length (a fill cut at any element equals the
whole fill: tandem-sycl, "Design", §Fills and §Normals), several pieces at once on host
threads.  Tolerances are those of the smaller parity tests: bit-exact for integers,
uniforms, bounded, choice, dropout (y and mask), exponential f32 and the ziggurat's
fast-path and wedge values; ziggurat tail values within 1e-12 relative; Box-Muller f32
within 4e-6 absolute; exponential f64 within 2 ulp.  The canary bytes around the output
are checked too.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import DevBuf, first_mismatch, log

pytestmark = pytest.mark.gpu

N = tk_inputs.FULL_N
CHUNK_BYTES = 256 << 20
TAIL_REL = 1e-12
F32_ABS = 4e-6
EXP_F64_ULP = 2


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_pool = None


def pool():
    global _pool
    if _pool is None:
        _pool = ThreadPoolExecutor(_threads())
    return _pool


_alias = None


def alias():
    """The library's table over the workload's Zipf weights, and the oracle's own build of
    it (the library's host build equals the oracle's: checked here once more)."""
    global _alias
    if _alias is None:
        w = tk_inputs.zipf_weights()
        table = tk.tk_alias_create(w)
        q, a, _ = oracle.alias_build(w)
        tq, ta = table.export()
        assert np.array_equal(tq, q) and np.array_equal(ta, a), "alias tables differ"
        _alias = (table, q, a)
    return _alias


L, LB = tk_inputs.LOW, tk_inputs.LOW_BOUND
TOP32, TOP64 = (1 << 32) - 2, (1 << 64) - 2

# name -> (device fill(out), oracle(start, m), numpy dtype, start draw, comparison)
FAMILIES = {
    "u8": (lambda o: tk.tk_fill_u8(1, 3, N, o), lambda s, m: oracle.fill_u8(1, s, m), np.uint8, 3, "bits"),
    "u16": (lambda o: tk.tk_fill_u16(1, 3, N, o), lambda s, m: oracle.fill_u16(1, s, m), np.uint16, 3, "bits"),
    "f16_bits": (lambda o: tk.tk_fill_f16_bits(1, 3, N, o), lambda s, m: oracle.fill_f16_bits(1, s, m),
                 np.uint16, 3, "bits"),
    "u32": (lambda o: tk.tk_fill_u32(2, 1, N, o), lambda s, m: oracle.fill_u32(2, s, m), np.uint32, 1, "bits"),
    "u64": (lambda o: tk.tk_fill_u64(2, 1, N, o), lambda s, m: oracle.fill_u64(2, s, m), np.uint64, 1, "bits"),
    "f32": (lambda o: tk.tk_fill_f32(3, 1, N, o), lambda s, m: oracle.fill_f32(3, s, m), np.float32, 1, "bits"),
    "f64": (lambda o: tk.tk_fill_f64(3, 3, N, o), lambda s, m: oracle.fill_f64(3, s, m), np.float64, 3, "bits"),
    "bool": (lambda o: tk.tk_fill_bool(1, 3, N, o), lambda s, m: oracle.fill_bool(1, s, m), np.uint8, 3, "bits"),
    "u32_below_1000": (lambda o: tk.tk_fill_u32_below(1, 0, N, 1000, o),
                       lambda s, m: oracle.fill_u32_below(1, s, m, 1000), np.uint32, 0, "bits"),
    "u32_below_2^32-2": (lambda o: tk.tk_fill_u32_below(1, 0, N, TOP32, o),
                         lambda s, m: oracle.fill_u32_below(1, s, m, TOP32), np.uint32, 0, "bits"),
    "u64_below_1000": (lambda o: tk.tk_fill_u64_below(1, 0, N, 1000, o),
                       lambda s, m: oracle.fill_u64_below(1, s, m, 1000), np.uint64, 0, "bits"),
    "u64_below_2^64-2": (lambda o: tk.tk_fill_u64_below(1, 0, N, TOP64, o),
                         lambda s, m: oracle.fill_u64_below(1, s, m, TOP64), np.uint64, 0, "bits"),
    "i32_below_low": (lambda o: tk.tk_fill_i32_below(1, 0, N, L, LB, o),
                      lambda s, m: oracle.fill_i32_below(1, s, m, L, LB), np.int32, 0, "bits"),
    "i64_below32_low": (lambda o: tk.tk_fill_i64_below32(1, 0, N, L, LB, o),
                        lambda s, m: oracle.fill_i64_below32(1, s, m, L, LB), np.int64, 0, "bits"),
    "i64_below_low": (lambda o: tk.tk_fill_i64_below(1, 0, N, L, LB, o),
                      lambda s, m: oracle.fill_i64_below(1, s, m, L, LB), np.int64, 0, "bits"),
    "normal_f64": (lambda o: tk.tk_fill_normal_f64(1, 3, N, o),
                   lambda s, m: oracle.fill_normal_f64(1, s, m, with_path=True), np.float64, 3, "ziggurat"),
    "normal_f32": (lambda o: tk.tk_fill_normal_f32(1, 1, N, o), lambda s, m: oracle.fill_normal_f32(1, s, m),
                   np.float32, 1, "f32abs"),
    "normal_f32_half_turn": (lambda o: tk.tk_fill_normal_f32_half_turn(1, 3, N, o),
                             lambda s, m: oracle.fill_normal_f32_half_turn(1, s, m), np.float32, 3, "f32abs"),
    "randn_f32": (lambda o: tk.tk_fill_randn_f32(1, 0, N, o), lambda s, m: oracle.fill_randn_f32(1, s, m),
                  np.float32, 0, "f32abs"),
    "exponential_f64": (lambda o: tk.tk_fill_exponential_f64(1, 3, N, o),
                        lambda s, m: oracle.fill_exponential_f64(1, s, m), np.float64, 3, "ulp"),
    "exponential_f32": (lambda o: tk.tk_fill_exponential_f32(1, 3, N, o),
                        lambda s, m: oracle.fill_exponential_f32(1, s, m), np.float32, 3, "bits"),
    "choice_u32": (lambda o: tk.tk_fill_choice_u32(1, 0, N, alias()[0], o),
                   lambda s, m: oracle.fill_choice_u32(1, s, m, alias()[1], alias()[2]), np.uint32, 0, "bits"),
    "philox_u32": (lambda o: tk.tk_philox_fill_u32(1, 1, N, o), lambda s, m: oracle.philox_fill_u32(1, s, m),
                   np.uint32, 1, "bits"),
    "philox_u64": (lambda o: tk.tk_philox_fill_u64(1, 3, N, o), lambda s, m: oracle.philox_fill_u64(1, s, m),
                   np.uint64, 3, "bits"),
    "philox_f32": (lambda o: tk.tk_philox_fill_f32(1, 2, N, o), lambda s, m: oracle.philox_fill_f32(1, s, m),
                   np.float32, 2, "bits"),
    "philox_f64": (lambda o: tk.tk_philox_fill_f64(1, 0, N, o), lambda s, m: oracle.philox_fill_f64(1, s, m),
                   np.float64, 0, "bits"),
    "philox_u32_below_1000": (lambda o: tk.tk_philox_fill_u32_below(1, 3, N, 1000, o),
                              lambda s, m: oracle.philox_fill_u32_below(1, s, m, 1000), np.uint32, 3, "bits"),
    "philox_u64_below_1000": (lambda o: tk.tk_philox_fill_u64_below(1, 1, N, 1000, o),
                              lambda s, m: oracle.philox_fill_u64_below(1, s, m, 1000), np.uint64, 1, "bits"),
    "philox_choice_u32": (lambda o: tk.tk_philox_fill_choice_u32(1, 0, N, alias()[0], o),
                          lambda s, m: oracle.philox_fill_choice_u32(1, s, m, alias()[1], alias()[2]),
                          np.uint32, 0, "bits"),
    "philox_normal_f32": (lambda o: tk.tk_philox_fill_normal_f32(1, 1, N, o),
                          lambda s, m: oracle.philox_fill_normal_f32(1, s, m), np.float32, 1, "f32abs"),
    "philox_normal_f64": (lambda o: tk.tk_philox_fill_normal_f64(1, 3, N, o),
                          lambda s, m: oracle.philox_fill_normal_f64(1, s, m, with_path=True), np.float64, 3,
                          "ziggurat"),
}


def compare(kind, got, want, what):
    if kind == "bits":
        if not np.array_equal(got.view(np.uint8), want.view(np.uint8)):
            raise AssertionError(f"{what}: {first_mismatch(got, want)}")
    elif kind == "ziggurat":
        want, path = want
        exact = path != 2
        g, w = got.view(np.uint64), want.view(np.uint64)
        bad = np.flatnonzero(exact & (g != w))
        assert bad.size == 0, (f"{what}: {bad.size} non-tail mismatches; first at {bad[0]}: got {got[bad[0]]!r} "
                               f"want {want[bad[0]]!r} path {path[bad[0]]}")
        t = ~exact
        if t.any():
            rel = np.abs(got[t] - want[t]) / np.abs(want[t])
            assert rel.max() <= TAIL_REL, f"{what}: tail relative error {rel.max()}"
    elif kind == "f32abs":
        err = np.abs(got.astype(np.float64) - want.astype(np.float64))
        assert np.isfinite(got).all(), f"{what}: non-finite values"
        assert err.max() <= F32_ABS, f"{what}: max abs error {err.max()} at {int(err.argmax())}"
    elif kind == "ulp":
        assert (got >= 0).all() and (want >= 0).all()
        d = np.abs(got.view(np.int64) - want.view(np.int64))
        assert d.max() <= EXP_F64_ULP, f"{what}: {int(d.max())} ulp at {int(d.argmax())}"
    else:
        raise ValueError(kind)


def check_whole(name, got, orc, start, kind, itemsize):
    """Compares `got` (all N elements) with the oracle computed piece by piece."""
    m = CHUNK_BYTES // itemsize
    pieces = [(c, min(m, N - c)) for c in range(0, N, m)]
    futs = [pool().submit(orc, start + c, k) for c, k in pieces]
    for (c, k), f in zip(pieces, futs):
        compare(kind, got[c:c + k], f.result(), f"{name}: elements [{c}, {c + k})")


@pytest.mark.parametrize("name", list(FAMILIES))
def test_every_element_full_size(name):
    fill, orc, dt, start, kind = FAMILIES[name]
    isz = np.dtype(dt).itemsize
    log(f"full size, every element: {name} start {start} ({N * isz >> 20} MiB)")
    b = DevBuf(N, isz)
    fill(b.ptr)
    got = b.host(dt)
    check_whole(name, got, orc, start, kind, isz)
    del b


def test_dropout_every_element_full_size():
    """The dropout workload: X = f32[2^20, 256] (numpy's seeded N(0, 1)), p = 0.1, key 8,
    counter = flat index; y and the mask, every element."""
    x = tk_inputs.normal_x(N)
    log("full size, every element: dropout_f32 (y and mask)")
    xd = torch.from_numpy(x).to("cuda")
    y = DevBuf(N, 4)
    mask = DevBuf(N, 1)
    tk.tk_dropout_f32(tk_inputs.DROPOUT_KEY, 0, N, tk_inputs.DROPOUT_P, xd, y.ptr, mask.ptr)
    gy, gm = y.host(np.uint32), mask.host(np.uint8)
    del xd
    m = CHUNK_BYTES // 4
    pieces = [(c, min(m, N - c)) for c in range(0, N, m)]
    futs = [pool().submit(oracle.dropout_f32, tk_inputs.DROPOUT_KEY, c, x[c:c + k], tk_inputs.DROPOUT_P)
            for c, k in pieces]
    for (c, k), f in zip(pieces, futs):
        wy, wm = f.result()
        compare("bits", gy[c:c + k], wy.view(np.uint32), f"dropout y [{c}, {c + k})")
        compare("bits", gm[c:c + k], wm, f"dropout mask [{c}, {c + k})")
