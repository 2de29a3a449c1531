"""GPU parity of the exponential fills against the oracle.  f32: bit-exact (both sides
give the correctly rounded value at every 2^-24 grid point, so every possible input
agrees; every grid point is checked through counters built with an inverse hash).  f64:
within 2 ulp (the device's table-driven logarithm is within 0.502 ulp of the exact value
and the host's libm about as close, so they differ by at most 1 ulp)."""
import numpy as np
import pytest

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import DevBuf, assert_bits_equal, log
from test_oracle_pins import _inverse_hash_np

pytestmark = pytest.mark.gpu


def run(fill, key, s, n, isz, dtype, off=0):
    b = DevBuf(n, isz, off * isz)
    fill(key, s, n, b.ptr)
    return b.host(dtype)


def ulp_diff64(got, want):
    """Distance in units in the last place, in integer arithmetic on the bit patterns of
    non-negative doubles (a float conversion of the patterns would round it away)."""
    return np.abs(got.view(np.int64) - want.view(np.int64))


def report64(got, want, key, draws):
    """Details of the elements more than 2 ulp apart, for the failure message."""
    d = ulp_diff64(got, want)
    bad = np.flatnonzero(d > 2)[:8]
    if bad.size == 0:
        return ""
    import mpmath as mp
    mp.mp.dps = 40
    raw = oracle.fill_u64(key, 0, 0, draws=np.asarray(draws, dtype=np.uint64)[bad])
    lines = []
    for j, r in zip(bad, raw):
        u = mp.mpf(int(r) & ((1 << 53) - 1)) * mp.mpf(2) ** -53
        ref = -mp.log(1 - u)
        sp = mp.mpf(float(np.spacing(want[j])))
        lines.append(f"draw {int(draws[j])} u={float(u):.17g} got={got[j]!r} want={want[j]!r} "
                     f"got-ref={float((mp.mpf(got[j]) - ref) / sp):.2f}ulp want-ref={float((mp.mpf(want[j]) - ref) / sp):.2f}ulp")
    return "\n".join(lines)


@pytest.mark.parametrize("key", (1, 2, 0xFFFFFFFF))
def test_exponential_f32_sweep(key):
    for s in (0, 1, 3, 5):
        for n in (1, 3, 4, 5, 17, 4097, (1 << 20) + 3):
            for off in (0, 1):
                got = run(tk.tk_fill_exponential_f32, key, s, n, 4, np.float32, off)
                assert_bits_equal(got, oracle.fill_exponential_f32(key, s, n), f"s={s} n={n} off={off}")


def test_exponential_f32_every_grid_point():
    """Fill the whole counter space in 2^28-element pieces and read back one element per
    2^-24 grid value (the counters whose words end in that value)."""
    key = 5
    m = np.arange(1 << 24, dtype=np.uint64)
    counters = (_inverse_hash_np(m) ^ np.uint64(oracle.hash32(key))).astype(np.int64)
    want = oracle.fill_exponential_f32(key, 0, 0, draws=counters.astype(np.uint64))
    got = np.empty(m.size, dtype=np.float32)
    n = tk_inputs.FULL_N
    b = DevBuf(n, 4)
    for piece in range(16):
        s = piece * n
        sel = np.flatnonzero((counters >= s) & (counters < s + n))
        log(f"exponential_f32 piece {piece}: {sel.size} grid points")
        tk.tk_fill_exponential_f32(key, s, n, b.ptr)
        got[sel] = b.sample(counters[sel] - s, np.float32)
    assert_bits_equal(got, want, "every grid point")


def test_exponential_f64_sweep():
    for key in (1, 3):
        for s in (0, 1, 3):
            for n in (1, 2, 3, 17, 4097, (1 << 20) + 1):
                for off in (0, 1):
                    got = run(tk.tk_fill_exponential_f64, key, s, n, 8, np.float64, off)
                    want = oracle.fill_exponential_f64(key, s, n)
                    d = ulp_diff64(got, want)
                    assert d.max() <= 2, (key, s, n, off, d.max(), report64(got, want, key, np.arange(n) + s))


def _model64():
    """The host model of the f64 logarithm (tests/exp_f64_model.c, library form, built by
    build()): the kernel's operations in the same order, IEEE double with explicit fma."""
    import ctypes as C
    import os
    lib = C.CDLL(os.path.join(os.path.dirname(os.path.abspath(__file__)), "libexp_f64_model.so"))
    lib.tk_model_neg_ln_batch.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t]

    def model(d):
        d = np.ascontiguousarray(d, dtype=np.uint64)
        out = np.empty(d.size, dtype=np.float64)
        lib.tk_model_neg_ln_batch(d.ctypes.data, out.ctypes.data, d.size)
        return out
    return model


def test_exponential_f64_is_the_modelled_sequence():
    """Every element of the device's f64 exponential equals the host model of its
    operations bit for bit (the model's draws are the oracle's 64-bit draws), so the error
    bound the model establishes on the host (0.502 ulp; tests/test_log_table.py) holds for
    what the device computes."""
    model = _model64()
    n = (1 << 20) + 3
    for key in (1, 0xFFFFFFFF):
        for s in (0, 1, 3, (1 << 31) - n):  # the last start ends at the top of the 2^31 draws
            for off in (0, 1):
                got = run(tk.tk_fill_exponential_f64, key, s, n, 8, np.float64, off)
                assert_bits_equal(got, model(oracle.fill_u64(key, s, n)), f"exponential_f64 key={key} s={s} off={off}")


def test_exponential_full_size_sampled():
    n = tk_inputs.FULL_N
    idx = tk_inputs.sample_indices(n, seed=18)
    b8, b4 = DevBuf(n, 8), DevBuf(n, 4)
    for s in tk_inputs.STARTS:
        tk.tk_fill_exponential_f64(1, s, n, b8.ptr)
        got = b8.sample(idx, np.float64)
        want = oracle.fill_exponential_f64(1, 0, draws=idx.astype(np.uint64) + s)
        d = ulp_diff64(got, want)
        log(f"exponential_f64 2^28 s={s}: max {d.max():.0f} ulp, {np.count_nonzero(d)} of {d.size} differ")
        assert d.max() <= 2, report64(got, want, 1, idx + s)
        tk.tk_fill_exponential_f32(1, s, n, b4.ptr)
        assert_bits_equal(b4.sample(idx, np.float32), oracle.fill_exponential_f32(1, 0, draws=idx.astype(np.uint64) + s))
