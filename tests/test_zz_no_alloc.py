"""tk_fill_normal_f64_no_alloc (the f64 normal fill without allocation) through the C ABI,
against the existing entry point tk_fill_normal_f64 and the oracle.

Two calls in a row on one device share its static miss lists; the second is smaller, so
any state the first leaves behind would show.  Tolerances are the f64 normal's: the
fast-path and wedge values bit-exact, tail values within 1e-12 relative (against the
oracle; the two device entry points finish misses with the same code and agree bit for
bit).  The call must also work while every device allocation of the library is made to
fail, and must not change the device memory the library holds."""
import ctypes as C

import numpy as np
import pytest
import torch

import bulk_fills_amd as tk
import oracle
from gpu_harness import DevBuf, assert_bits_equal, log

pytestmark = pytest.mark.gpu

MAX_N = 1 << 24


def no_alloc(key, start, n, ptr):
    """The entry point called through the C ABI directly (the binding's names are the
    same; this makes the status visible)."""
    return tk.lib.tk_fill_normal_f64_no_alloc(key, start, n, ptr, torch.cuda.current_stream().cuda_stream)


def compare(key, start, n, off):
    log(f"no-alloc normal_f64 key={key} start={start} n={n} off={off}")
    a = DevBuf(n, 8, 8 * off)
    b = DevBuf(n, 8, 8 * off)
    tk.tk_fill_normal_f64(key, start, n, a.ptr)
    assert no_alloc(key, start, n, b.ptr) == tk.TK_OK
    got, ref = b.host(np.float64), a.host(np.float64)
    assert_bits_equal(got, ref, f"no-alloc vs tk_fill_normal_f64 (n={n})")
    want, path = oracle.fill_normal_f64(key, start, n, with_path=True)
    exact = path != 2
    assert_bits_equal(got[exact], want[exact], f"no-alloc vs the oracle, non-tail (n={n})")
    if (~exact).any():
        assert np.max(np.abs(got[~exact] / want[~exact] - 1)) <= 1e-12


def test_two_calls_in_a_row_second_smaller():
    compare(1, 3, MAX_N, 0)               # the largest call the static lists hold
    compare(7, 123457, (1 << 20) + 3, 1)  # then a smaller one, output misaligned


def test_short_and_ragged():
    for n in (1, 2, 3, 2047, 2049, 4097):
        compare(5, 1, n, n & 1)


def test_refuses_sizes_beyond_the_limit():
    b = DevBuf(4, 8)
    assert no_alloc(1, 0, MAX_N + 1, b.ptr) == tk.TK_EINVAL
    with pytest.raises(tk.TkError):
        tk.tk_fill_normal_f64_no_alloc(1, 0, MAX_N + 1, b.ptr)
    assert b.host(np.uint64).size == 4  # canaries around the buffer untouched


def test_allocates_nothing():
    warm = DevBuf(16, 8)
    tk.tk_fill_normal_f64(1, 0, 16, warm.ptr)  # the existing entry point's tables exist before the hook
    torch.cuda.synchronize()
    held = tk.tk_debug_device_bytes()
    tk.tk_debug_fail_allocations(0, 1 << 30)  # every library allocation would now fail
    try:
        compare(9, 77, (1 << 18) + 5, 0)
        b = DevBuf(1 << 16, 8)
        assert no_alloc(2, 0, 1 << 16, b.ptr) == tk.TK_OK
        torch.cuda.synchronize()
    finally:
        tk.tk_debug_fail_allocations(0, 0)
    assert tk.tk_debug_device_bytes() == held
