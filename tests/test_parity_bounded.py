"""GPU parity of the bounded fills (Lemire multiply-shift, exact threshold, retries on the
per-index substream) against the oracle, bit-exact, including rejection-heavy bounds
where about half the draws take the substream path."""
import numpy as np
import pytest

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import DevBuf, assert_bits_equal, log

pytestmark = pytest.mark.gpu

B32 = (1, 2, 3, 1000, 65537, 3 << 30, (1 << 31) + 1, (1 << 32) - 2, (1 << 32) - 1)
B64 = (1, 2, 1000, (1 << 32) - 1, 1 << 32, (1 << 32) + 1, 3 << 62, (1 << 63) + 1, (1 << 64) - 2, (1 << 64) - 1)


def run(call, n, isz, dtype, off=0):
    b = DevBuf(n, isz, off * isz)
    call(b.ptr)
    return b.host(dtype)


@pytest.mark.parametrize("bound", B32)
def test_u32_below(bound):
    for s in (0, 1, 3, 5):
        for n in (1, 5, 17, 4099, (1 << 20) + 3):
            for off in (0, 1):
                log(f"u32_below bound={bound} s={s} n={n} off={off}")
                got = run(lambda p: tk.tk_fill_u32_below(2, s, n, bound, p), n, 4, np.uint32, off)
                assert_bits_equal(got, oracle.fill_u32_below(2, s, n, bound), f"bound={bound} s={s} n={n}")


@pytest.mark.parametrize("bound", B64)
def test_u64_below(bound):
    for s in (0, 1, 3):
        for n in (1, 5, 17, 4099, (1 << 19) + 3):
            for off in (0, 1):
                log(f"u64_below bound={bound} s={s} n={n} off={off}")
                got = run(lambda p: tk.tk_fill_u64_below(2, s, n, bound, p), n, 8, np.uint64, off)
                assert_bits_equal(got, oracle.fill_u64_below(2, s, n, bound), f"bound={bound} s={s} n={n}")


@pytest.mark.parametrize("low,bound", [(-500, 1000), (-(1 << 31), (1 << 32) - 1), (0, 1), (-7, (1 << 31) + 1),
                                       ((1 << 31) - 1, 1)])
def test_i32_below(low, bound):
    for s in (0, 3):
        for n in (3, 4099, (1 << 20) + 1):
            for off in (0, 1):
                got = run(lambda p: tk.tk_fill_i32_below(3, s, n, low, bound, p), n, 4, np.int32, off)
                assert_bits_equal(got, oracle.fill_i32_below(3, s, n, low, bound), f"low={low} bound={bound}")


@pytest.mark.parametrize("low,bound", [(-500, 1000), (-(1 << 62), (1 << 32) - 1), ((1 << 63) - (1 << 32), 1 << 31)])
def test_i64_below32(low, bound):
    for s in (0, 1, 3):
        for n in (3, 4099, (1 << 20) + 1):
            for off in (0, 1):
                got = run(lambda p: tk.tk_fill_i64_below32(3, s, n, low, bound, p), n, 8, np.int64, off)
                assert_bits_equal(got, oracle.fill_i64_below32(3, s, n, low, bound), f"low={low} bound={bound}")


@pytest.mark.parametrize("low,bound", [(-500, 1000), (-(1 << 62), 1 << 63), (-(1 << 63), (1 << 64) - 1),
                                       (-5, (1 << 63) + 1)])
def test_i64_below(low, bound):
    for s in (0, 1, 3):
        for n in (3, 4099, (1 << 19) + 1):
            for off in (0, 1):
                got = run(lambda p: tk.tk_fill_i64_below(3, s, n, low, bound, p), n, 8, np.int64, off)
                assert_bits_equal(got, oracle.fill_i64_below(3, s, n, low, bound), f"low={low} bound={bound}")


def test_full_size_sampled():
    """The 2^28-element bounded workload, compared on sampled elements."""
    n = tk_inputs.FULL_N
    idx = tk_inputs.sample_indices(n, seed=13)
    d = idx.astype(np.uint64)
    b4, b8 = DevBuf(n, 4), DevBuf(n, 8)
    for bound in tk_inputs.BOUNDS32:
        log(f"full u32_below({bound})")
        tk.tk_fill_u32_below(1, 0, n, bound, b4.ptr)
        assert_bits_equal(b4.sample(idx, np.uint32), oracle.fill_u32_below(1, 0, bound=bound, draws=d))
    for bound in tk_inputs.BOUNDS64:
        log(f"full u64_below({bound})")
        tk.tk_fill_u64_below(1, 0, n, bound, b8.ptr)
        assert_bits_equal(b8.sample(idx, np.uint64), oracle.fill_u64_below(1, 0, bound=bound, draws=d))
    tk.tk_fill_i32_below(1, 0, n, tk_inputs.LOW, tk_inputs.LOW_BOUND, b4.ptr)
    assert_bits_equal(b4.sample(idx, np.int32),
                      oracle.fill_i32_below(1, 0, low=tk_inputs.LOW, bound=tk_inputs.LOW_BOUND, draws=d))
    tk.tk_fill_i64_below32(1, 0, n, tk_inputs.LOW, tk_inputs.LOW_BOUND, b8.ptr)
    assert_bits_equal(b8.sample(idx, np.int64),
                      oracle.fill_i64_below32(1, 0, low=tk_inputs.LOW, bound=tk_inputs.LOW_BOUND, draws=d))


def test_every_rejection_at_full_size():
    """u32_below(1000) rejects about 18 of 2^28 draws; find them with the oracle's map over
    the oracle's words and check each one, so the substream path is exercised at size."""
    n = tk_inputs.FULL_N
    words = oracle.fill_u32(1, 0, n)
    _, acc = oracle.lemire32_map(words, 1000)
    rej = np.flatnonzero(~acc)
    assert rej.size > 0
    b = DevBuf(n, 4)
    tk.tk_fill_u32_below(1, 0, n, 1000, b.ptr)
    assert_bits_equal(b.sample(rej, np.uint32), oracle.fill_u32_below(1, 0, bound=1000, draws=rej.astype(np.uint64)))
