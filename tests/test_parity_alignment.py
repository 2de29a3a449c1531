"""GPU parity at outputs placed a chosen distance past a 4 KiB boundary.

The streaming and choice kernels store 16-byte vectors from the output's first 4 KiB
boundary and write the h elements before it one at a time; the default f64 normal fill
runs as two launches split at that boundary.  These cases put the output 8, 2056 or
4088 bytes past a boundary (1 byte for u8) and take lengths around h (h - 1, h, h + 1,
h + 2) and several tiles past it, at start draws 0 and 3, against the oracle, with
canaries on both sides of every output."""
import numpy as np
import pytest
import torch

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import CANARY, DevBuf, assert_bits_equal, log

pytestmark = pytest.mark.gpu

BOUNDARY = 4096
TILE_BYTES = 4096


class PlacedBuf(DevBuf):
    """A DevBuf whose output starts `past` bytes after a 4 KiB boundary."""

    def __init__(self, n, itemsize, past, pad=256):
        self.n, self.itemsize = int(n), int(itemsize)
        self.nbytes = self.n * self.itemsize
        self.buf = torch.full((256 + BOUNDARY + self.nbytes + pad,), CANARY, dtype=torch.uint8, device="cuda")
        lo = self.buf.data_ptr() + 256
        self.base = 256 + (past - lo) % BOUNDARY
        self.off = self.base - 256
        assert (self.buf.data_ptr() + self.base) % BOUNDARY == past


def lengths(itemsize, past):
    h = (BOUNDARY - past) // itemsize
    return sorted({max(1, h - 1), h, h + 1, h + 2, h + 3 * TILE_BYTES // itemsize + 5})


W = tk_inputs.zipf_weights()
Q, AL, _ = oracle.alias_build(W)

# name -> (itemsize, numpy dtype, device fill(start, n, ptr), oracle(start, n))
CASES = {
    "u8": (1, np.uint8, lambda s, n, p: tk.tk_fill_u8(1, s, n, p), lambda s, n: oracle.fill_u8(1, s, n)),
    "u16": (2, np.uint16, lambda s, n, p: tk.tk_fill_u16(1, s, n, p), lambda s, n: oracle.fill_u16(1, s, n)),
    "u32": (4, np.uint32, lambda s, n, p: tk.tk_fill_u32(1, s, n, p), lambda s, n: oracle.fill_u32(1, s, n)),
    "f64": (8, np.float64, lambda s, n, p: tk.tk_fill_f64(1, s, n, p), lambda s, n: oracle.fill_f64(1, s, n)),
    "u64_below": (8, np.uint64, lambda s, n, p: tk.tk_fill_u64_below(1, s, n, 1000, p),
                  lambda s, n: oracle.fill_u64_below(1, s, n, 1000)),
    "exponential_f32": (4, np.float32, lambda s, n, p: tk.tk_fill_exponential_f32(1, s, n, p),
                        lambda s, n: oracle.fill_exponential_f32(1, s, n)),
    "choice_u32": (4, np.uint32, None, lambda s, n: oracle.fill_choice_u32(1, s, n, Q, AL)),
    "philox_u32": (4, np.uint32, lambda s, n, p: tk.tk_philox_fill_u32(9, s, n, p),
                   lambda s, n: oracle.philox_fill_u32(9, s, n)),
}

_table = None


def table():
    global _table
    if _table is None:
        _table = tk.tk_alias_create(W)
    return _table


@pytest.mark.parametrize("name", list(CASES))
def test_exact_fills_around_the_boundary(name):
    isz, dt, fill, want = CASES[name]
    if name == "choice_u32":
        fill = lambda s, n, p: tk.tk_fill_choice_u32(1, s, n, table(), p)  # noqa: E731
    pasts = (8, 2056, 4088) + ((1,) if isz == 1 else ())
    for past in pasts:
        for n in lengths(isz, past):
            for s in (0, 3):
                log(f"{name}: {past} bytes past 4 KiB, n={n}, start={s}")
                b = PlacedBuf(n, isz, past)
                fill(s, n, b.ptr)
                assert_bits_equal(b.host(dt), want(s, n), f"{name} past={past} n={n} s={s}")


def test_f64_normal_around_the_boundary():
    """The default fill's two launches (and one launch when n fits before the boundary)."""
    for past in (8, 2056, 4088):
        for n in lengths(8, past):
            for s in (0, 3):
                log(f"normal_f64: {past} bytes past 4 KiB, n={n}, start={s}")
                b = PlacedBuf(n, 8, past)
                tk.tk_fill_normal_f64(2, s, n, b.ptr)
                got = b.host(np.float64)
                want, path = oracle.fill_normal_f64(2, s, n, with_path=True)
                exact = path != 2
                assert_bits_equal(got[exact], want[exact], f"normal_f64 past={past} n={n} s={s}")
                if (~exact).any():
                    assert np.max(np.abs(got[~exact] / want[~exact] - 1)) <= 1e-12


def test_f32_normal_around_the_boundary():
    for past in (8, 2056, 4088):
        for n in lengths(4, past):
            for s in (0, 3):
                log(f"normal_f32: {past} bytes past 4 KiB, n={n}, start={s}")
                b = PlacedBuf(n, 4, past)
                tk.tk_fill_normal_f32(1, s, n, b.ptr)
                got = b.host(np.float32).astype(np.float64)
                want = oracle.fill_normal_f32(1, s, n).astype(np.float64)
                assert np.max(np.abs(got - want)) <= 4e-6, f"normal_f32 past={past} n={n} s={s}"
