"""GPU parity of the uniform fills (and their Philox variant) against the oracle: bit-exact
for every type over start draws and lengths that cover every sub-word and pair offset,
misaligned outputs, ragged tails, several tiles, the counter-space edge, and the full
2^28-element workload (sampled)."""
import numpy as np
import pytest

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import DevBuf, assert_bits_equal, log

pytestmark = pytest.mark.gpu

# name -> (library call, oracle call, numpy dtype, largest draw + 1)
UNIFORM = {
    "u8": (tk.tk_fill_u8, oracle.fill_u8, np.uint8, 1 << 34),
    "u16": (tk.tk_fill_u16, oracle.fill_u16, np.uint16, 1 << 33),
    "u32": (tk.tk_fill_u32, oracle.fill_u32, np.uint32, 1 << 32),
    "u64": (tk.tk_fill_u64, oracle.fill_u64, np.uint64, 1 << 31),
    "f16_bits": (tk.tk_fill_f16_bits, oracle.fill_f16_bits, np.uint16, 1 << 33),
    "f32": (tk.tk_fill_f32, oracle.fill_f32, np.float32, 1 << 32),
    "f64": (tk.tk_fill_f64, oracle.fill_f64, np.float64, 1 << 31),
    "bool": (tk.tk_fill_bool, oracle.fill_bool, np.uint8, 1 << 37),
}
PHILOX = {
    "philox_u32": (tk.tk_philox_fill_u32, oracle.philox_fill_u32, np.uint32),
    "philox_u64": (tk.tk_philox_fill_u64, oracle.philox_fill_u64, np.uint64),
    "philox_f32": (tk.tk_philox_fill_f32, oracle.philox_fill_f32, np.float32),
    "philox_f64": (tk.tk_philox_fill_f64, oracle.philox_fill_f64, np.float64),
}

STARTS = (0, 1, 2, 3, 5, 15, 16, 17, 31, 33)
SIZES = (1, 2, 3, 15, 16, 17, 63, 64, 65, 1023, 4097, 65537)


def run(fill, key, start, n, dtype, offset_elems=0):
    isz = np.dtype(dtype).itemsize
    b = DevBuf(n, isz, offset_elems * isz)
    fill(key, start, n, b.ptr)
    return b.host(dtype)


@pytest.mark.parametrize("name", sorted(UNIFORM))
def test_small_sweep(name):
    """Every start offset class x ragged lengths x aligned and misaligned outputs."""
    fill, orc, dt, _ = UNIFORM[name]
    log(f"uniform sweep {name}")
    for off in (0, 1, 3):
        for s in STARTS:
            for n in SIZES:
                got = run(fill, 1, s, n, dt, off)
                assert_bits_equal(got, orc(1, s, n), f"{name} start={s} n={n} off={off}")


@pytest.mark.parametrize("name", sorted(UNIFORM))
def test_many_tiles(name):
    fill, orc, dt, _ = UNIFORM[name]
    for key in tk_inputs.KEYS + (0xFFFFFFFF,):
        for s in (0, 1, 3, 7):
            for off in (0, 1):
                n = (1 << 20) + 37
                log(f"uniform {name} key={key} start={s} n={n} off={off}")
                assert_bits_equal(run(fill, key, s, n, dt, off), orc(key, s, n), f"{name} key={key} s={s}")


@pytest.mark.parametrize("name", sorted(UNIFORM))
def test_counter_space_edge(name):
    fill, orc, dt, limit = UNIFORM[name]
    n = 4099
    got = run(fill, 9, limit - n, n, dt)
    assert_bits_equal(got, orc(9, limit - n, n), f"{name} at the end of the counter space")


@pytest.mark.parametrize("name", ["u32", "u64", "f32", "f64", "u8", "u16", "bool", "f16_bits"])
def test_full_size_sampled(name):
    """The 2^28-element workload: keys 1..3 x starts 0, 1, 3, compared on sampled elements
    (first/last 1024, around every power of two, 65536 random)."""
    fill, orc, dt, _ = UNIFORM[name]
    n = tk_inputs.FULL_N
    keys = tk_inputs.KEYS if name in ("u32", "u64", "f32", "f64") else (1,)
    isz = np.dtype(dt).itemsize
    b = DevBuf(n, isz)
    idx = tk_inputs.sample_indices(n, seed=11)
    for key in keys:
        for s in tk_inputs.STARTS:
            log(f"full {name} key={key} start={s}")
            fill(key, s, n, b.ptr)
            got = b.sample(idx, dt)
            assert_bits_equal(got, orc(key, 0, draws=idx.astype(np.uint64) + s), f"{name} key={key} s={s}")


def test_full_size_u32_every_element():
    """The first configuration (key 1, start 0, 2^20 elements) and the full 2^28 u32 fill
    compared element by element."""
    for n in (tk_inputs.SMALL_N, tk_inputs.FULL_N):
        log(f"u32 whole n={n}")
        got = run(tk.tk_fill_u32, 1, 0, n, np.uint32)
        assert_bits_equal(got, oracle.fill_u32(1, 0, n), f"u32 n={n}")


@pytest.mark.parametrize("name", sorted(PHILOX))
def test_philox(name):
    fill, orc, dt = PHILOX[name]
    for key in (0, 1, 0x0123456789ABCDEF, (1 << 64) - 1):
        for s in (0, 1, 2, 3, 5, 6, 7):
            for off in (0, 1):
                for n in (1, 3, 17, 65, 4097, (1 << 18) + 5):
                    got = run(fill, key, s, n, dt, off)
                    assert_bits_equal(got, orc(key, s, n), f"{name} key={key:#x} s={s} n={n} off={off}")
    big_start = (1 << 40) + 3  # block counters above 32 bits
    assert_bits_equal(run(fill, 5, big_start, 1000, dt), orc(5, big_start, 1000), f"{name} high counter")


def test_philox_full_size_sampled():
    n = tk_inputs.FULL_N
    b = DevBuf(n, 4)
    idx = tk_inputs.sample_indices(n, seed=12)
    for s in tk_inputs.STARTS:
        tk.tk_philox_fill_u32(1, s, n, b.ptr)
        assert_bits_equal(b.sample(idx, np.uint32), oracle.philox_fill_u32(1, 0, draws=idx.astype(np.uint64) + s))


def test_zero_length_writes_nothing():
    for name, (fill, _, dt, _) in UNIFORM.items():
        b = DevBuf(0, np.dtype(dt).itemsize)
        fill(1, 0, 0, b.ptr)
        assert b.host(dt).size == 0


def test_constant_fill():
    """The store-ceiling kernel writes exactly its n words at any 4-byte alignment."""
    for off in (0, 1, 3, 1021):
        for n in (1, 5, 1023, 1024 + off, (1 << 20) + 3):
            b = DevBuf(n, 4, 4 * off)
            tk.tk_fill_constant_u32(0xDEADBEEF, n, b.ptr)
            assert (b.host(np.uint32) == 0xDEADBEEF).all(), (off, n)
