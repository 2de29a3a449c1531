"""GPU parity of the generator and normal variants against the oracle: Philox bounded,
choice, Box-Muller and ziggurat fills; the half-turn Box-Muller; one normal per counter.

Bit-exact: Philox bounded and choice, the Philox ziggurat's fast-path and wedge values,
and its miss count.  Ziggurat tail values within 1e-12 relative; Box-Muller values within
4e-6 absolute.  randn must equal the even elements of the device's own pair fill bit for
bit (both are the header's tk_randn2_f32)."""
import numpy as np
import pytest
import torch

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import DevBuf, assert_bits_equal, log

pytestmark = pytest.mark.gpu

PK = 0x0123456789ABCDEF
STARTS = (0, 1, 2, 3, 5, (1 << 33) + 1)
LENGTHS = (1, 3, 4, 5, 17, 4097, (1 << 18) + 3)
F32_ABS = 4e-6
TAIL_REL = 1e-12


def run(fill, isz, dtype, start, n, *args, off=0):
    b = DevBuf(n, isz, off * isz)
    fill(PK, start, n, *args, b.ptr)
    return b.host(dtype)


@pytest.mark.parametrize("bound", [1000, (1 << 31) + 1, (1 << 32) - 2])
def test_philox_u32_below(bound):
    for s in STARTS:
        for n in LENGTHS:
            for off in (0, 1):
                got = run(tk.tk_philox_fill_u32_below, 4, np.uint32, s, n, bound, off=off)
                assert_bits_equal(got, oracle.philox_fill_u32_below(PK, s, n, bound), f"b={bound} s={s} n={n} off={off}")


@pytest.mark.parametrize("bound", [1000, (1 << 32) - 1, (1 << 63) + 1, (1 << 64) - 2])
def test_philox_u64_below(bound):
    for s in STARTS:
        for n in LENGTHS:
            got = run(tk.tk_philox_fill_u64_below, 8, np.uint64, s, n, bound, off=s & 1)
            assert_bits_equal(got, oracle.philox_fill_u64_below(PK, s, n, bound), f"b={bound} s={s} n={n}")


def test_philox_bounded_full_size_sampled():
    n = tk_inputs.FULL_N
    idx = tk_inputs.sample_indices(n, seed=31)
    b = DevBuf(n, 4)
    for s, bound in ((0, 1000), (3, (1 << 31) + 1)):
        log(f"philox u32_below 2^28 s={s} bound={bound}")
        tk.tk_philox_fill_u32_below(PK, s, n, bound, b.ptr)
        assert_bits_equal(b.sample(idx, np.uint32),
                          oracle.philox_fill_u32_below(PK, 0, 0, bound, draws=idx.astype(np.uint64) + s), "sampled")


@pytest.fixture(scope="module")
def zipf():
    w = tk_inputs.zipf_weights()
    table = tk.tk_alias_create(w)
    q, al, _ = oracle.alias_build(w)
    yield table, q, al
    table.close()


def test_philox_choice(zipf):
    table, q, al = zipf
    for s in STARTS:
        for n in LENGTHS:
            for off in (0, 1, 2, 3):
                b = DevBuf(n, 4, off * 4)
                tk.tk_philox_fill_choice_u32(PK, s, n, table, b.ptr)
                assert_bits_equal(b.host(np.uint32), oracle.philox_fill_choice_u32(PK, s, n, q, al),
                                  f"s={s} n={n} off={off}")


def test_philox_choice_full_size_sampled(zipf):
    table, q, al = zipf
    n = tk_inputs.FULL_N
    b = DevBuf(n, 4)
    idx = tk_inputs.sample_indices(n, seed=32)
    for s in (0, 2):
        log(f"philox choice 2^28 s={s}")
        tk.tk_philox_fill_choice_u32(PK, s, n, table, b.ptr)
        assert_bits_equal(b.sample(idx, np.uint32),
                          oracle.philox_fill_choice_u32(PK, 0, 0, q, al, draws=idx.astype(np.uint64) + s), "sampled")


def f32_close(got, want, what):
    err = float(np.max(np.abs(got.astype(np.float64) - want.astype(np.float64)))) if want.size else 0.0
    assert err <= F32_ABS, f"{what}: max abs err {err}"
    return err


def test_philox_normal_f32():
    for s in STARTS:
        for n in LENGTHS:
            for off in (0, 1, 3):
                got = run(tk.tk_philox_fill_normal_f32, 4, np.float32, s, n, off=off)
                f32_close(got, oracle.philox_fill_normal_f32(PK, s, n), f"s={s} n={n} off={off}")
    n = tk_inputs.FULL_N
    b = DevBuf(n, 4)
    idx = tk_inputs.sample_indices(n, seed=33)
    tk.tk_philox_fill_normal_f32(PK, 1, n, b.ptr)
    f32_close(b.sample(idx, np.float32), oracle.philox_fill_normal_f32(PK, 0, 0, draws=idx.astype(np.uint64) + 1),
              "2^28 sampled")


def test_half_turn_normal_f32():
    for s in (0, 1, 2, 3, 17):
        for n in (1, 2, 3, 5, 4097, (1 << 20) + 1):
            for off in (0, 1):
                b = DevBuf(n, 4, 4 * off)
                tk.tk_fill_normal_f32_half_turn(6, s, n, b.ptr)
                f32_close(b.host(np.float32), oracle.fill_normal_f32_half_turn(6, s, n), f"s={s} n={n}")


def test_randn_is_the_even_pair_elements():
    for s in (0, 1, 7):
        for n in (1, 3, 4, 5, 4097, (1 << 20) + 3):
            r, p = DevBuf(n, 4), DevBuf(2 * n, 4)
            tk.tk_fill_randn_f32(3, s, n, r.ptr)
            tk.tk_fill_normal_f32(3, 2 * s, 2 * n, p.ptr)
            got = r.host(np.float32)
            assert_bits_equal(got, p.host(np.float32)[0::2].copy(), f"randn vs pair fill s={s} n={n}")
            f32_close(got, oracle.fill_randn_f32(3, s, n), f"randn vs oracle s={s} n={n}")


MODES = {"default": 0, "two_kernels": 1, "fused": 2}


@pytest.fixture(params=sorted(MODES))
def f64_mode(request):
    """The library default (fused, uncounted) and each path the test hook chooses."""
    tk.tk_debug_set_normal_f64_mode(MODES[request.param])
    yield request.param
    tk.tk_debug_set_normal_f64_mode(0)


def check_f64(got, start, n=None, draws=None, what=""):
    want, path = oracle.philox_fill_normal_f64(PK, start, n, draws=draws, with_path=True)
    exact = path != 2
    bad = np.flatnonzero(got[exact].view(np.uint64) != want[exact].view(np.uint64))
    assert bad.size == 0, (f"{what}: {bad.size} non-tail mismatches; first got {got[exact][bad[0]]!r} "
                           f"want {want[exact][bad[0]]!r} path {path[exact][bad[0]]}")
    t = ~exact
    if t.any():
        rel = np.abs(got[t] - want[t]) / np.abs(want[t])
        assert rel.max() <= TAIL_REL, f"{what}: tail rel err {rel.max()}"
    return int((path != 0).sum())


def test_philox_normal_f64(f64_mode):
    for s in STARTS:
        for n in (1, 2, 3, 5, 17, 4097, (1 << 20) + 3):
            for off in (0, 1):
                b = DevBuf(n, 8, 8 * off)
                tk.tk_philox_fill_normal_f64(PK, s, n, b.ptr)
                misses = check_f64(b.host(np.float64), s, n, what=f"s={s} n={n} off={off}")
                if f64_mode == "default":  # uncounted: the hook refuses
                    with pytest.raises(tk.TkError):
                        tk.tk_debug_last_miss_count()
                else:
                    assert tk.tk_debug_last_miss_count() == misses, (s, n, off)


def test_philox_normal_f64_forced_overflow():
    n = (1 << 20) + 1
    try:
        for mode in (1, 2):
            tk.tk_debug_set_normal_f64_mode(mode)
            for per_group, overflow in ((1, 1 << 22), (1, 1), (16, 1)):
                tk.tk_debug_set_miss_capacity(per_group, overflow)
                b = DevBuf(n, 8)
                tk.tk_philox_fill_normal_f64(PK, 3, n, b.ptr)
                check_f64(b.host(np.float64), 3, n, what=f"mode={mode} cap={(per_group, overflow)}")
    finally:
        tk.tk_debug_set_miss_capacity(0, 0)
        tk.tk_debug_set_normal_f64_mode(0)


def test_philox_normal_f64_full_size_sampled(f64_mode):
    n = tk_inputs.FULL_N
    b = DevBuf(n, 8)
    idx = tk_inputs.sample_indices(n, seed=34)
    _, path = oracle.philox_fill_normal_f64(PK, 1, 1 << 21, with_path=True)
    miss = np.flatnonzero(path != 0).astype(np.uint64)
    log("philox normal_f64 2^28")
    tk.tk_philox_fill_normal_f64(PK, 1, n, b.ptr)
    check_f64(b.sample(idx, np.float64), 0, draws=idx.astype(np.uint64) + 1, what="2^28 sampled")
    check_f64(b.sample(miss, np.float64), 0, draws=miss + 1, what="2^28 misses in the first 2^21")
    if f64_mode != "default":  # the default fill keeps no counts
        assert abs(tk.tk_debug_last_miss_count() - 0.0042765667 * n) < 6 * np.sqrt(0.0043 * n)
