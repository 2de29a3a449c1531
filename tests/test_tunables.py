"""GPU parity of every launch shape a tunable selects (include/tk.h, tk_debug_set_tunable).

The defaults are the measured best; the alternatives stay in the library for measurement,
so each must compute the same values: the fills each shape touches, at a length that spans
several work-groups and ends ragged, at start draws 0, 1 and 3 and a misaligned output,
against the oracle (bit-exact; Box-Muller within 4e-6; ziggurat tails within 1e-12
relative; the f64 exponential within 2 ulp)."""
import numpy as np
import pytest
import torch

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import DevBuf, assert_bits_equal, log

pytestmark = pytest.mark.gpu

N = (1 << 20) + 5
KEY = 9
PK = 0x0123456789ABCDEF
STARTS = (0, 1, 3)


def run(fill, key, s, isz, dtype, *args, off=1):
    b = DevBuf(N, isz, off * isz)
    fill(key, s, N, *args, b.ptr)
    return b.host(dtype)


def check_streaming():
    for s in STARTS:
        for fill, orc, isz, dt in ((tk.tk_fill_u32, oracle.fill_u32, 4, np.uint32),
                                   (tk.tk_fill_u64, oracle.fill_u64, 8, np.uint64),
                                   (tk.tk_fill_u8, oracle.fill_u8, 1, np.uint8),
                                   (tk.tk_fill_bool, oracle.fill_bool, 1, np.uint8),
                                   (tk.tk_fill_f16_bits, oracle.fill_f16_bits, 2, np.uint16),
                                   (tk.tk_fill_f64, oracle.fill_f64, 8, np.float64)):
            assert_bits_equal(run(fill, KEY, s, isz, dt), orc(KEY, s, N), f"{fill.__name__} s={s}")
        assert_bits_equal(run(tk.tk_fill_u32_below, KEY, s, 4, np.uint32, 1000),
                          oracle.fill_u32_below(KEY, s, N, 1000), f"u32_below s={s}")
        assert_bits_equal(run(tk.tk_philox_fill_u32, PK, s, 4, np.uint32),
                          oracle.philox_fill_u32(PK, s, N), f"philox_u32 s={s}")
        got = run(tk.tk_fill_normal_f32, KEY, s, 4, np.float32)
        err = np.max(np.abs(got.astype(np.float64) - oracle.fill_normal_f32(KEY, s, N)))
        assert err <= 4e-6, f"normal_f32 s={s}: {err}"
    x = tk_inputs.normal_x(N, seed=7)
    xb = DevBuf(N, 4)
    xb.buf[xb.base:xb.base + x.nbytes].copy_(torch.from_numpy(x.view(np.uint8).copy()).to("cuda"))
    yb, mb = DevBuf(N, 4, 4), DevBuf(N, 1)
    tk.tk_dropout_f32(KEY, 3, N, 0.1, xb.ptr, yb.ptr, mb.ptr)
    y, m = oracle.dropout_f32(KEY, 3, x, 0.1)
    assert_bits_equal(yb.host(np.float32), y, "dropout y")
    assert_bits_equal(mb.host(np.uint8), m, "dropout mask")


def check_choice():
    w = tk_inputs.zipf_weights()
    table = tk.tk_alias_create(w)
    q, al, _ = oracle.alias_build(w)
    try:
        for s in STARTS:
            assert_bits_equal(run(tk.tk_fill_choice_u32, KEY, s, 4, np.uint32, table),
                              oracle.fill_choice_u32(KEY, s, N, q, al), f"choice s={s}")
            assert_bits_equal(run(tk.tk_philox_fill_choice_u32, PK, s, 4, np.uint32, table),
                              oracle.philox_fill_choice_u32(PK, s, N, q, al), f"philox choice s={s}")
    finally:
        table.close()


def check_exponential():
    for s in STARTS:
        assert_bits_equal(run(tk.tk_fill_exponential_f32, KEY, s, 4, np.float32),
                          oracle.fill_exponential_f32(KEY, s, N), f"exponential_f32 s={s}")
        got = run(tk.tk_fill_exponential_f64, KEY, s, 8, np.float64)
        d = np.abs(got.view(np.int64) - oracle.fill_exponential_f64(KEY, s, N).view(np.int64))
        assert d.max() <= 2, f"exponential_f64 s={s}: {d.max()} ulp"


def check_normal_f64():
    for fill, orc, key in ((tk.tk_fill_normal_f64, oracle.fill_normal_f64, KEY),
                           (tk.tk_philox_fill_normal_f64, oracle.philox_fill_normal_f64, PK)):
        for s in STARTS:
            got = run(fill, key, s, 8, np.float64)
            want, path = orc(key, s, N, with_path=True)
            exact = path != 2
            assert_bits_equal(got[exact], want[exact], f"{fill.__name__} s={s} non-tail")
            if (~exact).any():
                assert np.max(np.abs(got[~exact] / want[~exact] - 1)) <= 1e-12
            try:
                counted = tk.tk_debug_last_miss_count()
            except tk.TkError:  # the default fused fill keeps no counts
                counted = None
            assert counted in (None, int((path != 0).sum()))


def check_constant():
    for off in (0, 1, 3):
        b = DevBuf(N, 4, 4 * off)
        tk.tk_fill_constant_u32(0x01020304, N, b.ptr)
        assert (b.host(np.uint32) == 0x01020304).all(), off


def check_philox():
    for s in (0, 1, 2, 3, 5):
        for fill, orc, isz, dt in ((tk.tk_philox_fill_u32, oracle.philox_fill_u32, 4, np.uint32),
                                   (tk.tk_philox_fill_f32, oracle.philox_fill_f32, 4, np.float32),
                                   (tk.tk_philox_fill_u64, oracle.philox_fill_u64, 8, np.uint64),
                                   (tk.tk_philox_fill_f64, oracle.philox_fill_f64, 8, np.float64)):
            assert_bits_equal(run(fill, PK, s, isz, dt), orc(PK, s, N), f"{fill.__name__} s={s}")
        assert_bits_equal(run(tk.tk_philox_fill_u32_below, PK, s, 4, np.uint32, 1000),
                          oracle.philox_fill_u32_below(PK, s, N, 1000), f"philox u32_below s={s}")
        assert_bits_equal(run(tk.tk_philox_fill_u64_below, PK, s, 8, np.uint64, (1 << 63) + 1),
                          oracle.philox_fill_u64_below(PK, s, N, (1 << 63) + 1), f"philox u64_below s={s}")


def check_pairs():
    """Both Box-Muller pair fills at even and odd starts, lengths from one element to several
    tiles with ragged ends (the last tile's lanes past the end still feed their neighbours)."""
    for fill, orc in ((tk.tk_fill_normal_f32, oracle.fill_normal_f32),
                      (tk.tk_fill_normal_f32_half_turn, oracle.fill_normal_f32_half_turn)):
        for s in (0, 1, 3, 5, 255, (1 << 31) + 1):
            for n in (1, 2, 5, 1023, 1024, 1025, 4099, N):
                for off in (0, 1):
                    b = DevBuf(n, 4, 4 * off)
                    fill(KEY, s, n, b.ptr)
                    err = np.max(np.abs(b.host(np.float32).astype(np.float64) - orc(KEY, s, n)))
                    assert err <= 4e-6, f"{fill.__name__} s={s} n={n} off={off}: {err}"


def check_all():
    check_streaming()
    check_choice()
    check_exponential()
    check_normal_f64()


CASES = [
    ("unroll", 2, check_streaming), ("unroll", 4, check_streaming),
    ("max_blocks", 7, check_streaming), ("store_nt", 1, check_all),
    ("choice_tiles", 1, check_choice), ("choice_tiles", 4, check_choice), ("choice_tiles", 8, check_choice),
    ("exp_tiles", 1, check_exponential), ("exp_tiles", 4, check_exponential),
    ("zig_tiles", 1, check_normal_f64), ("zig_tiles", 2, check_normal_f64), ("zig_tiles", 8, check_normal_f64),
    ("zig_tiles", 16, check_normal_f64), ("zig_lds", 0, check_normal_f64), ("zig_fused", 0, check_normal_f64),
    ("const_work", 16, check_constant), ("const_work", 200, check_constant),
    ("philox_lds", 0, check_philox), ("philox_lds", 1, check_philox),
    ("pair_lds", 0, check_pairs), ("pair_lds", 1, check_pairs),
    ("lds_pad", 0, check_streaming), ("lds_pad", 49152, check_streaming), ("lds_pad", 49152, check_exponential),
    ("lds_pad", 16384, check_choice),
    ("zig_lds_pad", 16384, check_normal_f64),
]


@pytest.mark.parametrize("name,value,check", CASES, ids=[f"{n}={v}" for n, v, _ in CASES])
def test_launch_shape(name, value, check):
    log(f"tunable {name}={value}")
    tk.tk_debug_set_tunable(name, value)
    try:
        check()
    finally:
        tk.tk_debug_set_tunable(name, -1)
