"""GPU parity of the per-element device API (include/tk_device_api.h) and of dropout
backward by redrawing.

Kernels written against the header (tests/api_kernels.hip, built with the compiler's
default floating-point flags) must give the library's fills bit for bit -- uniform f32
and f64, Box-Muller pairs, the one-normal-per-counter randn (the even elements of the
normal fill) and Phobos's dropout_rows -- and match the oracle (bit-exact, or within the
Box-Muller tolerance of 4e-6).  tk_dropout_backward_f32 must reproduce the forward call's
mask decisions without reading the mask: dx = mask ? dy / (1 - p) : +0."""
import ctypes as C
import os

import numpy as np
import pytest
import torch

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import DevBuf, assert_bits_equal, log

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
F32_ABS = 4e-6


@pytest.fixture(scope="module")
def api():
    path = os.path.join(HERE, "libtk_api_kernels.so")
    if not os.path.exists(path):
        import build_api_kernels
        build_api_kernels.build()
    lib = C.CDLL(path)
    u32, p = C.c_uint32, C.c_void_p
    for name in ("tkt_uniform_f32", "tkt_uniform_f64", "tkt_randn_f32", "tkt_randn2_f32"):
        getattr(lib, name).argtypes = [u32, u32, u32, p, p]
        getattr(lib, name).restype = C.c_int
    lib.tkt_dropout_rows.argtypes = [u32, u32, C.c_float, p, p, p]
    lib.tkt_dropout_rows.restype = C.c_int
    return lib


def stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def launch(rc):
    assert rc == 0, f"launch failed: hipError {rc}"


def to_dev(a):
    b = DevBuf(a.size, a.dtype.itemsize)
    b.buf[b.base:b.base + a.nbytes].copy_(torch.from_numpy(a.view(np.uint8).copy()).to("cuda"))
    return b


@pytest.mark.parametrize("c0", [0, 5, (1 << 32) - 4099])
def test_uniform_f32(api, c0):
    n = 4097
    a, f = DevBuf(n, 4), DevBuf(n, 4)
    launch(api.tkt_uniform_f32(3, c0, n, a.ptr, stream()))
    tk.tk_fill_f32(3, c0, n, f.ptr)
    got = a.host(np.float32)
    assert_bits_equal(got, f.host(np.float32), "api vs fill")
    assert_bits_equal(got, oracle.fill_f32(3, c0, n), "api vs oracle")


def test_uniform_f64(api):
    n = (1 << 20) + 3
    a, f = DevBuf(n, 8), DevBuf(n, 8)
    launch(api.tkt_uniform_f64(2, 17, n, a.ptr, stream()))
    tk.tk_fill_f64(2, 17, n, f.ptr)
    got = a.host(np.float64)
    assert_bits_equal(got, f.host(np.float64), "api vs fill")
    assert_bits_equal(got, oracle.fill_f64(2, 17, n), "api vs oracle")


@pytest.mark.parametrize("c0", [0, 7])
def test_randn_pairs_and_single(api, c0):
    """Pairs c0 .. c0+m-1 are fill elements 2 c0 .. 2 (c0+m) - 1; randn(c) is element 2c."""
    m = (1 << 20) + 1
    pairs, single, f = DevBuf(2 * m, 4), DevBuf(m, 4), DevBuf(2 * m, 4)
    launch(api.tkt_randn2_f32(5, c0, m, pairs.ptr, stream()))
    launch(api.tkt_randn_f32(5, c0, m, single.ptr, stream()))
    tk.tk_fill_normal_f32(5, 2 * c0, 2 * m, f.ptr)
    fill = f.host(np.float32)
    got = pairs.host(np.float32)
    assert_bits_equal(got, fill, "pairs vs fill")
    assert_bits_equal(single.host(np.float32), fill[0::2].copy(), "randn vs even fill elements")
    want = oracle.fill_normal_f32(5, 2 * c0, 2 * m)
    err = np.max(np.abs(got.astype(np.float64) - want.astype(np.float64)))
    log(f"randn pairs c0={c0}: max abs err vs oracle {err:.2e}")
    assert err <= F32_ABS


@pytest.mark.parametrize("rows", [1, 15, 17, 1 << 16])
def test_dropout_rows(api, rows):
    """Phobos's dropout_rows: Y = dropout(X, 0.1, key, flat index), X ~ N(0, 1)."""
    n = rows * 256
    x = tk_inputs.normal_x(n, seed=21)
    xb = to_dev(x)
    y_api, y_fill = DevBuf(n, 4), DevBuf(n, 4)
    launch(api.tkt_dropout_rows(8, rows, 0.1, xb.ptr, y_api.ptr, stream()))
    tk.tk_dropout_f32(8, 0, n, 0.1, xb.ptr, y_fill.ptr)
    got = y_api.host(np.float32)
    assert_bits_equal(got, y_fill.host(np.float32), "api vs fill")
    assert_bits_equal(got, oracle.dropout_f32(8, 0, x, 0.1, with_mask=False), "api vs oracle")


@pytest.mark.parametrize("p", [0.0, 0.1, 0.5])
def test_dropout_backward_redraws_the_mask(p):
    for s in (0, 3):
        for n in (1, 5, 4097, (1 << 20) + 3):
            x = tk_inputs.normal_x(n, seed=22)
            dy = tk_inputs.normal_x(n, seed=23)
            xb, dyb = to_dev(x), to_dev(dy)
            yb, mb, dxb = DevBuf(n, 4), DevBuf(n, 1), DevBuf(n, 4)
            tk.tk_dropout_f32(9, s, n, p, xb.ptr, yb.ptr, mb.ptr)
            tk.tk_dropout_backward_f32(9, s, n, p, dyb.ptr, dxb.ptr)
            mask = mb.host(np.uint8)
            dx = dxb.host(np.float32)
            q = np.float32(1.0) - np.float32(p)
            want = np.where(mask == 1, dy / q, np.float32(0.0)).astype(np.float32)
            assert_bits_equal(dx, want, f"dx from the stored mask p={p} s={s} n={n}")
            assert_bits_equal(dx, oracle.dropout_f32(9, s, dy, p, with_mask=False), f"dx vs oracle p={p} s={s} n={n}")
            tk.tk_dropout_backward_f32(9, s, n, p, dyb.ptr, dyb.ptr)  # in place
            assert_bits_equal(dyb.host(np.float32), want, f"in place p={p} s={s} n={n}")
