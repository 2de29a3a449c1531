"""GPU parity at the top of each fill's counter space: the last draws a fill may take
(draw limits of include/tk.h) against the oracle, with a ragged length and a misaligned
output, for every family not covered by the uniform and bounded edge tests."""
import numpy as np
import pytest

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import DevBuf, assert_bits_equal

pytestmark = pytest.mark.gpu

N = 4099
PK = 0x0123456789ABCDEF
W31, W32, W63, W64 = 1 << 31, 1 << 32, 1 << 63, 1 << 64


def run(fill, key, start, isz, dtype, *args, off=1):
    b = DevBuf(N, isz, off * isz)
    fill(key, start, N, *args, b.ptr)
    return b.host(dtype)


def close(got, want, tol, what):
    err = float(np.max(np.abs(got.astype(np.float64) - want.astype(np.float64))))
    assert err <= tol, f"{what}: max abs err {err}"


def test_normal_f64_edge():
    got = run(tk.tk_fill_normal_f64, 3, W31 - N, 8, np.float64)
    want, path = oracle.fill_normal_f64(3, W31 - N, N, with_path=True)
    exact = path != 2
    assert_bits_equal(got[exact], want[exact], "normal_f64 non-tail")
    if (~exact).any():
        assert np.max(np.abs(got[~exact] / want[~exact] - 1)) <= 1e-12


def test_philox_normal_f64_edge():
    got = run(tk.tk_philox_fill_normal_f64, PK, W63 - N, 8, np.float64)
    want, path = oracle.philox_fill_normal_f64(PK, W63 - N, N, with_path=True)
    exact = path != 2
    assert_bits_equal(got[exact], want[exact], "philox normal_f64 non-tail")
    if (~exact).any():
        assert np.max(np.abs(got[~exact] / want[~exact] - 1)) <= 1e-12


@pytest.mark.parametrize("name", ["normal_f32", "half_turn", "randn", "philox_normal_f32"])
def test_f32_normals_edge(name):
    fill, orc, key, top = {
        "normal_f32": (tk.tk_fill_normal_f32, oracle.fill_normal_f32, 3, W32),
        "half_turn": (tk.tk_fill_normal_f32_half_turn, oracle.fill_normal_f32_half_turn, 3, W32),
        "randn": (tk.tk_fill_randn_f32, oracle.fill_randn_f32, 3, W31),
        "philox_normal_f32": (tk.tk_philox_fill_normal_f32, oracle.philox_fill_normal_f32, PK, W64),
    }[name]
    close(run(fill, key, top - N, 4, np.float32), orc(key, top - N, N), 4e-6, name)


def test_exponentials_edge():
    assert_bits_equal(run(tk.tk_fill_exponential_f32, 5, W32 - N, 4, np.float32),
                      oracle.fill_exponential_f32(5, W32 - N, N), "exponential_f32")
    got = run(tk.tk_fill_exponential_f64, 5, W31 - N, 8, np.float64)
    want = oracle.fill_exponential_f64(5, W31 - N, N)
    assert np.max(np.abs(got.view(np.int64) - want.view(np.int64))) <= 2


def test_bounded_and_choice_edge():
    assert_bits_equal(run(tk.tk_philox_fill_u32_below, PK, W64 - N, 4, np.uint32, (1 << 31) + 1),
                      oracle.philox_fill_u32_below(PK, W64 - N, N, (1 << 31) + 1), "philox u32_below")
    assert_bits_equal(run(tk.tk_philox_fill_u64_below, PK, W63 - N, 8, np.uint64, (1 << 63) + 1),
                      oracle.philox_fill_u64_below(PK, W63 - N, N, (1 << 63) + 1), "philox u64_below")
    w = tk_inputs.zipf_weights()
    table = tk.tk_alias_create(w)
    q, al, _ = oracle.alias_build(w)
    assert_bits_equal(run(tk.tk_fill_choice_u32, 2, W31 - N, 4, np.uint32, table),
                      oracle.fill_choice_u32(2, W31 - N, N, q, al), "choice")
    assert_bits_equal(run(tk.tk_philox_fill_choice_u32, PK, W63 - N, 4, np.uint32, table),
                      oracle.philox_fill_choice_u32(PK, W63 - N, N, q, al), "philox choice")
    table.close()


def test_dropout_edge():
    x = tk_inputs.normal_x(N, seed=41)
    xb = DevBuf(N, 4)
    import torch
    xb.buf[xb.base:xb.base + x.nbytes].copy_(torch.from_numpy(x.view(np.uint8).copy()).to("cuda"))
    yb, mb = DevBuf(N, 4, 4), DevBuf(N, 1, 3)
    tk.tk_dropout_f32(8, W32 - N, N, 0.1, xb.ptr, yb.ptr, mb.ptr)
    y, m = oracle.dropout_f32(8, W32 - N, x, 0.1)
    assert_bits_equal(yb.host(np.float32), y, "dropout y")
    assert_bits_equal(mb.host(np.uint8), m, "dropout mask")
