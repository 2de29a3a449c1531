"""GPU parity of fused dropout and of the weighted choice fill against the oracle,
bit-exact (dropout's y and mask; choice indices and the uploaded alias table)."""
import numpy as np
import pytest
import torch

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import CANARY, DevBuf, assert_bits_equal, log

pytestmark = pytest.mark.gpu


def to_dev(a, offset_elems=0):
    """A device copy of host array `a` at an element offset inside a larger buffer."""
    isz = a.dtype.itemsize
    b = DevBuf(a.size, isz, offset_elems * isz)
    src = torch.from_numpy(a.view(np.uint8).copy()).to("cuda")
    b.buf[b.base:b.base + a.nbytes].copy_(src)
    return b


@pytest.mark.parametrize("p", [0.0, 0.1, 0.5, 0.999])
def test_dropout_sweep(p):
    x_all = tk_inputs.normal_x((1 << 18) + 64, seed=3)
    x_all[:4] = [0.0, -0.0, np.inf, -3.5e-39]  # signed zero, infinity, subnormal
    for s in (0, 1, 3, 5):
        for n in (1, 3, 4, 5, 17, 4097, (1 << 18) + 7):
            for xo, yo, mo in ((0, 0, 0), (1, 1, 1), (0, 1, 2), (3, 0, 1)):
                x = x_all[:n]
                xb, yb, mb = to_dev(x, xo), DevBuf(n, 4, yo * 4), DevBuf(n, 1, mo)
                tk.tk_dropout_f32(8, s, n, p, xb.ptr, yb.ptr, mb.ptr)
                y, m = oracle.dropout_f32(8, s, x, p)
                assert_bits_equal(yb.host(np.float32), y, f"y p={p} s={s} n={n} offs={(xo, yo, mo)}")
                assert_bits_equal(mb.host(np.uint8), m, f"mask p={p} s={s} n={n}")


def test_dropout_in_place_and_without_mask():
    n = (1 << 20) + 3
    x = tk_inputs.normal_x(n, seed=4)
    xb = to_dev(x)
    tk.tk_dropout_f32(8, 0, n, 0.1, xb.ptr, xb.ptr)
    assert_bits_equal(xb.host(np.float32), oracle.dropout_f32(8, 0, x, 0.1, with_mask=False), "in place")


def test_dropout_full_workload_sampled():
    """X = f32[2^20, 256] ~ N(0, 1) (seeded numpy), p = 0.1, key 8, counter = flat index."""
    n = tk_inputs.DROPOUT_ROWS * tk_inputs.DROPOUT_COLS
    x = tk_inputs.normal_x(n)
    xb = to_dev(x)
    yb, mb = DevBuf(n, 4), DevBuf(n, 1)
    log("dropout full")
    tk.tk_dropout_f32(tk_inputs.DROPOUT_KEY, 0, n, tk_inputs.DROPOUT_P, xb.ptr, yb.ptr, mb.ptr)
    idx = tk_inputs.sample_indices(n, m=1 << 18, seed=16)
    y, m = oracle.dropout_f32(tk_inputs.DROPOUT_KEY, 0, x[idx], tk_inputs.DROPOUT_P, draws=idx.astype(np.uint64))
    assert_bits_equal(yb.sample(idx, np.float32), y, "y")
    assert_bits_equal(mb.sample(idx, np.uint8), m, "mask")
    keep = mb.sample(np.arange(0, n, 4099), np.uint8).mean()
    assert abs(keep - 0.9) < 0.01


@pytest.mark.parametrize("weights", [
    [1.0], [2.0, 1.0], [1.0, 2.0, 3.0], [0.0, 5.0, 0.0, 1.0], list(tk_inputs.zipf_weights()),
    list(np.random.default_rng(9).random(5000)), list(np.random.default_rng(11).random(8191) + 0.1),
    list(np.random.default_rng(12).random(8192) + 0.1), list(np.random.default_rng(10).random(10000) + 0.5),
])
def test_choice(weights):
    table = tk.tk_alias_create(weights)
    try:
        q, a = table.export()
        qo, ao, _ = oracle.alias_build(weights)
        assert np.array_equal(q, qo) and np.array_equal(a, ao)
        for s in (0, 1, 3):
            for n in (1, 3, 5, 17, 4099, (1 << 20) + 1):
                for off in (0, 1, 2):
                    b = DevBuf(n, 4, off * 4)
                    tk.tk_fill_choice_u32(1, s, n, table, b.ptr)
                    assert_bits_equal(b.host(np.uint32), oracle.fill_choice_u32(1, s, n, qo, ao),
                                      f"n_w={len(weights)} s={s} n={n} off={off}")
    finally:
        table.close()


def test_choice_full_workload_sampled():
    w = tk_inputs.zipf_weights()
    table = tk.tk_alias_create(w)
    q, a, _ = oracle.alias_build(w)
    n = tk_inputs.FULL_N
    b = DevBuf(n, 4)
    idx = tk_inputs.sample_indices(n, seed=17)
    try:
        log("choice full")
        tk.tk_fill_choice_u32(1, 0, n, table, b.ptr)
        assert_bits_equal(b.sample(idx, np.uint32), oracle.fill_choice_u32(1, 0, None, q, a, draws=idx.astype(np.uint64)))
        counts = np.bincount(b.host(np.uint32), minlength=w.size)
        assert counts.sum() == n and counts[0] > counts[-1]
    finally:
        table.close()
    assert CANARY == 0xA5
