"""GPU parity of the normal fills against the oracle.

f64 (1024-layer ziggurat): every fast-path and wedge value bit-exact, tail values within
1e-12 relative (the device and host logarithms may differ in the last bit); the number of
draws that left the fast path equals the oracle's; forcing the miss list to overflow
(the continuation pass then walks the whole fill) gives the same bits; fills on two
streams sharing the per-device list stay correct.
f32 (Box-Muller pairs): within 4e-6 absolute everywhere (|x| < 5.65)."""
import numpy as np
import pytest
import torch

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import DevBuf, log

pytestmark = pytest.mark.gpu

TAIL_REL = 1e-12
F32_ABS = 4e-6
MODES = {"default": 0, "two_kernels": 1, "fused": 2}


@pytest.fixture(params=sorted(MODES))
def f64_mode(request):
    """Runs a test once per way of finishing the misses (results must be identical): the
    library default (fused, uncounted, no per-device state), and each path chosen by the
    test hook, which also keeps the miss counts."""
    tk.tk_debug_set_normal_f64_mode(MODES[request.param])
    yield request.param
    tk.tk_debug_set_normal_f64_mode(0)


def miss_count(mode):
    """The last fill's miss count, or None after an uncounted default fill (which the hook
    must refuse)."""
    if mode == "default":
        with pytest.raises(tk.TkError):
            tk.tk_debug_last_miss_count()
        return None
    return tk.tk_debug_last_miss_count()


def check_f64(got, key, start, n=None, draws=None, what=""):
    want, path = oracle.fill_normal_f64(key, start, n, draws=draws, with_path=True)
    exact = path != 2
    bad = np.flatnonzero(got[exact].view(np.uint64) != want[exact].view(np.uint64))
    assert bad.size == 0, (f"{what}: {bad.size} non-tail mismatches; first at {np.flatnonzero(exact)[bad[0]]}: "
                           f"got {got[exact][bad[0]]!r} want {want[exact][bad[0]]!r} path {path[exact][bad[0]]}")
    t = ~exact
    if t.any():
        rel = np.abs(got[t] - want[t]) / np.abs(want[t])
        assert rel.max() <= TAIL_REL, f"{what}: tail rel err {rel.max()}"
    return int((path != 0).sum())


def run_f64(key, start, n, off=0):
    b = DevBuf(n, 8, off * 8)
    tk.tk_fill_normal_f64(key, start, n, b.ptr)
    return b.host(np.float64)


def test_f64_small_sweep(f64_mode):
    for off in (0, 1):
        for s in (0, 1, 2, 3, 5, 17):
            for n in (1, 2, 3, 5, 16, 17, 255, 4097):
                check_f64(run_f64(1, s, n, off), 1, s, n, what=f"s={s} n={n} off={off}")


@pytest.mark.parametrize("key", (1, 2, 3, 0xFFFFFFFF))
def test_f64_many_tiles_and_miss_count(key, f64_mode):
    n = (1 << 20) + 3
    for s in tk_inputs.STARTS:
        for off in (0, 1):
            log(f"normal_f64 key={key} start={s} off={off}")
            got = run_f64(key, s, n, off)
            misses = check_f64(got, key, s, n, what=f"key={key} s={s}")
            assert miss_count(f64_mode) in (None, misses)


def test_f64_full_2p24_every_element(f64_mode):
    n = 1 << 24
    for s in tk_inputs.STARTS:
        log(f"normal_f64 2^24 start={s}")
        got = run_f64(1, s, n)
        misses = check_f64(got, 1, s, n, what=f"2^24 s={s}")
        assert miss_count(f64_mode) in (None, misses)
        assert abs(misses / n - 0.0042765667) < 5 * np.sqrt(0.0043 / n)


def test_f64_full_2p28_sampled(f64_mode):
    n = tk_inputs.FULL_N
    b = DevBuf(n, 8)
    idx = tk_inputs.sample_indices(n, seed=14)
    for s in tk_inputs.STARTS:
        log(f"normal_f64 2^28 start={s}")
        tk.tk_fill_normal_f64(1, s, n, b.ptr)
        check_f64(b.sample(idx, np.float64), 1, 0, draws=idx.astype(np.uint64) + s, what=f"2^28 s={s}")
        misses = miss_count(f64_mode)
        if misses is not None:
            assert abs(misses - 0.0042765667 * n) < 6 * np.sqrt(0.0043 * n), misses


def test_f64_sampled_misses_at_full_size(f64_mode):
    """Every element that leaves the fast path within the first 2^22 of a 2^28 fill."""
    n = tk_inputs.FULL_N
    m = 1 << 22
    _, path = oracle.fill_normal_f64(1, 0, m, with_path=True)
    miss = np.flatnonzero(path != 0)
    b = DevBuf(n, 8)
    tk.tk_fill_normal_f64(1, 0, n, b.ptr)
    check_f64(b.sample(miss, np.float64), 1, 0, draws=miss.astype(np.uint64), what="misses")


def test_f64_forced_list_overflow():
    """Two kernels: shrinking the per-group slots pushes misses to the overflow list, and
    shrinking that too makes the continuation pass walk the whole fill.  Fused: a group
    whose misses exceed its queue walks its own elements again.  No bit may change."""
    n = (1 << 20) + 1
    tk.tk_debug_set_normal_f64_mode(2)
    want = run_f64(4, 3, n)
    total = tk.tk_debug_last_miss_count()
    try:
        for mode in (1, 2):  # two kernels: slot -> overflow list -> whole-fill walk; fused: group re-walk
            tk.tk_debug_set_normal_f64_mode(mode)
            for per_group, overflow in ((2, 1 << 22), (1, 1 << 22), (1, 1), (3, 16), (16, 1)):
                tk.tk_debug_set_miss_capacity(per_group, overflow)
                got = run_f64(4, 3, n)
                assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), (mode, per_group, overflow)
                assert tk.tk_debug_last_miss_count() == total, (mode, per_group, overflow)
    finally:
        tk.tk_debug_set_miss_capacity(0, 0)
        tk.tk_debug_set_normal_f64_mode(0)
    check_f64(run_f64(4, 3, n), 4, 3, n, what="after reset")


def test_f64_two_streams_share_the_list(f64_mode):
    n = (1 << 20) + 7
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs = [DevBuf(n, 8) for _ in range(4)]
    for j, b in enumerate(bufs):
        tk.tk_fill_normal_f64(10 + j, j, n, b.ptr, stream=streams[j % 2])
    torch.cuda.synchronize()
    for j, b in enumerate(bufs):
        check_f64(b.host(np.float64), 10 + j, j, n, what=f"stream fill {j}")


def f32_err(got, key, start, n=None, draws=None):
    want = oracle.fill_normal_f32(key, start, n, draws=draws)
    return float(np.max(np.abs(got.astype(np.float64) - want.astype(np.float64)))) if want.size else 0.0


def run_f32(key, start, n, off=0):
    b = DevBuf(n, 4, off * 4)
    tk.tk_fill_normal_f32(key, start, n, b.ptr)
    return b.host(np.float32)


def test_f32_small_sweep():
    for off in (0, 1, 3):
        for s in (0, 1, 2, 3, 5, 16, 17):
            for n in (1, 2, 3, 4, 5, 7, 65, 4097):
                assert f32_err(run_f32(2, s, n, off), 2, s, n) <= F32_ABS, (s, n, off)


def test_f32_many_tiles_and_all_grid_points():
    """2^24 elements cover all 2^23 values of the first uniform about once each, including
    the smallest 1 - u1 (largest radius) and u1 = 0."""
    for s in (0, 1):
        for key in (1, 5):
            n = 1 << 24
            log(f"normal_f32 key={key} start={s}")
            got = run_f32(key, s, n)
            err = f32_err(got, key, s, n)
            log(f"  max abs err {err:.3e}")
            assert err <= F32_ABS
            assert np.abs(got).max() <= 5.6468


def test_f32_full_2p28_sampled():
    n = tk_inputs.FULL_N
    b = DevBuf(n, 4)
    idx = tk_inputs.sample_indices(n, seed=15)
    for s in tk_inputs.STARTS:
        tk.tk_fill_normal_f32(1, s, n, b.ptr)
        assert f32_err(b.sample(idx, np.float32), 1, 0, draws=idx.astype(np.uint64) + s) <= F32_ABS


def test_host_threads_share_the_device_state(f64_mode):
    """Any host thread may call (include/tk.h): four threads, each with its own stream,
    fill normals and exponentials at once (ctypes releases the GIL during the calls).  In
    the default mode the fills share only the constant layer tables and run concurrently;
    in the counted modes they race on the per-device state's mutex and event.  Every
    result must equal the oracle's."""
    import threading
    n = (1 << 19) + 5
    keys = [21, 22, 23, 24]
    bufs = {k: (DevBuf(n, 8), DevBuf(n, 4)) for k in keys}
    errors = []
    torch.cuda.synchronize()

    def work(key):
        try:
            s = torch.cuda.Stream()
            for rep in range(6):
                tk.tk_fill_normal_f64(key, rep, n, bufs[key][0].ptr, stream=s)
                tk.tk_fill_exponential_f32(key, rep, n, bufs[key][1].ptr, stream=s)
            s.synchronize()
        except Exception as e:  # reported after the join
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(k,)) for k in keys]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in keys:
        check_f64(bufs[k][0].host(np.float64), k, 5, n, what=f"thread key {k}")
        got = bufs[k][1].host(np.float32)
        assert np.array_equal(got.view(np.uint32), oracle.fill_exponential_f32(k, 5, n).view(np.uint32)), k
