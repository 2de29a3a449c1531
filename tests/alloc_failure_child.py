"""Forced allocation failures, run by tests/test_alloc_failure.py in a process of its own so
that the library's per-device state is created here for the first time.

Each failed call must return TK_ENOMEM, leave its output untouched (it enqueues nothing)
and leave the library holding no more device memory than before it; the next call must
allocate again and fill exactly what the oracle fills.  Prints each step; exit status 0
when every check holds."""
import numpy as np
import torch

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import assert_bits_equal, log

SENTINEL = 7.0


def expect_enomem(fn, what):
    try:
        fn()
    except tk.TkError as e:
        assert e.code == tk.TK_ENOMEM, f"{what}: {e}"
        return
    raise AssertionError(f"{what}: the call succeeded")


def check_normal(out, want, path, what):
    got = out.cpu().numpy()
    exact = path != 2
    assert_bits_equal(got[exact], want[exact], what)
    if (~exact).any():
        assert np.max(np.abs(got[~exact] / want[~exact] - 1)) <= 1e-12, f"{what}: tail"


def untouched(out, what):
    torch.cuda.synchronize()
    assert bool((out == SENTINEL).all()), f"{what}: a refused fill wrote its output"


def main():
    n = (1 << 16) + 5
    dev = torch.device("cuda")
    out = torch.full((n,), SENTINEL, dtype=torch.float64, device=dev)
    want, path = oracle.fill_normal_f64(9, 2, n, with_path=True)
    assert tk.tk_debug_device_bytes() == 0, "device memory held before the first fill"

    # the first f64 normal fill on the device allocates the layer pairs, the f table and a
    # counter: fail each of the three in turn
    tk.tk_debug_set_normal_f64_mode(0)
    for skip in range(3):
        log(f"first fill, allocation {skip} fails")
        tk.tk_debug_fail_allocations(skip, 1)
        expect_enomem(lambda: tk.tk_fill_normal_f64(9, 2, n, out), f"first fill, allocation {skip}")
        held = tk.tk_debug_device_bytes()
        assert held == 0, f"first fill, allocation {skip}: {held} bytes held after the failure"
        untouched(out, f"first fill, allocation {skip}")
    tk.tk_debug_fail_allocations(0, 0)
    log("first fill after the failures")
    tk.tk_fill_normal_f64(9, 2, n, out)
    torch.cuda.synchronize()
    check_normal(out, want, path, "first fill after the failures")
    tables = tk.tk_debug_device_bytes()
    assert tables > 0

    # the two-kernel path allocates the miss counts, the slot arrays and the overflow list
    # on its first fill: fail each in turn
    tk.tk_debug_set_normal_f64_mode(1)
    for skip in range(3):
        log(f"two-kernel fill, allocation {skip} fails")
        out.fill_(SENTINEL)
        tk.tk_debug_fail_allocations(skip, 1)
        expect_enomem(lambda: tk.tk_fill_normal_f64(9, 2, n, out), f"two-kernel fill, allocation {skip}")
        held = tk.tk_debug_device_bytes()
        assert held == tables, f"two-kernel fill, allocation {skip}: {held} bytes held, {tables} before"
        untouched(out, f"two-kernel fill, allocation {skip}")
        # the failed fill's counts are gone with the lists
        try:
            tk.tk_debug_last_miss_count()
            raise AssertionError("a miss count after a failed fill")
        except tk.TkError as e:
            assert e.code == tk.TK_EINVAL, e
    tk.tk_debug_fail_allocations(0, 0)
    log("two-kernel fill after the failures")
    tk.tk_fill_normal_f64(9, 2, n, out)
    torch.cuda.synchronize()
    check_normal(out, want, path, "two-kernel fill after the failures")
    assert tk.tk_debug_last_miss_count() == int((path != 0).sum())
    lists = tk.tk_debug_device_bytes()
    assert lists > tables
    tk.tk_fill_normal_f64(9, 2, n, out)  # same size: no new allocation
    torch.cuda.synchronize()
    assert tk.tk_debug_device_bytes() == lists
    tk.tk_debug_set_normal_f64_mode(0)

    # alias tables: one allocation each (n columns padded to an even count)
    log("alias table, allocation fails")
    w = tk_inputs.zipf_weights()
    tk.tk_debug_fail_allocations(0, 1)
    expect_enomem(lambda: tk.tk_alias_create(w), "tk_alias_create")
    assert tk.tk_debug_device_bytes() == lists
    table = tk.tk_alias_create(w)
    assert tk.tk_debug_device_bytes() == lists + ((w.size + 1) & ~1) * 8
    ch = torch.empty(n, dtype=torch.int32, device=dev)
    tk.tk_fill_choice_u32(4, 0, n, table, ch)
    torch.cuda.synchronize()
    q, al, _ = oracle.alias_build(w)
    assert_bits_equal(ch.cpu().numpy().view(np.uint32), oracle.fill_choice_u32(4, 0, n, q, al), "choice")
    del table
    import gc
    gc.collect()
    assert tk.tk_debug_device_bytes() == lists, "a destroyed alias table is still counted"

    # a fill that allocates nothing is not affected by pending failures
    log("pending failures and a streaming fill")
    tk.tk_debug_fail_allocations(0, 5)
    u = torch.empty(n, dtype=torch.int32, device=dev)
    tk.tk_fill_u32(1, 3, n, u)
    torch.cuda.synchronize()
    assert_bits_equal(u.cpu().numpy().view(np.uint32), oracle.fill_u32(1, 3, n), "u32")
    tk.tk_debug_fail_allocations(0, 0)
    print("alloc_failure_child: ok", flush=True)


def env_mode():
    """Run with TK_DEBUG_FAIL_ALLOC=2: the first two fills fail (each at its first
    allocation), the third allocates and fills."""
    n = (1 << 12) + 3
    out = torch.full((n,), SENTINEL, dtype=torch.float64, device="cuda")
    for attempt in range(2):
        log(f"environment: fill {attempt} fails")
        expect_enomem(lambda: tk.tk_fill_normal_f64(5, 0, n, out), f"environment, fill {attempt}")
        assert tk.tk_debug_device_bytes() == 0
        untouched(out, f"environment, fill {attempt}")
    tk.tk_fill_normal_f64(5, 0, n, out)
    torch.cuda.synchronize()
    want, path = oracle.fill_normal_f64(5, 0, n, with_path=True)
    check_normal(out, want, path, "environment, third fill")
    print("alloc_failure_child: ok", flush=True)


if __name__ == "__main__":
    import sys
    env_mode() if sys.argv[1:] == ["env"] else main()
