"""Device allocation failure, forced through tk_debug_fail_allocations.

The library allocates device memory in three places: a device's ziggurat tables on its
first f64 normal fill, the two-kernel path's miss lists as they grow, and alias tables.
A failure there must return TK_ENOMEM, enqueue nothing, keep no memory the call had taken,
and let a later call allocate again.  The GPU case runs tests/alloc_failure_child.py in a
process of its own, since the per-device tables of this process may already exist."""
import os
import subprocess
import sys

import pytest

import bulk_fills_amd as tk

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_hook_arguments():
    assert tk.lib.tk_debug_device_bytes(None) == tk.TK_EINVAL
    import torch
    if not torch.cuda.is_available():  # no fill can have allocated anything
        assert tk.tk_debug_device_bytes() == 0
    tk.tk_debug_fail_allocations(2, 3)
    tk.tk_debug_fail_allocations(0, 0)


def run_child(args, extra_env=None):
    env = dict(os.environ)
    env.pop("TK_DEBUG_FAIL_ALLOC", None)
    env.update(extra_env or {})
    env["PYTHONPATH"] = os.pathsep.join([ROOT, HERE] + [p for p in [env.get("PYTHONPATH")] if p])
    print("alloc_failure_child.py", *args, flush=True)
    return subprocess.run([sys.executable, "-u", os.path.join(HERE, "alloc_failure_child.py")] + args, cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=110)


@pytest.mark.gpu
def test_failures_from_the_environment():
    r = run_child(["env"], {"TK_DEBUG_FAIL_ALLOC": "2"})
    print(r.stdout[-4000:], r.stderr[-4000:], flush=True)
    assert r.returncode == 0, f"exit status {r.returncode}"
    assert "alloc_failure_child: ok" in r.stdout
    assert r.stderr.count("TK_DEBUG_FAIL_ALLOC=2 is set") == 1  # announced once


def test_environment_hook_announces_itself():
    """TK_DEBUG_FAIL_ALLOC is read once and reported on stderr (no device needed: the hook
    call reads the environment before anything else)."""
    code = ("import ctypes, sys; lib = ctypes.CDLL(sys.argv[1]); "
            "lib.tk_debug_fail_allocations(0, 0); lib.tk_debug_fail_allocations(0, 0)")
    env = dict(os.environ, TK_DEBUG_FAIL_ALLOC="3")
    r = subprocess.run([sys.executable, "-c", code, tk.LIB_PATH], env=env, capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stderr.count("libtk: TK_DEBUG_FAIL_ALLOC=3 is set") == 1, r.stderr
    env.pop("TK_DEBUG_FAIL_ALLOC")
    r = subprocess.run([sys.executable, "-c", code, tk.LIB_PATH], env=env, capture_output=True, text=True,
                       timeout=60)
    assert "TK_DEBUG_FAIL_ALLOC" not in r.stderr


@pytest.mark.gpu
def test_forced_failures_in_a_fresh_process():
    r = run_child([])
    print(r.stdout[-4000:], r.stderr[-4000:], flush=True)
    assert r.returncode == 0, f"exit status {r.returncode}"
    assert "alloc_failure_child: ok" in r.stdout
