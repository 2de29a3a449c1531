"""The C ABI on the CPU: the library loads, exports every symbol include/tk.h declares,
and refuses bad arguments before any HIP call (so no device is needed here).  Also checks
the library's host-side tables against the oracle's independent builds, bit for bit."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import bulk_fills_amd as tk
import oracle
import tk_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "tk.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tk_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 30
    raw = C.CDLL(tk.LIB_PATH)
    missing = [n for n in names if not hasattr(raw, n)]
    assert not missing, missing
    assert set(tk.SIGNATURES) | {"tk_status_string", "tk_last_hip_error", "tk_alias_size"} >= set(names)


def test_binding_names_match_the_c_abi():
    for name in declared_functions():
        if name in ("tk_status_string", "tk_last_hip_error", "tk_alias_size", "tk_alias_destroy", "tk_alias_export"):
            continue
        assert hasattr(tk, name), name


L = tk.lib
FAKE = 0x10000  # never dereferenced: every call below is refused before any launch
U32MAX = (1 << 32) - 1

SIMPLE = [("tk_fill_u8", 1, 1 << 34), ("tk_fill_u16", 2, 1 << 33), ("tk_fill_u32", 4, 1 << 32),
          ("tk_fill_u64", 8, 1 << 31), ("tk_fill_f16_bits", 2, 1 << 33), ("tk_fill_f32", 4, 1 << 32),
          ("tk_fill_f64", 8, 1 << 31), ("tk_fill_bool", 1, 1 << 37), ("tk_fill_normal_f64", 8, 1 << 31),
          ("tk_fill_normal_f32", 4, 1 << 32), ("tk_fill_exponential_f64", 8, 1 << 31),
          ("tk_fill_exponential_f32", 4, 1 << 32), ("tk_fill_normal_f32_half_turn", 4, 1 << 32),
          ("tk_fill_randn_f32", 4, 1 << 31)]


@pytest.mark.parametrize("name,size,limit", SIMPLE)
def test_simple_fill_validation(name, size, limit):
    f = getattr(L, name)
    assert f(1, 0, 0, None, None) == tk.TK_OK          # n == 0: nothing to do
    assert f(1, 0, 0, FAKE + 1, None) == tk.TK_OK      # not even the pointer is looked at
    assert f(1, 0, 5, None, None) == tk.TK_EINVAL      # NULL output
    if size > 1:
        assert f(1, 0, 5, FAKE + 1, None) == tk.TK_EINVAL  # not element aligned
    assert f(1, limit - 1, 2, FAKE, None) == tk.TK_ERANGE   # crosses the counter space
    assert f(1, limit, 1, FAKE, None) == tk.TK_ERANGE
    assert f(1, 1 << 63, 1 << 63, FAKE, None) == tk.TK_ERANGE  # start + n overflows


def test_bounded_validation():
    assert L.tk_fill_u32_below(1, 0, 4, 0, FAKE, None) == tk.TK_EINVAL
    assert L.tk_fill_u64_below(1, 0, 4, 0, FAKE, None) == tk.TK_EINVAL
    assert L.tk_fill_u32_below(1, U32MAX, 2, 7, FAKE, None) == tk.TK_ERANGE
    assert L.tk_fill_u64_below(1, 1 << 31, 1, 7, FAKE, None) == tk.TK_ERANGE
    assert L.tk_fill_i32_below(1, 0, 4, (1 << 31) - 10, 11, FAKE, None) == tk.TK_ERANGE
    assert L.tk_fill_i32_below(1, 0, 4, 0, 0, FAKE, None) == tk.TK_EINVAL
    assert L.tk_fill_i64_below32(1, 0, 4, (1 << 63) - 10, 11, FAKE, None) == tk.TK_ERANGE
    assert L.tk_fill_i64_below(1, 0, 4, (1 << 63) - 10, 11, FAKE, None) == tk.TK_ERANGE
    assert L.tk_fill_i64_below(1, 0, 4, 0, 0, FAKE, None) == tk.TK_EINVAL
    assert L.tk_fill_i32_below(1, 0, 0, 0, 0, None, None) == tk.TK_EINVAL  # bound is checked first


def test_dropout_validation():
    for p in (1.0, -0.25, float("nan"), float("inf")):
        assert L.tk_dropout_f32(1, 0, 4, p, FAKE, FAKE + 64, None, None) == tk.TK_EINVAL
    assert L.tk_dropout_f32(1, 0, 4, 0.1, None, FAKE, None, None) == tk.TK_EINVAL
    assert L.tk_dropout_f32(1, 0, 4, 0.1, FAKE, FAKE + 2, None, None) == tk.TK_EINVAL   # misaligned y
    assert L.tk_dropout_f32(1, 0, 8, 0.1, FAKE, FAKE + 4, None, None) == tk.TK_EINVAL   # partial overlap
    assert L.tk_dropout_f32(1, U32MAX, 2, 0.1, FAKE, FAKE + 64, None, None) == tk.TK_ERANGE
    assert L.tk_dropout_f32(1, 0, 0, 0.1, None, None, None, None) == tk.TK_OK
    for p in (-0.1, 1.0, float("nan")):
        assert L.tk_dropout_backward_f32(1, 0, 4, p, FAKE, FAKE + 64, None) == tk.TK_EINVAL
    assert L.tk_dropout_backward_f32(1, 0, 4, 0.1, None, FAKE, None) == tk.TK_EINVAL
    assert L.tk_dropout_backward_f32(1, 0, 8, 0.1, FAKE, FAKE + 4, None) == tk.TK_EINVAL
    assert L.tk_dropout_backward_f32(1, U32MAX, 2, 0.1, FAKE, FAKE + 64, None) == tk.TK_ERANGE
    assert L.tk_dropout_backward_f32(1, 0, 0, 0.1, None, None, None) == tk.TK_OK


def test_choice_and_alias_validation():
    w = np.ones(4)
    h = C.c_void_p()
    assert L.tk_alias_create(None, 4, C.byref(h)) == tk.TK_EINVAL
    assert L.tk_alias_create(w.ctypes.data, 0, C.byref(h)) == tk.TK_EINVAL
    for bad in ([1.0, -1.0], [0.0, 0.0], [1.0, float("nan")], [1.0, float("inf")]):
        b = np.array(bad)
        assert L.tk_alias_create(b.ctypes.data, b.size, C.byref(h)) == tk.TK_EINVAL
    assert L.tk_fill_choice_u32(1, 0, 4, None, FAKE, None) == tk.TK_EINVAL
    assert L.tk_alias_destroy(None) == tk.TK_EINVAL
    assert L.tk_alias_size(None) == 0


def test_philox_validation():
    assert L.tk_philox_fill_u32(1, 0, 4, None, None) == tk.TK_EINVAL
    assert L.tk_philox_fill_u32(1, (1 << 64) - 1, 2, FAKE, None) == tk.TK_ERANGE
    assert L.tk_philox_fill_u64(1, 1 << 63, 1, FAKE, None) == tk.TK_ERANGE
    assert L.tk_philox_fill_f64(1, 0, 4, FAKE + 4, None) == tk.TK_EINVAL


def test_philox_variant_validation():
    top = (1 << 64) - 1
    assert L.tk_philox_fill_u32_below(1, 0, 4, 0, FAKE, None) == tk.TK_EINVAL
    assert L.tk_philox_fill_u32_below(1, 0, 4, 7, None, None) == tk.TK_EINVAL
    assert L.tk_philox_fill_u32_below(1, top, 2, 7, FAKE, None) == tk.TK_ERANGE
    assert L.tk_philox_fill_u32_below(1, 0, 0, 0, None, None) == tk.TK_EINVAL  # bound first
    assert L.tk_philox_fill_u64_below(1, 0, 4, 0, FAKE, None) == tk.TK_EINVAL
    assert L.tk_philox_fill_u64_below(1, 1 << 63, 1, 5, FAKE, None) == tk.TK_ERANGE
    assert L.tk_philox_fill_u64_below(1, 0, 4, 5, FAKE + 4, None) == tk.TK_EINVAL
    assert L.tk_philox_fill_normal_f32(1, top, 2, FAKE, None) == tk.TK_ERANGE
    assert L.tk_philox_fill_normal_f32(1, 0, 4, FAKE + 2, None) == tk.TK_EINVAL
    assert L.tk_philox_fill_normal_f64(1, 1 << 63, 1, FAKE, None) == tk.TK_ERANGE
    assert L.tk_philox_fill_normal_f64(1, 0, 1 << 32, FAKE, None) == tk.TK_EINVAL  # n per call
    assert L.tk_philox_fill_normal_f64(1, 0, 0, None, None) == tk.TK_OK
    assert L.tk_philox_fill_choice_u32(1, 0, 4, None, FAKE, None) == tk.TK_EINVAL


def test_no_alloc_normal_validation():
    f = L.tk_fill_normal_f64_no_alloc
    assert f(1, 0, 0, None, None) == tk.TK_OK
    assert f(1, 0, 4, None, None) == tk.TK_EINVAL
    assert f(1, 0, 4, FAKE + 4, None) == tk.TK_EINVAL       # not 8-byte aligned
    assert f(1, 0, (1 << 24) + 1, FAKE, None) == tk.TK_EINVAL  # beyond the per-call limit
    assert f(1, (1 << 31) - 1, 2, FAKE, None) == tk.TK_ERANGE


_ALIAS_OOM_CHILD = """
import ctypes as C, resource, sys
import numpy as np
lib = C.CDLL(sys.argv[1])
n = 1 << 24
w = np.ones(n)
q = np.empty(n, dtype=np.uint32)
a = np.empty(n, dtype=np.uint32)
lib.tk_alias_build_host.argtypes = [C.c_void_p, C.c_uint32, C.c_void_p, C.c_void_p]
lib.tk_alias_create.argtypes = [C.c_void_p, C.c_uint32, C.c_void_p]
ok = lib.tk_alias_build_host(w.ctypes.data, n, q.ctypes.data, a.ctypes.data)
used = int(open("/proc/self/statm").read().split()[0]) * resource.getpagesize()
resource.setrlimit(resource.RLIMIT_AS, (used + (64 << 20), resource.RLIM_INFINITY))
bad = lib.tk_alias_build_host(w.ctypes.data, n, q.ctypes.data, a.ctypes.data)
h = C.c_void_p()
bad2 = lib.tk_alias_create(w.ctypes.data, n, C.byref(h))
print(ok, bad, bad2, h.value is None)
"""


def test_alias_host_allocation_failure_is_enomem():
    """A host allocation failure while building a 2^24-column table (forced in a child
    process by an address-space limit) returns TK_ENOMEM through the C ABI and creates no
    handle, instead of ending the caller with an exception."""
    import subprocess
    import sys
    out = subprocess.run([sys.executable, "-c", _ALIAS_OOM_CHILD, tk.LIB_PATH], check=True,
                         capture_output=True, text=True, timeout=120).stdout.split()
    assert out == [str(tk.TK_OK), str(tk.TK_ENOMEM), str(tk.TK_ENOMEM), "True"], out


def test_constant_fill_validation():
    assert L.tk_fill_constant_u32(7, 0, None, None) == tk.TK_OK
    assert L.tk_fill_constant_u32(7, 4, None, None) == tk.TK_EINVAL
    assert L.tk_fill_constant_u32(7, 4, FAKE + 2, None) == tk.TK_EINVAL
    assert L.tk_fill_constant_u32(7, 1 << 62, FAKE, None) == tk.TK_ERANGE


def test_status_strings():
    for code in range(5):
        s = L.tk_status_string(code).decode()
        assert s.startswith(["TK_OK", "TK_EINVAL", "TK_ERANGE", "TK_ENOMEM", "TK_EHIP"][code])
    assert L.tk_last_hip_error() == 0
    assert L.tk_debug_set_miss_capacity(0, 1 << 40) == tk.TK_EINVAL
    assert L.tk_debug_set_miss_capacity(17, 0) == tk.TK_EINVAL
    assert L.tk_debug_set_miss_capacity(0, 0) == tk.TK_OK


def test_ziggurat_table_is_the_oracles():
    """Two independent builds (mpmath secant in the package, binary128 bisection in the
    oracle) of the 1024-layer table agree in every double."""
    x, f = tk.tk_ziggurat_table()
    xo, fo, r, v = oracle.zig_table(1024)
    assert np.array_equal(x.view(np.uint64), xo.view(np.uint64))
    assert np.array_equal(f.view(np.uint64), fo.view(np.uint64))
    assert x[1] == r


@pytest.mark.parametrize("weights", [
    [1.0], [1.0, 2.0, 3.0], [0.0, 5.0, 0.0, 1.0], [1.0] * 7, [3.0, 3.0, 1.0],
    list(tk_inputs.zipf_weights()), list(np.random.default_rng(4).random(5000)),
])
def test_alias_host_build_is_the_oracles(weights):
    q, a = tk.tk_alias_build_host(weights)
    qo, ao, _ = oracle.alias_build(weights)
    assert np.array_equal(q, qo) and np.array_equal(a, ao)


def test_binding_refuses_host_tensors_and_bad_buffers():
    """The binding passes device buffers only; host tensors are refused before any call."""
    import torch
    with pytest.raises(ValueError, match="HIP device"):
        tk.tk_fill_u32(1, 0, 4, torch.empty(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="HIP device"):
        tk.tk_dropout_f32(1, 0, 4, 0.1, torch.empty(4), torch.empty(4))


def test_tunable_hook_validation():
    """tk_debug_set_tunable accepts exactly the documented names and values; a negative
    value restores the environment's setting (no device involved)."""
    ok = {"store_nt": (0, 1), "max_blocks": (1, 7, (1 << 31) - 1), "unroll": (1, 2, 4),
          "choice_tiles": (1, 2, 4, 8), "exp_tiles": (1, 2, 4), "zig_tiles": (1, 2, 4, 8, 16),
          "zig_lds": (0, 1), "zig_fused": (0, 1), "philox_lds": (0, 1), "pair_lds": (0, 1), "lds_pad": (0, 4096, 65536), "zig_lds_pad": (0, 65536),
          "const_work": (0, 1, 4096)}
    bad = {"store_nt": (2,), "max_blocks": (0, 1 << 31), "unroll": (3, 8), "choice_tiles": (3, 16),
           "exp_tiles": (8,), "zig_tiles": (3, 32), "zig_lds": (2,), "zig_fused": (7,), "philox_lds": (2,), "pair_lds": (2,), "lds_pad": (65537,), "zig_lds_pad": (65537,),
           "const_work": (4097,)}
    assert set(ok) == set(tk.TUNABLES)
    try:
        for name, values in ok.items():
            for v in values:
                assert L.tk_debug_set_tunable(name.encode(), v) == tk.TK_OK, (name, v)
            for v in bad[name]:
                assert L.tk_debug_set_tunable(name.encode(), v) == tk.TK_EINVAL, (name, v)
            assert L.tk_debug_set_tunable(name.encode(), -1) == tk.TK_OK
        assert L.tk_debug_set_tunable(b"no_such_tunable", 1) == tk.TK_EINVAL
        assert L.tk_debug_set_tunable(b"no_such_tunable", -1) == tk.TK_EINVAL
        assert L.tk_debug_set_tunable(None, 1) == tk.TK_EINVAL
        with pytest.raises(tk.TkError):
            tk.tk_debug_set_tunable("unroll", 3)
    finally:
        for name in tk.TUNABLES:
            tk.tk_debug_set_tunable(name, -1)
