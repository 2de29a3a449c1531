"""ctypes wrapper around the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and the
benchmark's CPU-baseline leg.  The product path never imports it.

Each fill returns a numpy array of n elements for draws start .. start+n-1, or, when
`draws` is given, for those draw indices (a gather used for sampled comparisons).
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ORC_OK, ORC_EINVAL, ORC_ERANGE = 0, 1, 2
P_NORMAL64 = 0x4E4F524D
P_BELOW32 = 0x424C3332
P_BELOW64 = 0x424C3634


class OracleError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: oracle status {code}")
        self.code = code


def _load():
    if not os.path.exists(_LIB_PATH):
        _build.build()
    return C.CDLL(_LIB_PATH)


_lib = _load()

_u8p, _u16p, _u32p, _u64p = (C.POINTER(t) for t in (C.c_uint8, C.c_uint16, C.c_uint32, C.c_uint64))
_fp, _dp, _i32p, _i64p = C.POINTER(C.c_float), C.POINTER(C.c_double), C.POINTER(C.c_int32), C.POINTER(C.c_int64)

_lib.orc_hash32.restype = C.c_uint32
_lib.orc_hash32.argtypes = [C.c_uint32]
_lib.orc_word.restype = C.c_uint32
_lib.orc_word.argtypes = [C.c_uint32, C.c_uint32]
_lib.orc_uniform.restype = C.c_float
_lib.orc_uniform.argtypes = [C.c_uint32, C.c_uint32]
_lib.orc_randn.restype = C.c_float
_lib.orc_randn.argtypes = [C.c_uint32, C.c_uint32]
_lib.orc_sub.restype = C.c_uint32
_lib.orc_sub.argtypes = [C.c_uint32, C.c_uint32]
_lib.orc_split.restype = C.c_uint32
_lib.orc_split.argtypes = [C.c_uint32, C.c_uint32]
_lib.orc_lemire32.restype = C.c_uint32
_lib.orc_lemire32.argtypes = [C.c_uint32, C.c_uint32, C.c_uint32]
_lib.orc_lemire64.restype = C.c_uint64
_lib.orc_lemire64.argtypes = [C.c_uint32, C.c_uint32, C.c_uint64]

hash32 = _lib.orc_hash32
word = _lib.orc_word
uniform = _lib.orc_uniform
randn = _lib.orc_randn
sub = _lib.orc_sub
split = _lib.orc_split
lemire32 = _lib.orc_lemire32
lemire64 = _lib.orc_lemire64


def _ptr(a, ctype):
    return a.ctypes.data_as(ctype) if a is not None else None


def _draws(draws):
    if draws is None:
        return None, None
    d = np.ascontiguousarray(draws, dtype=np.uint64)
    return d, _ptr(d, _u64p)


def _check(rc, what):
    if rc != ORC_OK:
        raise OracleError(rc, what)


def _simple(fname, np_dtype, ctype, key_ctype=C.c_uint32):
    f = getattr(_lib, fname)
    f.restype = C.c_int
    f.argtypes = [key_ctype, C.c_uint64, C.c_uint64, _u64p, ctype]

    def fill(key, start=0, n=None, draws=None):
        d, dp = _draws(draws)
        if d is not None:
            n = d.size
        out = np.empty(int(n), dtype=np_dtype)
        _check(f(key, start, int(n), dp, _ptr(out, ctype)), fname)
        return out

    fill.__name__ = fname[len("orc_"):]
    return fill


fill_u8 = _simple("orc_fill_u8", np.uint8, _u8p)
fill_u16 = _simple("orc_fill_u16", np.uint16, _u16p)
fill_u32 = _simple("orc_fill_u32", np.uint32, _u32p)
fill_u64 = _simple("orc_fill_u64", np.uint64, _u64p)
fill_f16_bits = _simple("orc_fill_f16_bits", np.uint16, _u16p)
fill_f32 = _simple("orc_fill_f32", np.float32, _fp)
fill_f64 = _simple("orc_fill_f64", np.float64, _dp)
fill_bool = _simple("orc_fill_bool", np.uint8, _u8p)
fill_normal_f32 = _simple("orc_fill_normal_f32", np.float32, _fp)
fill_exponential_f64 = _simple("orc_fill_exponential_f64", np.float64, _dp)
fill_exponential_f32 = _simple("orc_fill_exponential_f32", np.float32, _fp)
philox_fill_u32 = _simple("orc_philox_fill_u32", np.uint32, _u32p, C.c_uint64)
philox_fill_u64 = _simple("orc_philox_fill_u64", np.uint64, _u64p, C.c_uint64)
philox_fill_f32 = _simple("orc_philox_fill_f32", np.float32, _fp, C.c_uint64)
philox_fill_f64 = _simple("orc_philox_fill_f64", np.float64, _dp, C.c_uint64)
philox_fill_normal_f32 = _simple("orc_philox_fill_normal_f32", np.float32, _fp, C.c_uint64)
fill_normal_f32_half_turn = _simple("orc_fill_normal_f32_half_turn", np.float32, _fp)
fill_randn_f32 = _simple("orc_fill_randn_f32", np.float32, _fp)

_lib.orc_fill_u32_below.argtypes = [C.c_uint32, C.c_uint64, C.c_uint64, _u64p, C.c_uint32, _u32p]
_lib.orc_fill_u64_below.argtypes = [C.c_uint32, C.c_uint64, C.c_uint64, _u64p, C.c_uint64, _u64p]
_lib.orc_fill_i32_below.argtypes = [C.c_uint32, C.c_uint64, C.c_uint64, _u64p, C.c_int32, C.c_uint32, _i32p]
_lib.orc_fill_i64_below32.argtypes = [C.c_uint32, C.c_uint64, C.c_uint64, _u64p, C.c_int64, C.c_uint32, _i64p]
_lib.orc_fill_i64_below.argtypes = [C.c_uint32, C.c_uint64, C.c_uint64, _u64p, C.c_int64, C.c_uint64, _i64p]
_lib.orc_fill_normal_f64.argtypes = [C.c_uint32, C.c_uint64, C.c_uint64, _u64p, _dp, _u8p]
_lib.orc_dropout_f32.argtypes = [C.c_uint32, C.c_uint64, C.c_uint64, _u64p, C.c_float, _fp, _fp, _u8p]
_lib.orc_alias_build.argtypes = [_dp, C.c_uint32, _u32p, _u32p, _u64p]
_lib.orc_fill_choice_u32.argtypes = [C.c_uint32, C.c_uint64, C.c_uint64, _u64p, _u32p, _u32p, C.c_uint32, _u32p]
_lib.orc_zig_table.argtypes = [C.c_uint32, _dp, _dp, _dp, _dp]
_lib.orc_philox_sub_word.restype = C.c_uint32
_lib.orc_philox_sub_word.argtypes = [C.c_uint64, C.c_uint64, C.c_uint32, C.c_uint32]
philox_sub_word = _lib.orc_philox_sub_word
_lib.orc_philox_fill_u32_below.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, _u64p, C.c_uint32, _u32p]
_lib.orc_philox_fill_u64_below.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, _u64p, C.c_uint64, _u64p]
_lib.orc_philox_fill_choice_u32.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, _u64p, _u32p, _u32p, C.c_uint32, _u32p]
_lib.orc_philox_fill_normal_f64.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, _u64p, _dp, _u8p]


def _n(n, d):
    return int(d.size if d is not None else n)


def fill_u32_below(key, start=0, n=None, bound=1, draws=None):
    d, dp = _draws(draws)
    out = np.empty(_n(n, d), dtype=np.uint32)
    _check(_lib.orc_fill_u32_below(key, start, out.size, dp, bound, _ptr(out, _u32p)), "u32_below")
    return out


def fill_u64_below(key, start=0, n=None, bound=1, draws=None):
    d, dp = _draws(draws)
    out = np.empty(_n(n, d), dtype=np.uint64)
    _check(_lib.orc_fill_u64_below(key, start, out.size, dp, bound, _ptr(out, _u64p)), "u64_below")
    return out


def fill_i32_below(key, start=0, n=None, low=0, bound=1, draws=None):
    d, dp = _draws(draws)
    out = np.empty(_n(n, d), dtype=np.int32)
    _check(_lib.orc_fill_i32_below(key, start, out.size, dp, low, bound, _ptr(out, _i32p)), "i32_below")
    return out


def fill_i64_below32(key, start=0, n=None, low=0, bound=1, draws=None):
    d, dp = _draws(draws)
    out = np.empty(_n(n, d), dtype=np.int64)
    _check(_lib.orc_fill_i64_below32(key, start, out.size, dp, low, bound, _ptr(out, _i64p)), "i64_below32")
    return out


def fill_i64_below(key, start=0, n=None, low=0, bound=1, draws=None):
    d, dp = _draws(draws)
    out = np.empty(_n(n, d), dtype=np.int64)
    _check(_lib.orc_fill_i64_below(key, start, out.size, dp, low, bound, _ptr(out, _i64p)), "i64_below")
    return out


def fill_normal_f64(key, start=0, n=None, draws=None, with_path=False):
    """Returns the values, and with with_path=True also the path code per element
    (0 fast path, 1 wedge, 2 tail, 3 restart ending in the fast path)."""
    d, dp = _draws(draws)
    out = np.empty(_n(n, d), dtype=np.float64)
    path = np.empty(out.size, dtype=np.uint8) if with_path else None
    _check(_lib.orc_fill_normal_f64(key, start, out.size, dp, _ptr(out, _dp), _ptr(path, _u8p)), "normal_f64")
    return (out, path) if with_path else out


def dropout_f32(key, start, x, p, draws=None, with_mask=True):
    x = np.ascontiguousarray(x, dtype=np.float32)
    d, dp = _draws(draws)
    if d is not None and d.size != x.size:
        raise ValueError("draws and x differ in length")
    y = np.empty_like(x)
    mask = np.empty(x.size, dtype=np.uint8) if with_mask else None
    _check(_lib.orc_dropout_f32(key, start, x.size, dp, C.c_float(p), _ptr(x, _fp), _ptr(y, _fp),
                                _ptr(mask, _u8p)), "dropout_f32")
    return (y, mask) if with_mask else y


def alias_build(weights):
    """Integer Vose alias table: returns (q, alias, mass) as uint32, uint32, uint64 arrays."""
    w = np.ascontiguousarray(weights, dtype=np.float64)
    n = w.size
    q = np.empty(n, dtype=np.uint32)
    al = np.empty(n, dtype=np.uint32)
    mass = np.empty(n, dtype=np.uint64)
    _check(_lib.orc_alias_build(_ptr(w, _dp), n, _ptr(q, _u32p), _ptr(al, _u32p), _ptr(mass, _u64p)), "alias_build")
    return q, al, mass


def fill_choice_u32(key, start, n, q, alias, draws=None):
    q = np.ascontiguousarray(q, dtype=np.uint32)
    alias = np.ascontiguousarray(alias, dtype=np.uint32)
    d, dp = _draws(draws)
    out = np.empty(_n(n, d), dtype=np.uint32)
    _check(_lib.orc_fill_choice_u32(key, start, out.size, dp, _ptr(q, _u32p), _ptr(alias, _u32p), q.size,
                                    _ptr(out, _u32p)), "choice_u32")
    return out


def philox_fill_u32_below(key, start=0, n=None, bound=1, draws=None):
    d, dp = _draws(draws)
    out = np.empty(_n(n, d), dtype=np.uint32)
    _check(_lib.orc_philox_fill_u32_below(key, start, out.size, dp, bound, _ptr(out, _u32p)), "philox_u32_below")
    return out


def philox_fill_u64_below(key, start=0, n=None, bound=1, draws=None):
    d, dp = _draws(draws)
    out = np.empty(_n(n, d), dtype=np.uint64)
    _check(_lib.orc_philox_fill_u64_below(key, start, out.size, dp, bound, _ptr(out, _u64p)), "philox_u64_below")
    return out


def philox_fill_choice_u32(key, start, n, q, alias, draws=None):
    q = np.ascontiguousarray(q, dtype=np.uint32)
    alias = np.ascontiguousarray(alias, dtype=np.uint32)
    d, dp = _draws(draws)
    out = np.empty(_n(n, d), dtype=np.uint32)
    _check(_lib.orc_philox_fill_choice_u32(key, start, out.size, dp, _ptr(q, _u32p), _ptr(alias, _u32p), q.size,
                                           _ptr(out, _u32p)), "philox_choice_u32")
    return out


def philox_fill_normal_f64(key, start=0, n=None, draws=None, with_path=False):
    """As fill_normal_f64 over the Philox source."""
    d, dp = _draws(draws)
    out = np.empty(_n(n, d), dtype=np.float64)
    path = np.empty(out.size, dtype=np.uint8) if with_path else None
    _check(_lib.orc_philox_fill_normal_f64(key, start, out.size, dp, _ptr(out, _dp), _ptr(path, _u8p)),
           "philox_normal_f64")
    return (out, path) if with_path else out


_lib.orc_lemire32_map.argtypes = [_u32p, C.c_uint64, C.c_uint32, _u32p, _u8p]
_lib.orc_lemire64_map.argtypes = [_u64p, C.c_uint64, C.c_uint64, _u64p, _u8p]


def lemire32_map(x, s, out=None, acc=None):
    """The multiply-shift step over raw words: returns (value, accepted).  `out` (uint32)
    and `acc` (bool) may be given to reuse buffers."""
    x = np.ascontiguousarray(x, dtype=np.uint32)
    out = np.empty_like(x) if out is None else out
    acc = np.empty(x.size, dtype=np.bool_) if acc is None else acc
    assert out.dtype == np.uint32 and acc.dtype == np.bool_ and out.size == acc.size == x.size
    _check(_lib.orc_lemire32_map(_ptr(x, _u32p), x.size, s, _ptr(out, _u32p), _ptr(acc.view(np.uint8), _u8p)),
           "lemire32_map")
    return out, acc


def lemire64_map(x, s):
    x = np.ascontiguousarray(x, dtype=np.uint64)
    out = np.empty_like(x)
    acc = np.empty(x.size, dtype=np.bool_)
    _check(_lib.orc_lemire64_map(_ptr(x, _u64p), x.size, s, _ptr(out, _u64p), _ptr(acc.view(np.uint8), _u8p)),
           "lemire64_map")
    return out, acc


def zig_table(nlayers=1024):
    """Returns (X, F, r, v): X and F hold nlayers+1 doubles each."""
    x = np.empty(nlayers + 1, dtype=np.float64)
    f = np.empty(nlayers + 1, dtype=np.float64)
    r = C.c_double()
    v = C.c_double()
    _check(_lib.orc_zig_table(nlayers, _ptr(x, _dp), _ptr(f, _dp), C.byref(r), C.byref(v)), "zig_table")
    return x, f, r.value, v.value
