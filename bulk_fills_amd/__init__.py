"""Python binding of libtk (include/tk.h): counter-based random bulk fills on MI355X.

Argument marshalling only: every function has the name of its C entry point, takes the
same arguments in the same order, passes device pointers and the HIP stream through, and
raises TkError on a non-zero status.  All computation happens in the HIP kernels of
libtk.so; there is no CPU fallback, and importing this package without the built library
fails.

A buffer argument may be a torch tensor on a HIP device (its data_ptr is passed after a
check that it holds n elements of the right size) or a raw device address (int).
`stream` defaults to torch's current stream of the tensor's device; pass an int handle or
a torch.cuda.Stream to choose another.
"""
import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtk.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "(bulk_fills_amd has no CPU fallback)")

# torch ships its own HIP runtime (libamdhip64.so.7).  Loading it first lets libtk bind to
# that same runtime; loading libtk first would bring a second HIP/HSA runtime into the
# process, and one of the two would then find no device.
try:
    import torch  # noqa: F401
except ImportError:  # the C library still loads on its own
    torch = None

lib = C.CDLL(LIB_PATH)

TK_OK, TK_EINVAL, TK_ERANGE, TK_ENOMEM, TK_EHIP = 0, 1, 2, 3, 4

_u32, _u64, _i32, _i64, _f32 = C.c_uint32, C.c_uint64, C.c_int32, C.c_int64, C.c_float
_p = C.c_void_p

# C signatures (argument types in declaration order; every fill returns tk_status).
SIGNATURES = {
    "tk_fill_u8": [_u32, _u64, _u64, _p, _p],
    "tk_fill_u16": [_u32, _u64, _u64, _p, _p],
    "tk_fill_u32": [_u32, _u64, _u64, _p, _p],
    "tk_fill_u64": [_u32, _u64, _u64, _p, _p],
    "tk_fill_f16_bits": [_u32, _u64, _u64, _p, _p],
    "tk_fill_f32": [_u32, _u64, _u64, _p, _p],
    "tk_fill_f64": [_u32, _u64, _u64, _p, _p],
    "tk_fill_bool": [_u32, _u64, _u64, _p, _p],
    "tk_fill_u32_below": [_u32, _u64, _u64, _u32, _p, _p],
    "tk_fill_u64_below": [_u32, _u64, _u64, _u64, _p, _p],
    "tk_fill_i32_below": [_u32, _u64, _u64, _i32, _u32, _p, _p],
    "tk_fill_i64_below32": [_u32, _u64, _u64, _i64, _u32, _p, _p],
    "tk_fill_i64_below": [_u32, _u64, _u64, _i64, _u64, _p, _p],
    "tk_fill_normal_f64": [_u32, _u64, _u64, _p, _p],
    "tk_fill_normal_f32": [_u32, _u64, _u64, _p, _p],
    "tk_fill_normal_f32_half_turn": [_u32, _u64, _u64, _p, _p],
    "tk_fill_randn_f32": [_u32, _u64, _u64, _p, _p],
    "tk_fill_exponential_f64": [_u32, _u64, _u64, _p, _p],
    "tk_fill_exponential_f32": [_u32, _u64, _u64, _p, _p],
    "tk_dropout_f32": [_u32, _u64, _u64, _f32, _p, _p, _p, _p],
    "tk_dropout_backward_f32": [_u32, _u64, _u64, _f32, _p, _p, _p],
    "tk_alias_create": [_p, _u32, _p],
    "tk_alias_destroy": [_p],
    "tk_alias_export": [_p, _p, _p],
    "tk_alias_build_host": [_p, _u32, _p, _p],
    "tk_fill_choice_u32": [_u32, _u64, _u64, _p, _p, _p],
    "tk_philox_fill_u32": [_u64, _u64, _u64, _p, _p],
    "tk_philox_fill_u64": [_u64, _u64, _u64, _p, _p],
    "tk_philox_fill_f32": [_u64, _u64, _u64, _p, _p],
    "tk_philox_fill_f64": [_u64, _u64, _u64, _p, _p],
    "tk_philox_fill_u32_below": [_u64, _u64, _u64, _u32, _p, _p],
    "tk_philox_fill_u64_below": [_u64, _u64, _u64, _u64, _p, _p],
    "tk_philox_fill_choice_u32": [_u64, _u64, _u64, _p, _p, _p],
    "tk_philox_fill_normal_f32": [_u64, _u64, _u64, _p, _p],
    "tk_philox_fill_normal_f64": [_u64, _u64, _u64, _p, _p],
    "tk_ziggurat_table": [_p, _p],
    "tk_debug_set_miss_capacity": [_u32, _u64],
    "tk_debug_last_miss_count": [_p],
    "tk_debug_set_normal_f64_mode": [_u32],
    "tk_debug_set_tunable": [C.c_char_p, _i64],
    "tk_debug_fail_allocations": [_u32, _u32],
    "tk_debug_device_bytes": [_p],
    "tk_fill_constant_u32": [_u32, _u64, _p, _p],
    "tk_fill_normal_f64_no_alloc": [_u32, _u64, _u64, _p, _p],
}
for _name, _args in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = C.c_int
lib.tk_status_string.argtypes = [C.c_int]
lib.tk_status_string.restype = C.c_char_p
lib.tk_last_hip_error.argtypes = []
lib.tk_last_hip_error.restype = C.c_int
lib.tk_alias_size.argtypes = [_p]
lib.tk_alias_size.restype = C.c_uint32


class TkError(RuntimeError):
    def __init__(self, code, where):
        msg = lib.tk_status_string(code).decode()
        if code == TK_EHIP:
            msg += f" (hipError {lib.tk_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.code = code


def _check(code, where):
    if code != TK_OK:
        raise TkError(code, where)


def _buf(x, itemsize, n, where):
    """Device address of a buffer argument (tensor or int), checking size for tensors."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError(f"{where}: buffer must live on a HIP device")
    import torch
    if x.device.index != torch.cuda.current_device():
        # the library launches on the calling thread's current device
        raise ValueError(f"{where}: buffer is on {x.device}, the current device is cuda:{torch.cuda.current_device()}")
    if x.element_size() != itemsize:
        raise ValueError(f"{where}: element size {x.element_size()} != {itemsize}")
    if not x.is_contiguous() or x.numel() < n:
        raise ValueError(f"{where}: need a contiguous buffer of at least {n} elements")
    return x.data_ptr()


def _stream(stream, *bufs):
    if isinstance(stream, int):
        return stream
    if stream is not None:
        return stream.cuda_stream
    import torch
    dev = next((b.device for b in bufs if b is not None and not isinstance(b, int)), None)
    return torch.cuda.current_stream(dev).cuda_stream


def _fill(cname, itemsize):
    fn = getattr(lib, cname)

    def call(key, start_draw, n, out, stream=None):
        _check(fn(key, start_draw, n, _buf(out, itemsize, n, cname), _stream(stream, out)), cname)

    call.__name__ = cname
    call.__doc__ = f"{cname}(key, start_draw, n, out, stream=None): see include/tk.h."
    return call


tk_fill_u8 = _fill("tk_fill_u8", 1)
tk_fill_u16 = _fill("tk_fill_u16", 2)
tk_fill_u32 = _fill("tk_fill_u32", 4)
tk_fill_u64 = _fill("tk_fill_u64", 8)
tk_fill_f16_bits = _fill("tk_fill_f16_bits", 2)
tk_fill_f32 = _fill("tk_fill_f32", 4)
tk_fill_f64 = _fill("tk_fill_f64", 8)
tk_fill_bool = _fill("tk_fill_bool", 1)
tk_fill_normal_f64 = _fill("tk_fill_normal_f64", 8)
tk_fill_normal_f32 = _fill("tk_fill_normal_f32", 4)
tk_fill_normal_f64_no_alloc = _fill("tk_fill_normal_f64_no_alloc", 8)
tk_fill_normal_f32_half_turn = _fill("tk_fill_normal_f32_half_turn", 4)
tk_fill_randn_f32 = _fill("tk_fill_randn_f32", 4)
tk_fill_exponential_f64 = _fill("tk_fill_exponential_f64", 8)
tk_fill_exponential_f32 = _fill("tk_fill_exponential_f32", 4)
tk_philox_fill_u32 = _fill("tk_philox_fill_u32", 4)
tk_philox_fill_u64 = _fill("tk_philox_fill_u64", 8)
tk_philox_fill_f32 = _fill("tk_philox_fill_f32", 4)
tk_philox_fill_f64 = _fill("tk_philox_fill_f64", 8)
tk_philox_fill_normal_f32 = _fill("tk_philox_fill_normal_f32", 4)
tk_philox_fill_normal_f64 = _fill("tk_philox_fill_normal_f64", 8)


def tk_fill_constant_u32(value, n, out, stream=None):
    _check(lib.tk_fill_constant_u32(value, n, _buf(out, 4, n, "tk_fill_constant_u32"), _stream(stream, out)),
           "tk_fill_constant_u32")


def tk_philox_fill_u32_below(key, start_draw, n, bound, out, stream=None):
    _check(lib.tk_philox_fill_u32_below(key, start_draw, n, bound, _buf(out, 4, n, "tk_philox_fill_u32_below"),
                                        _stream(stream, out)), "tk_philox_fill_u32_below")


def tk_philox_fill_u64_below(key, start_draw, n, bound, out, stream=None):
    _check(lib.tk_philox_fill_u64_below(key, start_draw, n, bound, _buf(out, 8, n, "tk_philox_fill_u64_below"),
                                        _stream(stream, out)), "tk_philox_fill_u64_below")


def tk_fill_u32_below(key, start_draw, n, bound, out, stream=None):
    _check(lib.tk_fill_u32_below(key, start_draw, n, bound, _buf(out, 4, n, "tk_fill_u32_below"),
                                 _stream(stream, out)), "tk_fill_u32_below")


def tk_fill_u64_below(key, start_draw, n, bound, out, stream=None):
    _check(lib.tk_fill_u64_below(key, start_draw, n, bound, _buf(out, 8, n, "tk_fill_u64_below"),
                                 _stream(stream, out)), "tk_fill_u64_below")


def tk_fill_i32_below(key, start_draw, n, low, bound, out, stream=None):
    _check(lib.tk_fill_i32_below(key, start_draw, n, low, bound, _buf(out, 4, n, "tk_fill_i32_below"),
                                 _stream(stream, out)), "tk_fill_i32_below")


def tk_fill_i64_below32(key, start_draw, n, low, bound, out, stream=None):
    _check(lib.tk_fill_i64_below32(key, start_draw, n, low, bound, _buf(out, 8, n, "tk_fill_i64_below32"),
                                   _stream(stream, out)), "tk_fill_i64_below32")


def tk_fill_i64_below(key, start_draw, n, low, bound, out, stream=None):
    _check(lib.tk_fill_i64_below(key, start_draw, n, low, bound, _buf(out, 8, n, "tk_fill_i64_below"),
                                 _stream(stream, out)), "tk_fill_i64_below")


def tk_dropout_f32(key, start_draw, n, p, x, y, mask=None, stream=None):
    _check(lib.tk_dropout_f32(key, start_draw, n, p, _buf(x, 4, n, "tk_dropout_f32"),
                              _buf(y, 4, n, "tk_dropout_f32"), _buf(mask, 1, n, "tk_dropout_f32"),
                              _stream(stream, y)), "tk_dropout_f32")


def tk_dropout_backward_f32(key, start_draw, n, p, dy, dx, stream=None):
    _check(lib.tk_dropout_backward_f32(key, start_draw, n, p, _buf(dy, 4, n, "tk_dropout_backward_f32"),
                                       _buf(dx, 4, n, "tk_dropout_backward_f32"), _stream(stream, dx)),
           "tk_dropout_backward_f32")


class Alias:
    """Owner of a tk_alias handle (tk_alias_create / tk_alias_destroy)."""

    def __init__(self, weights):
        import numpy as np
        w = np.ascontiguousarray(weights, dtype=np.float64)
        h = C.c_void_p()
        _check(lib.tk_alias_create(w.ctypes.data, w.size, C.byref(h)), "tk_alias_create")
        self.handle = h.value
        self.n = w.size

    def export(self):
        import numpy as np
        q = np.empty(self.n, dtype=np.uint32)
        a = np.empty(self.n, dtype=np.uint32)
        _check(lib.tk_alias_export(self.handle, q.ctypes.data, a.ctypes.data), "tk_alias_export")
        return q, a

    def close(self):
        if self.handle:
            _check(lib.tk_alias_destroy(self.handle), "tk_alias_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tk_alias_create(weights):
    return Alias(weights)


def tk_alias_build_host(weights):
    """The library's host alias construction alone: returns (q, alias) numpy arrays."""
    import numpy as np
    w = np.ascontiguousarray(weights, dtype=np.float64)
    q = np.empty(w.size, dtype=np.uint32)
    a = np.empty(w.size, dtype=np.uint32)
    _check(lib.tk_alias_build_host(w.ctypes.data, w.size, q.ctypes.data, a.ctypes.data), "tk_alias_build_host")
    return q, a


def tk_fill_choice_u32(key, start_draw, n, table, out, stream=None):
    _check(lib.tk_fill_choice_u32(key, start_draw, n, table.handle, _buf(out, 4, n, "tk_fill_choice_u32"),
                                  _stream(stream, out)), "tk_fill_choice_u32")


def tk_philox_fill_choice_u32(key, start_draw, n, table, out, stream=None):
    _check(lib.tk_philox_fill_choice_u32(key, start_draw, n, table.handle, _buf(out, 4, n, "tk_philox_fill_choice_u32"),
                                         _stream(stream, out)), "tk_philox_fill_choice_u32")


def tk_ziggurat_table():
    import numpy as np
    x = np.empty(1025, dtype=np.float64)
    f = np.empty(1025, dtype=np.float64)
    _check(lib.tk_ziggurat_table(x.ctypes.data, f.ctypes.data), "tk_ziggurat_table")
    return x, f


def tk_debug_set_miss_capacity(per_group, overflow):
    _check(lib.tk_debug_set_miss_capacity(per_group, overflow), "tk_debug_set_miss_capacity")


def tk_debug_set_normal_f64_mode(mode):
    _check(lib.tk_debug_set_normal_f64_mode(mode), "tk_debug_set_normal_f64_mode")


TUNABLES = ("store_nt", "max_blocks", "unroll", "choice_tiles", "exp_tiles", "zig_tiles", "zig_lds", "zig_fused",
            "philox_lds", "pair_lds", "lds_pad", "zig_lds_pad", "const_work")


def tk_debug_set_tunable(name, value):
    """Sets a launch tunable (see include/tk.h); a negative value restores the environment's."""
    _check(lib.tk_debug_set_tunable(name.encode(), int(value)), "tk_debug_set_tunable")


def tk_debug_fail_allocations(skip, count):
    _check(lib.tk_debug_fail_allocations(skip, count), "tk_debug_fail_allocations")


def tk_debug_device_bytes():
    v = C.c_uint64()
    _check(lib.tk_debug_device_bytes(C.byref(v)), "tk_debug_device_bytes")
    return v.value


def tk_debug_last_miss_count():
    v = C.c_uint64()
    _check(lib.tk_debug_last_miss_count(C.byref(v)), "tk_debug_last_miss_count")
    return v.value
