"""Host checks of the exponential fills' logarithm tables (log256.inc, logf256.inc), against
mpmath, and of the logarithms' arithmetic (host models of the kernels' operations).

The tables are product data (the kernels read them; the oracle uses the C library's log).
These tests check the properties the device logarithms' error bounds rest on: multipliers
with few enough significant bits that the reduction q = z m - 1 is exact (9 for f64, whose
z has 53; 24 for f32, whose z has 24), |q| inside its bound at both ends of every entry,
ln v to the stated precision (f64: hi on the 2^-45 grid plus a 21-bit low part; f32: rounded
to nearest), the ln 2 split, and that both files are what their generator writes.  Host
models of the two logarithms then show the f32 one correctly rounded at all 2^24 inputs
and the f64 one within 0.51 ulp with exact reductions."""
import os
import re
import struct
import subprocess
import sys
from fractions import Fraction

import mpmath as mp
import numpy as np
import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "bulk_fills_amd", "csrc")
INC = os.path.join(CSRC, "log256.inc")
INC_F = os.path.join(CSRC, "logf256.inc")
HERE = os.path.dirname(os.path.abspath(__file__))


def high_word_double(w):
    return struct.unpack("<d", struct.pack("<Q", int(w, 16) << 32))[0]


def parse():
    text = open(INC).read()
    defs = dict(re.findall(r"#define (TK_\w+) (\S+)\n", text))
    rows = [(float.fromhex(h), high_word_double(m), high_word_double(lo))
            for h, m, lo in re.findall(r"\{(\S+), 0x([0-9A-F]+)u, 0x([0-9A-F]+)u\}", text)]
    return defs, rows


def generator():
    import importlib.util
    spec = importlib.util.spec_from_file_location("gen_log_table", os.path.join(CSRC, "gen_log_table.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    return gen


def test_shape_and_constants():
    defs, rows = parse()
    entries, split = int(defs["TK_LOGD_ENTRIES"]), int(defs["TK_LOGD_SPLIT"])
    assert len(rows) == entries == 256 and split == 96
    # the kernel's halving test: fraction bits of the high word >= split << 12, which the
    # borrow of (((1044 << 20) | 0x5FFFF) - xh) >> 20 takes (tk_log.h)
    assert (split << 12) - 1 == 0x5FFFF
    mp.mp.dps = 60
    hi, lo = float.fromhex(defs["TK_LN2_HI"]), float.fromhex(defs["TK_LN2_LO"])
    assert (Fraction(hi) * 2 ** 45).denominator == 1
    assert abs(mp.mpf(hi) + mp.mpf(lo) - mp.log(2)) < mp.mpf(2) ** -100
    # the halved entries cover [0.6875, 1): entry 96 starts at 1.375 before the halving
    assert 1 + Fraction(split, entries) == Fraction(11, 8)


def sig_bits(x):
    f = abs(Fraction(x))
    while f.denominator != 1:
        f *= 2
    n = f.numerator
    while n and n % 2 == 0:
        n //= 2
    return n.bit_length()


def test_entries():
    """Per entry: m has at most 9 significant bits, so z m (z with 53) has at most 62 and
    z m - 1 with |q| < 2^-8 fits in 53: exact.  |q| is checked at the entry's first z and
    its last (z on the 2^-52 grid of [1, 2)); ln v to 2^-66 by l_hi + l_lo."""
    defs, rows = parse()
    entries, split = int(defs["TK_LOGD_ENTRIES"]), int(defs["TK_LOGD_SPLIT"])
    mp.mp.dps = 60
    for j, (l_hi, m, l_lo) in enumerate(rows):
        assert sig_bits(m) <= 9, j
        a = 1 + Fraction(j, entries)
        last = a + Fraction(1, entries) - Fraction(1, 1 << 52)
        q = max(abs(a * Fraction(m) - 1), abs(last * Fraction(m) - 1))
        assert q < Fraction(1, 256), (j, float(q))
        v = Fraction(m) * (2 if j >= split else 1)
        if j in (0, entries - 1):
            assert v == 1 and l_hi == 0.0 and l_lo == 0.0
        assert (Fraction(l_hi) * 2 ** 45).denominator == 1
        assert sig_bits(l_lo) <= 21
        exact = mp.log(mp.mpf(v.numerator) / v.denominator)
        assert abs(mp.mpf(l_hi) + mp.mpf(l_lo) - exact) <= mp.mpf(2) ** -66, j
        assert abs(l_lo) <= 2.0 ** -46


def test_fma_high_part_is_exact():
    """n LN2_HI + l_hi (0 <= n <= 53) needs at most 53 significant bits, so the kernel's
    single fused multiply-add computes it exactly."""
    defs, rows = parse()
    hi = Fraction(float.fromhex(defs["TK_LN2_HI"]))
    for n in range(54):
        for l_hi, _, _ in rows:
            s = n * hi + Fraction(l_hi)
            assert Fraction(float(s)) == s, (n, l_hi)


def test_file_matches_generator():
    gen = generator()
    rows, ln2_hi, ln2_lo = gen.build()
    defs, parsed = parse()
    assert parsed == rows
    assert float.fromhex(defs["TK_LN2_HI"]) == ln2_hi and float.fromhex(defs["TK_LN2_LO"]) == ln2_lo
    assert parse_f()[1] == gen.build_f32()


def test_f64_logarithm_model(tmp_path):
    """The host model of the f64 logarithm: within 0.51 ulp of -ln(1 - u) over the 2^-24 grid
    and 2^25 points of the 2^-53 grid, every reduction exact, +0 at u = 0."""
    exe = str(tmp_path / "exp_f64_model")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-I", CSRC, "-o", exe,
                    os.path.join(HERE, "exp_f64_model.c"), "-lm"], check=True)
    worst, inexact, wrong_zero = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    assert int(inexact) == 0
    assert int(wrong_zero) == 0
    assert float(worst) < 0.51, worst


def parse_f():
    text = open(INC_F).read()
    defs = dict(re.findall(r"#define (TK_\w+) (\S+)\n", text))
    rows = [tuple(float.fromhex(v) for v in m) for m in re.findall(r"\{(\S+), (\S+)\}", text)]
    return defs, rows


def test_f64_model_library_form():
    """The library form of the model (tests/libexp_f64_model.so, which the GPU test compares
    with the fill bit for bit) is the same model: +0 at u = 0, the correctly rounded ln 2
    at u = 1/2, and within one ulp of numpy's log1p on random 53-bit draws."""
    import ctypes as C
    sys.path.insert(0, HERE)
    import build_exp_model
    path = build_exp_model.LIB if os.path.exists(build_exp_model.LIB) else build_exp_model.build()
    lib = C.CDLL(path)
    lib.tk_model_neg_ln_batch.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t]
    rng = np.random.default_rng(5)
    d = rng.integers(0, 1 << 63, 100000, dtype=np.uint64)  # high words carry bits the fill ignores
    d[:3] = [0, 1 << 52, (1 << 53) - 1]
    out = np.empty(d.size, dtype=np.float64)
    lib.tk_model_neg_ln_batch(d.ctypes.data, out.ctypes.data, d.size)
    assert out[0] == 0.0 and not np.signbit(out[0])
    assert out[1] == float.fromhex("0x1.62e42fefa39efp-1")
    u = (d & np.uint64((1 << 53) - 1)).astype(np.float64) * 2.0 ** -53
    want = -np.log1p(-u)
    ulp = np.spacing(np.maximum(want, 1e-300))
    assert np.max(np.abs(out - want) / ulp) <= 1.0


def test_f32_table_entries():
    defs, rows = parse_f()
    entries, split = int(defs["TK_LOGF_ENTRIES"]), int(defs["TK_LOGF_SPLIT"])
    assert len(rows) == entries == 256 and split == 96
    # the kernel's halving test: fraction bits of k's high word >= split << 12, which the
    # borrow of (0x4175FFFF - xh) >> 20 takes (tk_log.h)
    assert (split << 12) - 1 == 0x5FFFF
    mp.mp.dps = 60
    for j, (mult, lv) in enumerate(rows):
        v = Fraction(mult) * (2 if j >= split else 1)   # the multiplier of the reduced z
        assert sig_bits(mult) <= 24, j                  # z (<= 24 bits) times it is exact
        lo = 1 + Fraction(j, entries)
        a, b = lo, lo + Fraction(1, entries)            # z in [1, 2) for this entry
        if j >= split:
            a, b = a / 2, b / 2
        q = max(abs(a * v - 1), abs(b * v - 1))
        assert q <= Fraction(1, 256 if j == 0 else 512) * (1 + Fraction(1, 1 << 20)), (j, float(q))
        if j in (0, entries - 1):
            assert v == 1 and lv == 0.0
        exact = mp.log(mp.mpf(v.numerator) / v.denominator)
        assert lv == float(mp.mpf(lv)) and abs(mp.mpf(lv) - exact) <= mp.mpf(abs(lv)) * mp.mpf(2) ** -53, j
        assert float(exact) == lv, j                    # ln v rounded to nearest


def test_f32_ln2_constant():
    text = open(os.path.join(CSRC, "tk_log.h")).read()
    c = float.fromhex(re.search(r"constexpr double kLn2 = (\S+);", text).group(1))
    mp.mp.dps = 40
    assert c == float(mp.log(2))


def test_f32_logarithm_every_input(tmp_path):
    """All 2^24 inputs of the f32 exponential: the host model of the kernel's operations
    rounds to the correctly rounded f32 everywhere (and gives +0 at m = 0)."""
    exe = str(tmp_path / "exp_f32_model")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-I", CSRC, "-o", exe,
                    os.path.join(HERE, "exp_f32_model.c"), "-lm"], check=True)
    wrong, undecided, worst = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    assert int(undecided) == 0
    assert int(wrong) == 0
    assert float(worst) < 0.5, worst
