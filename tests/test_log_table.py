"""Host checks of the exponential fills' logarithm tables (log128.inc, logf256.inc), against
mpmath, and of the f32 exponential's arithmetic over every one of its inputs.

The tables are product data (the kernels read them; the oracle uses the C library's log).
These tests check the properties the device logarithms' error bounds rest on: for the f64
table every c_j exact with few bits, z - c_j inside the bound on |q|, 1/c_j rounded to
nearest, -ln c_j = hi + lo to far beyond double precision with hi on the 2^-45 grid, the
ln 2 split; for the f32 table multipliers of at most 24 significant bits (so the reduction
is exact), |q| inside its bound and ln v rounded to nearest; and that both files are what
their generator writes.  A host model of the f32 logarithm's operations then shows the
correctly rounded f32 at all 2^24 inputs."""
import os
import re
from fractions import Fraction

import subprocess

import mpmath as mp
import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "bulk_fills_amd", "csrc")
INC = os.path.join(CSRC, "log128.inc")
INC_F = os.path.join(CSRC, "logf256.inc")
HERE = os.path.dirname(os.path.abspath(__file__))


def parse():
    text = open(INC).read()
    defs = dict(re.findall(r"#define (TK_\w+) (\S+)\n", text))
    rows = [tuple(float.fromhex(v) for v in m)
            for m in re.findall(r"\{(\S+), (\S+), (\S+), (\S+)\}", text)]
    return defs, rows


def z_interval(j, entries, split):
    lo = 1 + Fraction(j, entries)
    hi = lo + Fraction(1, entries)
    return (lo / 2, hi / 2) if j >= split else (lo, hi)


def test_shape_and_constants():
    defs, rows = parse()
    entries, split = int(defs["TK_LOG_ENTRIES"]), int(defs["TK_LOG_SPLIT"])
    assert len(rows) == entries == 128
    mp.mp.dps = 60
    hi, lo = float.fromhex(defs["TK_LN2_HI"]), float.fromhex(defs["TK_LN2_LO"])
    assert (Fraction(hi) * 2 ** 45).denominator == 1
    assert abs(mp.mpf(hi) + mp.mpf(lo) - mp.log(2)) < mp.mpf(2) ** -100
    # the reduction covers [0.6875, 1.375): entry 47 ends at 1.375, entry 48 starts at 0.6875
    assert z_interval(split - 1, entries, split)[1] == Fraction(11, 8)
    assert z_interval(split, entries, split)[0] == Fraction(11, 16)


def test_entries():
    defs, rows = parse()
    entries, split = int(defs["TK_LOG_ENTRIES"]), int(defs["TK_LOG_SPLIT"])
    mp.mp.dps = 60
    for j, (invc, nhi, nlo, c) in enumerate(rows):
        C = Fraction(c)
        a, b = z_interval(j, entries, split)
        # c has at most 10 significant bits and lies in the entry's binade, so z - c is exact
        assert (C * 2 ** 9 * (2 if C < 1 else 1)).denominator == 1, j
        assert (C < 1) == (j >= split) or C == 1
        # |q| = |z - c| / c within 2^-8, or 2^-7 at the first entry (c = 1 next to x = 1)
        q = max(abs(a - C), abs(b - C)) / C
        assert q <= Fraction(1, 128 if j == 0 else 256), (j, float(q))
        if j in (0, entries - 1):
            assert C == 1 and invc == 1.0 and nhi == 0.0 and nlo == 0.0
        assert invc == float(1 / C)  # Fraction -> float rounds to nearest
        assert (Fraction(nhi) * 2 ** 45).denominator == 1
        exact = -mp.log(mp.mpf(C.numerator) / C.denominator)
        assert abs(mp.mpf(nhi) + mp.mpf(nlo) - exact) <= mp.mpf(2) ** -98, j
        assert abs(nlo) <= 2.0 ** -46


def test_fma_high_part_is_exact():
    """n ln2_hi + nlog_hi (0 <= n <= 53) needs at most 53 significant bits, so the kernels'
    single fused multiply-add computes it exactly."""
    defs, rows = parse()
    hi = Fraction(float.fromhex(defs["TK_LN2_HI"]))
    for n in range(54):
        for _, nhi, _, _ in rows:
            s = n * hi + Fraction(nhi)
            assert Fraction(float(s)) == s, (n, nhi)


def test_file_matches_generator(tmp_path):
    import importlib.util
    spec = importlib.util.spec_from_file_location("gen_log_table", os.path.join(CSRC, "gen_log_table.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    rows, ln2_hi, ln2_lo = gen.build()
    defs, parsed = parse()
    assert parsed == rows
    assert float.fromhex(defs["TK_LN2_HI"]) == ln2_hi and float.fromhex(defs["TK_LN2_LO"]) == ln2_lo
    assert parse_f()[1] == gen.build_f32()


def parse_f():
    text = open(INC_F).read()
    defs = dict(re.findall(r"#define (TK_\w+) (\S+)\n", text))
    rows = [tuple(float.fromhex(v) for v in m) for m in re.findall(r"\{(\S+), (\S+)\}", text)]
    return defs, rows


def sig_bits(x):
    f = Fraction(x)
    while f.denominator != 1:
        f *= 2
    n = f.numerator
    while n % 2 == 0:
        n //= 2
    return n.bit_length()


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
