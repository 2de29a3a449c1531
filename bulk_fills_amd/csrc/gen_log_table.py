"""Writes the reduction tables of the exponential fills' logarithms: log256.inc (f64) and
logf256.inc (f32).

Both logarithms reduce after Tang (1990, "Table-driven implementation of the logarithm
function in IEEE floating-point arithmetic", ACM TOMS 16(4)): for x = 1 - u in (0, 1],

    x = 2^E z,  z in [0.6875, 1.375)      (the leading fraction bits of x pick entry j)
    ln x = E ln 2 - ln v_j + ln(1 + q),   q = z v_j - 1,

with a multiplier v_j close to 1 / z over the entry.  Giving v_j few significant bits makes
q exact in one fused multiply-add (the product z v_j has few more bits than z, and its
leading bits cancel against 1), so neither c_j nor a correction term is read.  The kernels
keep z in [1, 2) and put the halving into the stored multiplier m_j (z m_j = (z / 2) v_j
exactly).  v_0 = v_255 = 1: the entries next to x = 1 then reduce to ln(1 + q) with q = z - 1
exact (after the halving for j = 255), and -ln x keeps its relative accuracy for x just
below 1 (u near 0), where -ln x ~ u.

f64 (log256.inc).  x = 1 - u on the 2^-53 grid has up to 53 significant bits.  256 entries
(entry j: z in 1 + [j, j+1)/256, halved into [0.6875, 1) from j = 96 on); v_j has at most 9
significant bits, chosen to minimise max |q| over the entry, and the generator checks
|q| < 2^-8 at both ends of every entry, which makes z m_j - 1 exact for every z of it.  Per
entry 16 bytes:
    l_hi     ln v_j rounded to a multiple of 2^-45
    m        the high word of m_j (its low word is zero: 9 significant bits)
    l_lo     the high word of ln v_j - l_hi rounded to 21 significant bits (low word zero)
and ln 2 = LN2_HI + LN2_LO with LN2_HI a multiple of 2^-45, so that n LN2_HI + l_hi
(0 <= n <= 53) is exact in one fused multiply-add.

f32 (logf256.inc).  x = k 2^-24 (1 <= k <= 2^24) has at most 24 significant bits, so v_j
may have 24 and q is still exact.  256 entries (|q| <= 2^-9, 2^-8 at j = 0), halved from
entry 96 on; per entry
    m        v_j = 1 / c_j rounded to 24 significant bits (1 at j = 0 and j = 255), halved
             for j >= 96: the multiplier of z in [1, 2)
    l        ln v_j rounded to nearest, so that -ln x = n ln 2 + l - ln(1 + q)

Run:  python gen_log_table.py  (rewrites log256.inc and logf256.inc next to this file).
"""
import os
from fractions import Fraction

import mpmath as mp
from mpmath.libmp import to_float

mp.mp.dps = 50
HI_QUANTUM = 45
D_ENTRIES = 256
D_SPLIT = 96  # entries from here on halve z into [0.6875, 1)
D_VBITS = 9
D_ZULP = Fraction(1, 1 << 52)  # spacing of z in [1, 2)


def split_hi(x):
    """x rounded to a multiple of 2^-HI_QUANTUM, and the nearest double of the rest."""
    hi = mp.nint(x * mp.mpf(2) ** HI_QUANTUM) / mp.mpf(2) ** HI_QUANTUM
    return to_float(hi._mpf_, rnd="n"), to_float((x - hi)._mpf_, rnd="n")


def d_interval(j):
    """The reduced arguments of entry j: [a, b) (b excluded)."""
    a = 1 + Fraction(j, D_ENTRIES)
    b = a + Fraction(1, D_ENTRIES)
    return (a / 2, b / 2) if j >= D_SPLIT else (a, b)


def d_max_q(j, v):
    """max |z v - 1| over the z of entry j (its last z is b less one z spacing)."""
    a, b = d_interval(j)
    last = b - (D_ZULP / 2 if j >= D_SPLIT else D_ZULP)
    return max(abs(a * v - 1), abs(last * v - 1))


def round_bits(x, bits):
    """The mpf x rounded to nearest at `bits` significant bits, as a double (exact)."""
    with mp.workprec(bits):
        r = +x
    return to_float(r._mpf_, rnd="n")


def build():
    """Rows (l_hi, m, l_lo) of the f64 table, and LN2_HI, LN2_LO."""
    rows = []
    for j in range(D_ENTRIES):
        if j in (0, D_ENTRIES - 1):
            v = Fraction(1)
        else:
            a, b = d_interval(j)
            v0 = round_sig(2 / (a + b), D_VBITS)
            q0 = quantum(v0, D_VBITS)
            cands = [c for c in (v0 + d * q0 for d in range(-2, 3)) if round_sig(c, D_VBITS) == c]
            v = min(cands, key=lambda c: (d_max_q(j, c), c))
        assert d_max_q(j, v) < Fraction(1, 256), j
        m = v / 2 if j >= D_SPLIT else v
        mf = float(m)
        assert Fraction(mf) == m
        lv = mp.log(mp.mpf(v.numerator) / v.denominator)
        hi = mp.nint(lv * mp.mpf(2) ** HI_QUANTUM) / mp.mpf(2) ** HI_QUANTUM
        rows.append((to_float(hi._mpf_, rnd="n"), mf, round_bits(lv - hi, 21)))
    ln2_hi, ln2_lo = split_hi(mp.log(2))
    return rows, ln2_hi, ln2_lo


def quantum(v, bits):
    """The spacing of `bits`-significant-bit numbers at the Fraction v > 0."""
    e = 0
    while v >= 2:
        v /= 2
        e += 1
    while v < 1:
        v *= 2
        e -= 1
    return Fraction(2) ** (e - (bits - 1))


def high_word(f):
    import struct
    return struct.unpack("<Q", struct.pack("<d", f))[0] >> 32


F32_ENTRIES = 256
F32_SPLIT = 96  # entries from here on halve z into [0.6875, 1)
F32_VBITS = 24


def f32_centre(j):
    if j in (0, F32_ENTRIES - 1):
        return Fraction(1)
    mid = 1 + Fraction(2 * j + 1, 2 * F32_ENTRIES)
    return mid / 2 if j >= F32_SPLIT else mid


def round_sig(x, bits):
    """The Fraction x rounded to nearest (ties to even) at `bits` significant bits."""
    e = 0
    while x >= 2:
        x /= 2
        e += 1
    while x < 1:
        x *= 2
        e -= 1
    m = x * 2 ** (bits - 1)
    r = round(m)  # Fraction rounds half to even
    return Fraction(r, 2 ** (bits - 1)) * Fraction(2) ** e


def build_f32():
    rows = []
    for j in range(F32_ENTRIES):
        v = round_sig(1 / f32_centre(j), F32_VBITS)
        m = v / 2 if j >= F32_SPLIT else v
        mf = float(m)
        assert Fraction(mf) == m
        lf = to_float(mp.log(mp.mpf(v.numerator) / v.denominator)._mpf_, rnd="n")
        rows.append((mf, lf))
    return rows


def write_f32():
    L = ["// Generated by gen_log_table.py: reduction table of the f32 exponential's logarithm",
         "// (arguments k 2^-24; exact reduction q = z v - 1).  Do not edit.",
         f"#define TK_LOGF_ENTRIES {F32_ENTRIES}",
         f"#define TK_LOGF_SPLIT {F32_SPLIT}",
         "// {m = v (halved from entry TK_LOGF_SPLIT on), ln v; v = 1 / c rounded to 24 significant bits}",
         "#define TK_LOGF_TABLE_ROWS \\"]
    for v, lv in build_f32():
        L.append(f"  {{{v.hex()}, {lv.hex()}}}, \\")
    L.append("")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "logf256.inc")
    with open(path, "w") as f:
        f.write("\n".join(L) + "\n")
    return path


def write_f64():
    rows, ln2_hi, ln2_lo = build()
    L = ["// Generated by gen_log_table.py: reduction table of the f64 exponential's logarithm",
         "// (arguments on the 2^-53 grid; exact reduction q = z m - 1).  Do not edit.",
         f"#define TK_LOGD_ENTRIES {D_ENTRIES}",
         f"#define TK_LOGD_SPLIT {D_SPLIT}",
         f"#define TK_LN2_HI {ln2_hi.hex()}",
         f"#define TK_LN2_LO {ln2_lo.hex()}",
         "// {l_hi = ln v (multiple of 2^-45), high word of m = v (halved from entry TK_LOGD_SPLIT on),",
         "//  high word of l_lo = ln v - l_hi (21 significant bits)}; v has at most 9 significant bits",
         "#define TK_LOGD_TABLE_ROWS \\"]
    for hi, m, lo in rows:
        L.append(f"  {{{hi.hex()}, 0x{high_word(m):08X}u, 0x{high_word(lo):08X}u}}, \\")
    L.append("")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "log256.inc")
    with open(path, "w") as f:
        f.write("\n".join(L) + "\n")
    return path


def main():
    return write_f32(), write_f64()


if __name__ == "__main__":
    print(main())
