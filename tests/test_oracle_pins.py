"""Pins for the CPU oracle: checks it against what the pages and the mathematics fix,
never against itself.  Runs on the CPU (no GPU marker).

Each test names the page passage or the closed form it relies on; several of them also
show that a plausible misreading (an arithmetic shift, a swapped operand, a dropped term)
would fail.
"""
import math

import numpy as np
import pytest
from scipy import special, stats

import oracle
from golden.load import load

PHOBOS = load("phobos_random.txt")
TANDEM = load("tandem_ziggurat.txt")
PUBLISHED_R = load("ziggurat_published_r.txt")

U32 = np.uint32
M32 = (1 << 32) - 1


# ---------------------------------------------------------------------------------------
# hash32 / uniform  (Phobos, "Random numbers", §hash32, §uniform, figure)
# ---------------------------------------------------------------------------------------

def _phobos_hash_i32(x):
    """The page's expression evaluated the way the page says Phobos evaluates it: wrapping
    i32 multiplies, and >> arithmetic on a signed value with the copied-in bits masked off.
    Constants come from the fixture (the page's decimals)."""
    x = np.asarray(x, dtype=np.int64)

    def wrap(v):
        return ((v + (1 << 31)) & M32) - (1 << 31)

    def mix(v, s):
        shifted = (v >> s) & ((1 << (32 - s)) - 1)  # arithmetic shift, masked
        return wrap(v ^ shifted)

    x = wrap(x)
    x = mix(x, PHOBOS["hash_shift_1"])
    x = wrap(x * PHOBOS["hash_mul_1"])
    x = mix(x, PHOBOS["hash_shift_2"])
    x = wrap(x * PHOBOS["hash_mul_2"])
    x = mix(x, PHOBOS["hash_shift_3"])
    return (x & M32).astype(np.uint64)


def test_hash_matches_page_i32_expression():
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.integers(0, 1 << 32, 20000, dtype=np.uint64),
                         np.array([0, 1, 2, 0x7FFFFFFF, 0x80000000, M32], dtype=np.uint64)])
    want = _phobos_hash_i32(xs.astype(np.int64))
    got = np.array([oracle.hash32(int(x)) for x in xs], dtype=np.uint64)
    assert np.array_equal(got, want)


def _inverse_hash(y):
    """Undo each step of lowbias32 (xorshift and odd multiply are bijections on u32)."""
    def unxorshift(v, s):
        r = v
        for _ in range(32 // s + 1):
            r = v ^ (r >> s)
        return r & M32

    m1 = PHOBOS["hash_mul_1"] & M32
    m2 = PHOBOS["hash_mul_2"] & M32
    y = unxorshift(y, 16)
    y = (y * pow(m2, -1, 1 << 32)) & M32
    y = unxorshift(y, 15)
    y = (y * pow(m1, -1, 1 << 32)) & M32
    return unxorshift(y, 16)


def test_hash_is_a_bijection_with_zero_fixed():
    assert oracle.hash32(0) == 0
    rng = np.random.default_rng(12)
    for x in rng.integers(0, 1 << 32, 3000, dtype=np.uint64):
        assert _inverse_hash(oracle.hash32(int(x))) == int(x)


def test_figure_mean_and_grid():
    """Figure: seed 1, an 8 x 32 tile, c = r*32 + col: mean 0.513, every value k * 2^-23."""
    rows, cols, seed = PHOBOS["figure_rows"], PHOBOS["figure_cols"], PHOBOS["figure_seed"]
    c = (np.arange(rows)[:, None] * cols + np.arange(cols)[None, :]).ravel()
    u = np.array([oracle.uniform(seed, int(ci)) for ci in c], dtype=np.float64)
    assert u.size == 256
    assert round(u.mean(), 3) == PHOBOS["figure_mean"]
    assert np.all((u >= 0) & (u < 1))
    k = u / PHOBOS["uniform_scale"]
    assert np.array_equal(k, np.floor(k)) and k.max() <= PHOBOS["uniform_mask"]
    # the f32 fill is the same function of the flat counter
    assert np.array_equal(oracle.fill_f32(seed, 0, 256), u.astype(np.float32))


def test_figure_rejects_plausible_misreadings():
    """The printed mean tells the logical-shift, counter ^ hash32(seed), low-bits reading
    apart from its neighbours (so a mistake in any of them would fail the pin above)."""
    c = np.arange(256, dtype=np.uint64)
    h = lambda v: _phobos_hash_i32(np.asarray(v, dtype=np.int64))
    hs = int(h(np.array([1]))[0])
    target = PHOBOS["figure_mean"]
    low23 = lambda w: (w & 8388607).astype(np.float64) * 2.0 ** -23
    assert round(low23(h(c ^ hs)).mean(), 3) == target
    assert round(low23(h(c) ^ hs).mean(), 3) != target          # hash of counter, then xor
    assert round(low23(h(c ^ 1)).mean(), 3) != target           # seed not hashed
    assert round(((h(c ^ hs) >> 9).astype(np.float64) * 2.0 ** -23).mean(), 3) != target  # high bits

    def arith_hash(v):  # shifts left arithmetic (sign bits not masked)
        v = np.asarray(v, dtype=np.int64)
        wrap = lambda t: ((t + (1 << 31)) & M32) - (1 << 31)
        v = wrap(v)
        for s, m in ((16, PHOBOS["hash_mul_1"]), (15, PHOBOS["hash_mul_2"])):
            v = wrap(v ^ (v >> s))
            v = wrap(v * m)
        v = wrap(v ^ (v >> 16))
        return (v & M32).astype(np.uint64)

    assert round(low23(arith_hash(c ^ int(arith_hash(np.array([1]))[0]))).mean(), 3) != target


def test_hash_high_bits_over_a_counter_block():
    """Records a property of the page's hash rather than of this code: over the aligned
    block of counters 0 .. 2^20-1 the top 10 bits of the words are uneven (chi-square far
    above its 1023 degrees of freedom for every key tried), while the low 10 bits and the
    top bits at random counters are even."""
    rng = np.random.default_rng(5)
    for key in (1, 2, 3):
        w = oracle.fill_u32(key, 0, 1 << 20)
        assert stats.chisquare(np.bincount(w >> 22, minlength=1024))[0] > 1150
        assert stats.chisquare(np.bincount(w & 1023, minlength=1024))[1] > 1e-4
        r = oracle.fill_u32(key, 0, 0, draws=rng.integers(0, 1 << 32, 1 << 20, dtype=np.uint64))
        assert stats.chisquare(np.bincount(r >> 22, minlength=1024))[1] > 1e-4


def test_word_stream_composition():
    """word(k, c) = hash32(c ^ hash32(k)) (Phobos, §uniform), sub/split built from it."""
    for k, c in [(1, 0), (2, 5), (0xDEADBEEF, M32)]:
        assert oracle.word(k, c) == oracle.hash32(c ^ oracle.hash32(k))
        assert oracle.split(k, c) == oracle.word(k, c)
    assert oracle.sub(7, oracle.P_NORMAL64) == oracle.hash32(oracle.hash32(7) ^ 0x4E4F524D)


# ---------------------------------------------------------------------------------------
# Layout of the typed fills on one stream (tandem-cuda "Performance" §GPU: narrow types
# write fewer bytes; tandem-sycl "Design" §Fills: bool is one byte per bit)
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("key,s", [(1, 0), (3, 5), (0xFFFFFFFF, 1000)])
def test_narrow_and_wide_types_share_the_byte_stream(key, s):
    n = 1024
    w = oracle.fill_u32(key, s, n)
    assert np.array_equal(oracle.fill_u64(key, s, n // 2).view(np.uint8), oracle.fill_u32(key, 2 * s, n).view(np.uint8))
    assert np.array_equal(oracle.fill_u16(key, 2 * s, 2 * n).view(np.uint8), w.view(np.uint8))
    assert np.array_equal(oracle.fill_u8(key, 4 * s, 4 * n), w.view(np.uint8))
    bits = np.unpackbits(w.view(np.uint8), bitorder="little")
    assert np.array_equal(oracle.fill_bool(key, 32 * s, 32 * n), bits)


def test_u64_low_word_is_even_counter():
    d = oracle.fill_u64(9, 3, 100)
    w = oracle.fill_u32(9, 6, 200)
    assert np.array_equal(d & np.uint64(M32), w[0::2].astype(np.uint64))
    assert np.array_equal(d >> np.uint64(32), w[1::2].astype(np.uint64))


def test_f32_f64_f16_grids():
    w = oracle.fill_u32(4, 0, 4096)
    f = oracle.fill_f32(4, 0, 4096)
    assert np.array_equal(f.astype(np.float64) * 2 ** 23, (w & 8388607).astype(np.float64))
    d = oracle.fill_u64(4, 0, 4096)
    g = oracle.fill_f64(4, 0, 4096)
    assert np.all((g >= 0) & (g < 1))
    assert np.array_equal((g * 2.0 ** 53).astype(np.uint64), d & np.uint64((1 << 53) - 1))
    # f16: numpy's own binary16 conversion of the exact grid value
    h = oracle.fill_u16(4, 0, 4096)
    want = (np.asarray(h & 0x7FF, dtype=np.float64) / 2048.0).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.fill_f16_bits(4, 0, 4096), want)


def test_f16_encoding_of_every_grid_point():
    """Find, for each 11-bit value m, a draw whose u16 has those low bits, and check the
    encoding against numpy's binary16 conversion of m / 2048."""
    h = oracle.fill_u16(5, 0, 1 << 16)
    f = oracle.fill_f16_bits(5, 0, 1 << 16)
    m = h & 0x7FF
    seen = np.zeros(2048, dtype=bool)
    seen[m] = True
    assert seen.all()
    want = (m.astype(np.float64) / 2048.0).astype(np.float16).view(np.uint16)
    assert np.array_equal(f, want)


FILLS = {
    "u8": oracle.fill_u8, "u16": oracle.fill_u16, "u32": oracle.fill_u32, "u64": oracle.fill_u64,
    "f16": oracle.fill_f16_bits, "f32": oracle.fill_f32, "f64": oracle.fill_f64, "bool": oracle.fill_bool,
    "normal_f32": oracle.fill_normal_f32, "normal_f64": oracle.fill_normal_f64,
    "u32_below": lambda k, s, n, draws=None: oracle.fill_u32_below(k, s, n, 1000, draws=draws),
    "u64_below": lambda k, s, n, draws=None: oracle.fill_u64_below(k, s, n, (1 << 64) - 2, draws=draws),
    "i32_below": lambda k, s, n, draws=None: oracle.fill_i32_below(k, s, n, -500, 1000, draws=draws),
    "i64_below32": lambda k, s, n, draws=None: oracle.fill_i64_below32(k, s, n, -500, 1000, draws=draws),
    "i64_below": lambda k, s, n, draws=None: oracle.fill_i64_below(k, s, n, -(1 << 40), 1 << 41, draws=draws),
    "philox_u32": oracle.philox_fill_u32, "philox_f64": oracle.philox_fill_f64,
    "exponential_f64": oracle.fill_exponential_f64, "exponential_f32": oracle.fill_exponential_f32,
    "normal_f32_half_turn": oracle.fill_normal_f32_half_turn, "randn_f32": oracle.fill_randn_f32,
    "philox_u32_below": lambda k, s, n, draws=None: oracle.philox_fill_u32_below(k, s, n, (1 << 31) + 1, draws=draws),
    "philox_u64_below": lambda k, s, n, draws=None: oracle.philox_fill_u64_below(k, s, n, (1 << 63) + 1, draws=draws),
    "philox_normal_f32": oracle.philox_fill_normal_f32, "philox_normal_f64": oracle.philox_fill_normal_f64,
    "philox_choice": lambda k, s, n, draws=None: oracle.philox_fill_choice_u32(
        k, s, n, *oracle.alias_build([1.0, 2.0, 3.0])[:2], draws=draws),
}


@pytest.mark.parametrize("name", sorted(FILLS))
def test_cut_invariant_and_gather(name):
    """tandem-sycl "Design" §Normals: a fill cut at any element equals the whole fill."""
    f = FILLS[name]
    whole = f(2, 3, 777)
    for j in (1, 2, 3, 5, 16, 17, 100, 776):
        assert np.array_equal(f(2, 3 + j, 777 - j).view(np.uint8), whole[j:].view(np.uint8)), j
    idx = np.array([3 + 700, 3, 3 + 64, 3 + 5], dtype=np.uint64)
    assert np.array_equal(f(2, 0, 0, draws=idx).view(np.uint8), whole[idx - 3].view(np.uint8))


def test_counter_space_edges():
    top = 1 << 32
    assert oracle.fill_u32(1, top - 1, 1).size == 1
    with pytest.raises(oracle.OracleError):
        oracle.fill_u32(1, top - 1, 2)
    assert oracle.fill_u64(1, (1 << 31) - 1, 1).size == 1
    with pytest.raises(oracle.OracleError):
        oracle.fill_u64(1, (1 << 31) - 1, 2)
    assert oracle.fill_u8(1, (1 << 34) - 1, 1).size == 1
    with pytest.raises(oracle.OracleError):
        oracle.fill_u8(1, 1 << 34, 1)
    assert oracle.fill_bool(1, (1 << 37) - 1, 1).size == 1
    with pytest.raises(oracle.OracleError):
        oracle.fill_bool(1, 1 << 37, 1)
    # the last word of the counter space is the hash of (2^32 - 1) ^ hash32(key)
    assert oracle.fill_u32(1, top - 1, 1)[0] == oracle.hash32(M32 ^ oracle.hash32(1))


# ---------------------------------------------------------------------------------------
# Bounded integers (perturbation-kernel "Backends" §Why the GPU can be exact: Lemire's
# multiply-shift with rejection; exact threshold of Lemire 2019)
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("s", [1000, (1 << 31) + 1])
def test_lemire32_exhaustive(s):
    """Over all 2^32 words each value in [0, s) is accepted exactly floor(2^32/s) times and
    exactly 2^32 mod s words are rejected (Lemire 2019, Theorem 1 with the exact threshold).
    Values are non-decreasing in the word, so per-value counts come from a binary search."""
    per = (1 << 32) // s
    chunk = 1 << 26
    ramp = np.arange(chunk, dtype=np.uint32)
    x = np.empty(chunk, dtype=np.uint32)
    v = np.empty(chunk, dtype=np.uint32)
    acc = np.empty(chunk, dtype=np.bool_)
    rejected = 0
    counts = np.zeros(s, dtype=np.int64) if s <= 1 << 20 else None
    edges = np.arange(s + 1, dtype=np.uint32) if counts is not None else None
    for base in range(0, 1 << 32, chunk):
        np.add(ramp, np.uint32(base), out=x)
        oracle.lemire32_map(x, s, out=v, acc=acc)
        nrej = chunk - np.count_nonzero(acc)
        rejected += nrej
        if counts is not None:
            counts += np.diff(np.searchsorted(v, edges))
            if nrej:
                np.subtract.at(counts, v[np.flatnonzero(~acc)].astype(np.int64), 1)
    assert rejected == (1 << 32) % s
    if counts is not None:
        assert np.all(counts == per)


def test_lemire_closed_forms():
    rng = np.random.default_rng(3)
    x32 = rng.integers(0, 1 << 32, 1 << 16, dtype=np.uint64).astype(np.uint32)
    for k in (1, 7, 31):  # s = 2^k: no rejection, value = top k bits
        v, acc = oracle.lemire32_map(x32, 1 << k)
        assert acc.all() and np.array_equal(v, x32 >> np.uint32(32 - k))
    v, acc = oracle.lemire32_map(x32, 1)
    assert acc.all() and not v.any()
    # s = 3 * 2^30: x*s mod 2^32 = (3x mod 4) 2^30, rejected iff x = 0 mod 4, value floor(3x/4)
    v, acc = oracle.lemire32_map(x32, 3 << 30)
    xi = x32.astype(np.uint64)
    assert np.array_equal(acc, (xi % 4) != 0)
    assert np.array_equal(v[acc].astype(np.uint64), (3 * xi[acc]) // 4)
    x64 = rng.integers(0, 1 << 64, 1 << 16, dtype=np.uint64)
    for k in (1, 33, 63):
        v, acc = oracle.lemire64_map(x64, 1 << k)
        assert acc.all() and np.array_equal(v, x64 >> np.uint64(64 - k))
    # s = 3 * 2^62: rejected iff x = 0 mod 4; accepted value 3 (x >> 2) + (0, 1, 2)[x%4 - 1]
    v, acc = oracle.lemire64_map(x64, 3 << 62)
    b = x64 & np.uint64(3)
    assert np.array_equal(acc, b != 0)
    want = np.uint64(3) * (x64 >> np.uint64(2)) + np.array([0, 0, 1, 2], dtype=np.uint64)[b]
    assert np.array_equal(v[acc], want[acc])
    # s = 2^64 - 2: x s = -2x mod 2^64 < 2 only for x in {0, 2^63}
    edge = np.array([0, 1, 1 << 63, (1 << 63) + 1, (1 << 64) - 1], dtype=np.uint64)
    v, acc = oracle.lemire64_map(edge, (1 << 64) - 2)
    assert acc.tolist() == [False, True, False, True, True]


@pytest.mark.parametrize("s", [1000, (1 << 31) + 1, (1 << 32) - 2])
def test_bounded_fill_is_map_then_substream(s):
    """Element i: the map of word i if accepted, else of the first accepted word of
    split(i) of sub(key, "BL32") (tandem-cuda "Performance": retries run out of line)."""
    key, start, n = 6, 1000, 4096
    out = oracle.fill_u32_below(key, start, n, s)
    words = oracle.fill_u32(key, start, n)
    v, acc = oracle.lemire32_map(words, s)
    assert np.array_equal(out[acc], v[acc])
    ksub = oracle.sub(key, oracle.P_BELOW32)
    for k in np.flatnonzero(~acc)[:200]:
        sg = oracle.split(ksub, start + int(k))
        for j in range(64):
            vv, aa = oracle.lemire32_map(np.array([oracle.word(sg, j)], dtype=np.uint32), s)
            if aa[0]:
                break
        assert out[k] == vv[0]
    if s == (1 << 31) + 1:
        assert 0.45 < (~acc).mean() < 0.55
        # the retried values follow the uniform law on [0, s) by themselves (a retry that
        # took a word correlated with the rejected one, or a fixed word, would not): 2^16
        # draws at a start far from the others, about 2^15 of them retried, in 16 bins
        big_start, m = 123456789, 1 << 16
        o2 = oracle.fill_u32_below(key, big_start, m, s)
        _, a2 = oracle.lemire32_map(oracle.fill_u32(key, big_start, m), s)
        r = o2[~a2].astype(np.uint64)
        assert r.size > 30000 and r.max() < s
        assert stats.chisquare(np.bincount((r * 16 // s).astype(np.int64), minlength=16))[1] > 1e-4
        assert stats.chisquare(np.bincount((o2.astype(np.uint64) * 16 // s).astype(np.int64), minlength=16))[1] > 1e-4


def test_bounded64_fill_is_map_then_substream():
    key, start, n, s = 8, 77, 4096, (1 << 63) + 1
    out = oracle.fill_u64_below(key, start, n, s)
    v, acc = oracle.lemire64_map(oracle.fill_u64(key, start, n), s)
    assert np.array_equal(out[acc], v[acc])
    ksub = oracle.sub(key, oracle.P_BELOW64)
    for k in np.flatnonzero(~acc)[:100]:
        sg = oracle.split(ksub, start + int(k))
        for j in range(64):
            d = oracle.word(sg, 2 * j) | (oracle.word(sg, 2 * j + 1) << 32)
            vv, aa = oracle.lemire64_map(np.array([d], dtype=np.uint64), s)
            if aa[0]:
                break
        assert out[k] == vv[0]


def test_bounded_low_offsets_and_uniformity():
    """Uniformity is tested on draws at random indices: the high bits of lowbias32 over an
    aligned block of consecutive counters are measurably uneven (a property of the hash
    the page defines; see test_hash_high_bits_over_a_counter_block)."""
    key, n = 1, 1 << 20
    a = oracle.fill_u32_below(key, 0, n, 1000)
    assert np.array_equal(oracle.fill_i32_below(key, 0, n, -500, 1000), a.astype(np.int32) - 500)
    assert np.array_equal(oracle.fill_i64_below32(key, 0, n, -500, 1000), a.astype(np.int64) - 500)
    rng = np.random.default_rng(21)
    d32 = rng.integers(0, 1 << 32, n, dtype=np.uint64)
    a = oracle.fill_u32_below(key, 0, 0, 1000, draws=d32)
    assert stats.chisquare(np.bincount(a, minlength=1000))[1] > 1e-4
    d64 = rng.integers(0, 1 << 31, n, dtype=np.uint64)
    b = oracle.fill_u64_below(key, 0, 0, 1000, draws=d64)
    assert int(b.max()) < 1000 and stats.chisquare(np.bincount(b.astype(np.int64), minlength=1000))[1] > 1e-4
    c = oracle.fill_i64_below(key, 0, 1000, -(1 << 62), 1 << 63)
    assert c.min() >= -(1 << 62) and c.max() < (1 << 62)
    with pytest.raises(oracle.OracleError):
        oracle.fill_i32_below(key, 0, 1, 2 ** 31 - 10, 11)
    with pytest.raises(oracle.OracleError):
        oracle.fill_u32_below(key, 0, 1, 0)


# ---------------------------------------------------------------------------------------
# Ziggurat (tandem-sycl "Design" §Normals; Marsaglia & Tsang 2000)
# ---------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def zig1024():
    return oracle.zig_table(1024)


def test_ziggurat_published_r():
    assert abs(oracle.zig_table(128)[2] - PUBLISHED_R["r_128"]) < 1e-11
    assert oracle.zig_table(256)[2] == PUBLISHED_R["r_256"]


def test_ziggurat_equal_areas(zig1024):
    """Every layer has area v; the base strip is r f(r) + the tail integral (scipy erfc)."""
    import mpmath as mp
    mp.mp.dps = 40
    X, F, r, v = zig1024
    N = TANDEM["layers"]
    f = lambda x: mp.e ** (-mp.mpf(x) ** 2 / 2)
    tail = math.sqrt(math.pi / 2) * special.erfc(r / math.sqrt(2))
    assert abs(r * math.exp(-r * r / 2) + tail - v) < 1e-15
    assert X[1] == r and X[N] == 0 and F[N] == 1.0
    assert abs(X[0] * math.exp(-r * r / 2) - v) < 1e-15
    areas = [mp.mpf(X[i]) * (f(X[i + 1]) - f(X[i])) for i in range(1, N)]
    rel = max(abs(a / v - 1) for a in areas)
    assert rel < 1e-10
    # F holds f at the binary128 edges; at the rounded edges f moves by |f'| * ulp(X) / 2
    for i in range(1, N):
        tol = X[i] * F[i] * np.spacing(X[i]) + 2 * np.spacing(F[i])
        assert abs(float(f(X[i])) - F[i]) <= tol


def test_ziggurat_miss_rate_is_the_pages(zig1024):
    """Exact miss probability of the fast path (threshold per layer by bisection over the
    2^-53 grid, IEEE multiply in numpy) prints as the page's 0.43 %, and the oracle's
    fast-path decision agrees with those thresholds draw by draw."""
    X, F, r, v = zig1024
    N = TANDEM["layers"]
    thr = np.empty(N, dtype=np.uint64)
    for L in range(N):
        lo, hi = 0, 1 << 53
        while lo < hi:
            m = (lo + hi) // 2
            if np.float64(m) * np.float64(2.0 ** -53) * X[L] >= X[L + 1]:
                hi = m
            else:
                lo = m + 1
        thr[L] = lo
    p_miss = float(sum((1 << 53) - int(t) for t in thr)) / (N * 2.0 ** 53)
    assert round(100 * p_miss, 2) == TANDEM["miss_percent"]
    n = 1 << 20
    d = oracle.fill_u64(5, 0, n)
    z, path = oracle.fill_normal_f64(5, 0, n, with_path=True)
    L = (d & np.uint64(N - 1)).astype(np.int64)
    m = d >> np.uint64(11)
    fast = m < thr[L]
    assert np.array_equal(path == 0, fast)
    sign = ((d >> np.uint64(10)) & np.uint64(1)).astype(bool)
    x = m[fast].astype(np.float64) * 2.0 ** -53 * X[L[fast]]
    assert np.array_equal(z[fast], np.where(sign[fast], -x, x))
    k = int((~fast).sum())
    assert abs(k - p_miss * n) < 5 * math.sqrt(n * p_miss)


def test_ziggurat_distribution():
    n = 1 << 23
    z, path = oracle.fill_normal_f64(1, 0, n, with_path=True)
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / n)
    # equiprobable bins under the normal law
    edges = special.ndtri(np.linspace(0, 1, 2049)[1:-1])
    counts = np.bincount(np.searchsorted(edges, z), minlength=2048)
    chi2, p = stats.chisquare(counts)
    assert p > 1e-4
    assert stats.kstest(z[: 1 << 20], "norm").pvalue > 1e-4
    # wedges and tail are reached; tail values lie beyond r and follow the normal tail law
    r = oracle.zig_table(1024)[2]
    assert (path == 1).any() and (path == 2).any() and (path == 3).any()
    t = np.abs(z[path == 2])
    assert t.min() > r
    big = np.abs(z) > r
    p_tail = special.erfc(r / math.sqrt(2))
    assert abs(big.sum() - p_tail * n) < 5 * math.sqrt(p_tail * n)
    cond = lambda x: 1 - special.erfc(x / math.sqrt(2)) / special.erfc(r / math.sqrt(2))
    assert stats.kstest(np.abs(z[big]), cond).pvalue > 1e-4


def test_ziggurat_wedge_density():
    """Values that left the fast path must fill exactly the wedge shapes: the conditional
    density inside layer L's wedge is f(x) - F[L] (the part under the curve), so their
    histogram over many layers matches it (a wedge accepting everything would be flat)."""
    n = 1 << 23
    z, path = oracle.fill_normal_f64(2, 0, n, with_path=True)
    X, F, r, v = oracle.zig_table(1024)
    w = np.abs(z[path == 1])
    # position of each wedge value within its layer's wedge, mapped through the exact
    # conditional CDF: uniform on [0, 1) iff the acceptance test is right.
    L = np.searchsorted(-X[1:], -w, side="left")  # X decreasing: X[L+1] <= w < X[L]
    ok = (X[L + 1] <= w) & (w < X[L])
    assert ok.mean() > 0.999
    w, L = w[ok], L[ok]
    g = lambda x, l: special.erf(x / math.sqrt(2)) * math.sqrt(math.pi / 2) - F[l] * x
    lo, hi = g(X[L + 1], L), g(X[L], L)
    uu = (g(w, L) - lo) / (hi - lo)
    assert stats.kstest(uu, "uniform").pvalue > 1e-4


# ---------------------------------------------------------------------------------------
# f32 normal by Box-Muller (Phobos §randn; tandem-sycl §Normals)
# ---------------------------------------------------------------------------------------

def test_box_muller_even_element_is_phobos_randn():
    n = 1 << 14
    z = oracle.fill_normal_f32(3, 0, 2 * n)
    want = np.array([oracle.randn(3, c) for c in range(n)], dtype=np.float32)
    assert np.max(np.abs(z[0::2] - want)) <= 1e-6


def test_box_muller_pair_geometry():
    """Radius: x_even^2 + x_odd^2 = -2 ln(1 - u1); angle: atan2(x_odd, x_even) = 2 pi t
    with t = u2 wrapped into [-1/2, 1/2)."""
    n = 1 << 16
    z = oracle.fill_normal_f32(7, 0, 2 * n).astype(np.float64)
    u = oracle.fill_f32(7, 0, 2 * n).astype(np.float64)
    u1, u2 = u[0::2], u[1::2]
    r2 = -2.0 * np.log1p(-u1)
    ok = r2 > 1e-4
    assert np.max(np.abs((z[0::2] ** 2 + z[1::2] ** 2)[ok] / r2[ok] - 1)) < 1e-6
    t = np.where(u2 >= 0.5, u2 - 1, u2)
    ang = np.arctan2(z[1::2], z[0::2])
    d = np.angle(np.exp(1j * (ang - 2 * np.pi * t)))
    assert np.max(np.abs(d[r2 > 1e-2])) < 1e-5
    # odd starts hand over the same values (cut invariant at a pair boundary)
    assert np.array_equal(oracle.fill_normal_f32(7, 1, 9), z[1:10].astype(np.float32))


def test_box_muller_tails_and_moments():
    tail = math.sqrt(-2 * math.log(2.0 ** -23))
    assert abs(tail - PHOBOS["randn_tail_near"]) < 0.05
    n = 1 << 22
    z = oracle.fill_normal_f32(1, 0, n).astype(np.float64)
    assert np.abs(z).max() <= tail
    assert abs(z.mean()) < 5 / math.sqrt(n) and abs(z.var() - 1) < 5 * math.sqrt(2 / n)
    assert stats.kstest(z[: 1 << 20], "norm").pvalue > 1e-4


# ---------------------------------------------------------------------------------------
# Dropout (Phobos §dropout)
# ---------------------------------------------------------------------------------------

def test_dropout_special_cases_and_expectation():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(1 << 18).astype(np.float32)
    y, mask = oracle.dropout_f32(8, 0, x, 0.0)
    assert np.array_equal(y.view(np.uint32), x.view(np.uint32)) and mask.all()
    p = np.float32(0.1)
    y, mask = oracle.dropout_f32(8, 0, x, p)
    u = oracle.fill_f32(8, 0, x.size)
    assert np.array_equal(mask.astype(bool), u >= p)
    q = np.float32(1) - p
    assert np.array_equal(y[mask == 1], x[mask == 1] / q)              # IEEE f32 division
    assert np.all(y[mask == 0].view(np.uint32) == 0)                   # +0.0
    n = x.size
    assert abs(mask.mean() - 0.9) < 5 * math.sqrt(0.09 / n)
    ones = np.ones(1 << 20, dtype=np.float32)
    y1 = oracle.dropout_f32(9, 0, ones, 0.25, with_mask=False)
    assert abs(y1.astype(np.float64).mean() - 1) < 5 * math.sqrt(1 / 3 / ones.size)
    # a multiply by the reciprocal would differ on a sizeable share of inputs
    assert np.mean(x / q != x * (np.float32(1) / q)) > 0.05
    for bad in (1.0, -0.1, float("nan")):
        with pytest.raises(oracle.OracleError):
            oracle.dropout_f32(8, 0, x[:4], bad)


# ---------------------------------------------------------------------------------------
# Alias table and choice (tandem-sycl §Fills; Vose 1991)
# ---------------------------------------------------------------------------------------

def _portions(q, alias):
    """Integer mass each index owns across all columns: q[c] for c itself, 2^32 - q[c]
    for alias[c]."""
    n = q.size
    own = np.zeros(n, dtype=object)
    for c in range(n):
        own[c] += int(q[c])
        own[int(alias[c])] += (1 << 32) - int(q[c])
    return own


@pytest.mark.parametrize("weights", [
    [1.0], [1.0, 2.0, 3.0], [0.0, 5.0, 0.0, 1.0], [1.0] * 7, [1e-300, 1.0, 2.0],
    list((np.arange(1000) + 1.0) ** -1.1),
])
def test_alias_masses_exact(weights):
    w = np.array(weights, dtype=np.float64)
    q, al, mass = oracle.alias_build(w)
    n = w.size
    assert sum(int(m) for m in mass) == n << 32
    ideal = w / w.sum() * float(n << 32)
    jmax = int(np.argmax(w))
    dev = np.abs(mass.astype(np.float64) - ideal)
    dev[jmax] = 0
    assert dev.max() <= 1.0 + 1e-6 * ideal.max()
    assert list(_portions(q, al)) == [int(m) for m in mass]
    assert np.all(mass[w == 0] == 0)


def test_choice_matches_exact_probabilities():
    w = (np.arange(1000) + 1.0) ** -1.1
    q, al, mass = oracle.alias_build(w)
    n = w.size
    # number of high words mapping to each column: #{h : (h n) >> 32 = c}
    cols = np.array([-((-(c + 1) << 32) // n) - (-((-c << 32) // n)) for c in range(n)], dtype=object)
    assert sum(cols) == 1 << 32
    prob = np.zeros(n, dtype=np.float64)
    for c in range(n):
        prob[c] += float(cols[c] * int(q[c]))
        prob[int(al[c])] += float(cols[c] * ((1 << 32) - int(q[c])))
    prob /= 2.0 ** 64
    assert np.max(np.abs(prob / (w / w.sum()) - 1)) < 1e-6
    N = 1 << 22
    out = oracle.fill_choice_u32(1, 0, N, q, al)
    counts = np.bincount(out, minlength=n)
    chi2, p = stats.chisquare(counts, prob * N)
    assert p > 1e-4
    # power-of-two category counts: the column is the top bits of the high word
    q4, al4, _ = oracle.alias_build(np.ones(4))
    d = oracle.fill_u64(1, 0, 64)
    o4 = oracle.fill_choice_u32(1, 0, 64, q4, al4)
    colw = (d >> np.uint64(62)).astype(np.uint32)
    coin = (d & np.uint64(M32)).astype(np.uint32)
    assert np.array_equal(o4, np.where(coin < q4[colw], colw, al4[colw]))


# ---------------------------------------------------------------------------------------
# Philox4x32-10: layout, statistics and inversion of the rounds here; its words equal
# rocRAND's (tests/test_oracle_philox_rocrand.py, which needs a HIP device)
# ---------------------------------------------------------------------------------------

def test_philox_layout_and_statistics():
    w = oracle.philox_fill_u32(0x0123456789ABCDEF, 0, 1 << 20)
    d = oracle.philox_fill_u64(0x0123456789ABCDEF, 0, 1 << 19)
    assert np.array_equal(d.view(np.uint32), w)
    f = oracle.philox_fill_f32(0x0123456789ABCDEF, 0, 1 << 20)
    assert np.array_equal(f.astype(np.float64) * 2 ** 23, (w & 8388607).astype(np.float64))
    counts = np.bincount(w.view(np.uint8), minlength=256)
    assert stats.chisquare(counts)[1] > 1e-4
    # the block counter spans 64 bits: blocks 2^32 apart differ
    hi = oracle.philox_fill_u32(1, 4 << 32, 4)
    lo = oracle.philox_fill_u32(1, 0, 4)
    assert not np.array_equal(hi, lo)


def _philox_unround(y, a, b):
    """Undoes one Philox4x32 round under round key (a, b) (Salmon et al., SC'11, section 5:
    the round is a bijection because the multipliers are odd).  The low halves of the two
    products are output lanes 1 and 3, so the multiplied inputs come back through the
    multipliers' inverses mod 2^32; the high halves then strip off lanes 0 and 2."""
    m0, m1 = 0xD2511F53, 0xCD9E8D57
    x2 = (y[1] * pow(m1, -1, 1 << 32)) & 0xFFFFFFFF
    x0 = (y[3] * pow(m0, -1, 1 << 32)) & 0xFFFFFFFF
    x1 = y[0] ^ ((m1 * x2) >> 32) ^ a
    x3 = y[2] ^ ((m0 * x0) >> 32) ^ b
    return [x0, x1, x2, x3]


def _philox_invert(block, key, rounds=10):
    k0, k1 = key & 0xFFFFFFFF, key >> 32
    y = list(block)
    for r in reversed(range(rounds)):
        y = _philox_unround(y, (k0 + r * 0x9E3779B9) & 0xFFFFFFFF, (k1 + r * 0xBB67AE85) & 0xFFFFFFFF)
    return y


def test_philox_blocks_invert_to_their_counters():
    """Structure pin: running ten inverse rounds (each undone from the round's definition,
    not by re-running it) over the oracle's block must give back the counter it was asked
    for, for counters in all four lanes.  A slip in the lane order, the hi/lo halves, the
    key words or the key schedule would not invert.  The constants and the output order are
    pinned by the comparison with rocRAND."""
    rng = np.random.default_rng(7)
    for key in (0, 1, 0xFFFFFFFFFFFFFFFF, 0x0123456789ABCDEF, int(rng.integers(0, 1 << 63))):
        for b in (0, 1, (1 << 32) + 5, (1 << 62) - 1):  # primary blocks: counter (lo32 b, hi32 b, 0, 0)
            blk = [int(v) for v in oracle.philox_fill_u32(key, 4 * b, 4)]
            assert _philox_invert(blk, key) == [b & 0xFFFFFFFF, b >> 32, 0, 0]
        for _ in range(50):  # substream blocks: counter (lo32 i, hi32 i, P, j >> 2)
            i, pur, jb = int(rng.integers(0, 1 << 63)), int(rng.integers(0, 1 << 32)), int(rng.integers(0, 1 << 28))
            blk = [int(oracle.philox_sub_word(key, i, pur, 4 * jb + lane)) for lane in range(4)]
            assert _philox_invert(blk, key) == [i & 0xFFFFFFFF, i >> 32, pur, jb]
            assert _philox_invert(blk, key, rounds=9) != [i & 0xFFFFFFFF, i >> 32, pur, jb]


# ---------------------------------------------------------------------------------------
# Exponentials (tandem-sycl "Design" §Exponentials; tandem-cuda "Performance" §GPU: the
# f32 exponential stays within 0.571 ulp so that 1 - exp(-x) maps back to the draw's own
# 2^-24 grid point)
# ---------------------------------------------------------------------------------------

def _inverse_hash_np(y):
    """Vectorised inverse of lowbias32 over uint64 arrays holding u32 values."""
    M = np.uint64(M32)

    def unxorshift(v, s):
        r = v.copy()
        for _ in range(32 // s + 1):
            r = v ^ (r >> np.uint64(s))
        return r & M

    inv2 = np.uint64(pow(PHOBOS["hash_mul_2"] & M32, -1, 1 << 32))
    inv1 = np.uint64(pow(PHOBOS["hash_mul_1"] & M32, -1, 1 << 32))
    y = unxorshift(y, 16)
    y = (y * inv2) & M
    y = unxorshift(y, 15)
    y = (y * inv1) & M
    return unxorshift(y, 16)


def test_exponential_f32_every_grid_point():
    """For every m < 2^24 build the counter whose word has low bits m (inverse hash), and
    check the oracle's x against the correctly rounded -ln(1 - m 2^-24) (long double) and
    the page's property that 1 - exp(-x) rounds back to m on the 2^-24 grid."""
    key = 11
    m = np.arange(1 << 24, dtype=np.uint64)
    counters = _inverse_hash_np(m) ^ np.uint64(oracle.hash32(key))
    x = oracle.fill_exponential_f32(key, 0, 0, draws=counters)
    assert np.array_equal(oracle.fill_u32(key, 0, 0, draws=counters[:4096]) & 0xFFFFFF, m[:4096].astype(np.uint32))
    u = m.astype(np.longdouble) * np.longdouble(2.0) ** -24
    exact = -np.log1p(-u)
    assert np.array_equal(x, exact.astype(np.float32))
    back = np.rint((-np.expm1(-x.astype(np.longdouble))) * np.longdouble(2.0) ** 24)
    assert np.array_equal(back.astype(np.uint64), m)
    assert x[0] == 0 and not np.signbit(x[0])


def test_exponential_f64_accuracy_and_law():
    import mpmath as mp
    mp.mp.dps = 40
    d = oracle.fill_u64(2, 0, 2000)
    x = oracle.fill_exponential_f64(2, 0, 2000)
    for di, xi in zip(d[:2000], x[:2000]):
        uu = mp.mpf(int(di) & ((1 << 53) - 1)) * mp.mpf(2) ** -53
        ref = -mp.log(1 - uu)
        if xi == 0:
            assert ref == 0
            continue
        assert abs(mp.mpf(xi) - ref) <= mp.mpf(np.spacing(xi)), (di, xi)
    n = 1 << 22
    rng = np.random.default_rng(6)
    z = oracle.fill_exponential_f64(1, 0, 0, draws=rng.integers(0, 1 << 31, n, dtype=np.uint64))
    assert abs(z.mean() - 1) < 5 / math.sqrt(n) and abs(z.var() - 1) < 5 * math.sqrt(8 / n)
    assert stats.kstest(z[: 1 << 20], "expon").pvalue > 1e-4
    f = oracle.fill_exponential_f32(1, 0, 0, draws=rng.integers(0, 1 << 32, n, dtype=np.uint64))
    assert abs(f.mean() - 1) < 5 / math.sqrt(n) and f.min() >= 0


# ---------------------------------------------------------------------------------------
# Generator and normal variants: Philox sources for the bounded, choice and normal fills;
# the pages' half-turn Box-Muller (tandem-sycl "Design" §Normals); Phobos's one normal per
# counter (§randn).  The Philox word source is pinned against rocRAND; these pins tie each
# variant to the maps and laws pinned above.
# ---------------------------------------------------------------------------------------
PK = 0x0123456789ABCDEF


def test_philox_substream_layout():
    """Substream word j of draw i is lane j & 3 of the block with counter
    (lo32 i, hi32 i, P, j >> 2): with P = 0 and j < 4 that is the primary block i."""
    for i in (0, 1, 5, (1 << 32) + 3, (1 << 40) + 17):
        prim = oracle.philox_fill_u32(PK, 4 * i, 4)
        assert [oracle.philox_sub_word(PK, i, 0, j) for j in range(4)] == list(prim)
    a = [oracle.philox_sub_word(PK, 9, oracle.P_BELOW32, j) for j in range(8)]
    b = [oracle.philox_sub_word(PK, 9, oracle.P_BELOW64, j) for j in range(8)]
    c = [oracle.philox_sub_word(PK, 10, oracle.P_BELOW32, j) for j in range(8)]
    assert len({tuple(a), tuple(b), tuple(c)}) == 3
    assert not set(a) & set(oracle.philox_fill_u32(PK, 0, 64))


@pytest.mark.parametrize("s", [1000, (1 << 31) + 1])
def test_philox_bounded_is_map_then_substream(s):
    start, n = (1 << 33) + 5, 4096
    out = oracle.philox_fill_u32_below(PK, start, n, s)
    v, acc = oracle.lemire32_map(oracle.philox_fill_u32(PK, start, n), s)
    assert np.array_equal(out[acc], v[acc])
    for k in np.flatnonzero(~acc)[:200]:
        for j in range(64):
            w = oracle.philox_sub_word(PK, start + int(k), oracle.P_BELOW32, j)
            vv, aa = oracle.lemire32_map(np.array([w], dtype=np.uint32), s)
            if aa[0]:
                break
        assert out[k] == vv[0]
    if s == (1 << 31) + 1:
        assert 0.45 < (~acc).mean() < 0.55
        # retried values are uniform too (a retry that reused the rejected word would not be)
        r = out[~acc]
        assert stats.chisquare(np.bincount((r.astype(np.uint64) * 16 // s).astype(np.int64), minlength=16))[1] > 1e-4


def test_philox_bounded64_is_map_then_substream():
    start, n, s = 77, 4096, (1 << 63) + 1
    out = oracle.philox_fill_u64_below(PK, start, n, s)
    v, acc = oracle.lemire64_map(oracle.philox_fill_u64(PK, start, n), s)
    assert np.array_equal(out[acc], v[acc])
    for k in np.flatnonzero(~acc)[:100]:
        for j in range(64):
            d = oracle.philox_sub_word(PK, start + int(k), oracle.P_BELOW64, 2 * j) | (
                oracle.philox_sub_word(PK, start + int(k), oracle.P_BELOW64, 2 * j + 1) << 32)
            vv, aa = oracle.lemire64_map(np.array([d], dtype=np.uint64), s)
            if aa[0]:
                break
        assert out[k] == vv[0]
    small = oracle.philox_fill_u64_below(PK, 0, 1 << 16, 1000)
    assert small.max() < 1000 and stats.chisquare(np.bincount(small.astype(np.int64), minlength=1000))[1] > 1e-4


def test_philox_choice_is_the_alias_map_of_philox_draws():
    w = (np.arange(1000) + 1.0) ** -1.1
    q, al, _ = oracle.alias_build(w)
    d = oracle.philox_fill_u64(PK, 3, 4096)
    col = ((d >> np.uint64(32)) * np.uint64(1000) >> np.uint64(32)).astype(np.int64)
    coin = (d & np.uint64(M32)).astype(np.uint32)
    assert np.array_equal(oracle.philox_fill_choice_u32(PK, 3, 4096, q, al), np.where(coin < q[col], col, al[col]))
    N = 1 << 21
    counts = np.bincount(oracle.philox_fill_choice_u32(PK, 0, N, q, al), minlength=1000)
    assert stats.chisquare(counts, w / w.sum() * N)[1] > 1e-4


def test_philox_box_muller_geometry_and_law():
    n = 1 << 16
    z = oracle.philox_fill_normal_f32(PK, 0, 2 * n).astype(np.float64)
    u = oracle.philox_fill_f32(PK, 0, 2 * n).astype(np.float64)
    u1, u2 = u[0::2], u[1::2]
    r2 = -2.0 * np.log1p(-u1)
    ok = r2 > 1e-4
    assert np.max(np.abs((z[0::2] ** 2 + z[1::2] ** 2)[ok] / r2[ok] - 1)) < 1e-6
    t = np.where(u2 >= 0.5, u2 - 1, u2)
    d = np.angle(np.exp(1j * (np.arctan2(z[1::2], z[0::2]) - 2 * np.pi * t)))
    assert np.max(np.abs(d[r2 > 1e-2])) < 1e-5
    assert np.array_equal(oracle.philox_fill_normal_f32(PK, 1, 9), z[1:10].astype(np.float32))
    big = oracle.philox_fill_normal_f32(PK, 1 << 40, 1 << 20).astype(np.float64)
    assert stats.kstest(big, "norm").pvalue > 1e-4


def test_philox_ziggurat_fast_path_and_law(zig1024):
    """Draw by draw, the fast path of the Philox ziggurat is that of its Philox 64-bit
    draws (layer, sign and threshold as pinned above), and the values follow the normal law."""
    X, F, r, v = zig1024
    N = 1024
    n = 1 << 19
    d = oracle.philox_fill_u64(PK, 0, n)
    z, path = oracle.philox_fill_normal_f64(PK, 0, n, with_path=True)
    L = (d & np.uint64(N - 1)).astype(np.int64)
    x = (d >> np.uint64(11)).astype(np.float64) * 2.0 ** -53 * X[L]
    fast = x < X[L + 1]
    assert np.array_equal(path == 0, fast)
    sign = ((d >> np.uint64(10)) & np.uint64(1)).astype(bool)
    assert np.array_equal(z[fast], np.where(sign[fast], -x[fast], x[fast]))
    assert abs((~fast).mean() - 0.0042765667) < 5 * math.sqrt(0.0043 / n)
    big, bpath = oracle.philox_fill_normal_f64(PK, 1 << 40, 1 << 22, with_path=True)
    assert (bpath == 1).any() and (bpath == 2).any()
    edges = special.ndtri(np.linspace(0, 1, 1025)[1:-1])
    assert stats.chisquare(np.bincount(np.searchsorted(edges, big), minlength=1024))[1] > 1e-4
    assert np.abs(big[bpath == 2]).min() > r


def test_half_turn_box_muller_negates_the_whole_turn():
    """Angle 2 pi u2 - pi: the same pairs and radius with both values negated (to within
    one f32 rounding, since the two angles round differently in f64; next to a zero of
    cos or sin both values are ~1e-16 and need not be opposite)."""
    n = 1 << 18
    h = oracle.fill_normal_f32_half_turn(4, 0, n)
    w = oracle.fill_normal_f32(4, 0, n)
    diff = np.abs(h.astype(np.float64) + w.astype(np.float64))
    assert np.all(diff <= np.maximum(np.spacing(np.abs(w)).astype(np.float64), 1e-12))
    assert (diff == 0).mean() > 0.999
    u = oracle.fill_f32(4, 0, n).astype(np.float64)
    ang = np.arctan2(h[1::2].astype(np.float64), h[0::2].astype(np.float64))
    dd = np.angle(np.exp(1j * (ang - (2 * np.pi * u[1::2] - np.pi))))
    r2 = -2.0 * np.log1p(-u[0::2])
    assert np.max(np.abs(dd[r2 > 1e-2])) < 1e-5


def test_randn_fill_is_phobos_randn_per_counter():
    """Element k is randn(key, start + k): the cosine of Box-Muller pair start + k, i.e. the
    even element 2(start + k) of the pair fill, to within one f32 rounding."""
    s, n = 11, 1 << 16
    z = oracle.fill_randn_f32(3, s, n)
    pairs = oracle.fill_normal_f32(3, 2 * s, 2 * n)
    diff = np.abs(z.astype(np.float64) - pairs[0::2].astype(np.float64))
    assert np.all(diff <= np.spacing(np.abs(pairs[0::2])).astype(np.float64))
    assert np.array_equal(z[:64], np.array([oracle.randn(3, s + c) for c in range(64)], dtype=np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.fill_randn_f32(3, (1 << 31) - 1, 2)
