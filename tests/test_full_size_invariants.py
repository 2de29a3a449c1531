"""Whole 2^28-element fills on the device, in the benchmark's launch configuration, checked
by properties that hold at any size (the oracle checks these sizes on sampled elements in
the parity tests):

  - the cut invariant (tandem-sycl, "Design", §Fills and §Normals): the fill started j
    draws later, into an output shifted by one element, equals the whole fill from
    element j, for every fill;
  - the byte identities between widths (tandem-cuda, "Performance", §GPU: narrow types
    write fewer bytes of the same stream; 64-bit draws are word pairs);
  - statistics of the f64 normals and exponentials at the full size.  Their values come
    from the low bits of the words (the layer index) or from a transform that spreads
    every bit, and the oracle's own fill of the same key and start passes the same tests
    (1000 equiprobable bins, p = 0.27 and 0.61).  The uniform-derived fills are not
    tested this way: over an aligned block of consecutive counters the high bits of the
    page's hash are uneven, a property of the generator that the oracle pins record.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import bulk_fills_amd as tk
import tk_inputs
from gpu_harness import log

pytestmark = pytest.mark.gpu

N = tk_inputs.FULL_N
CUTS = (1, 3, 4097, (1 << 27) + 5)
DEV = torch.device("cuda")
MISS_P = 0.0042765667  # exact miss probability of the 1024-layer ziggurat (oracle pins)

_table = None


def table():
    global _table
    if _table is None:
        _table = tk.tk_alias_create(tk_inputs.zipf_weights())
    return _table


_x = None


def dropout_x():
    global _x
    if _x is None:
        _x = torch.empty(N + 1, dtype=torch.float32, device=DEV)
        tk.tk_fill_normal_f32(tk_inputs.DROPOUT_X_KEY, 0, N + 1, _x)
    return _x


def dropout(start, n, out, shift):
    # element k reads x[shift + k]: the fill from draw s + j over x[j:] is the cut
    tk.tk_dropout_f32(tk_inputs.DROPOUT_KEY, start, n, tk_inputs.DROPOUT_P, dropout_x()[shift:shift + n].data_ptr(),
                      out)


# name -> (fill(start, n, out), torch dtype); `out` a device address
FILLS = {
    "u8": (lambda s, n, o: tk.tk_fill_u8(1, s, n, o), torch.uint8),
    "u16": (lambda s, n, o: tk.tk_fill_u16(1, s, n, o), torch.int16),
    "u32": (lambda s, n, o: tk.tk_fill_u32(1, s, n, o), torch.int32),
    "u64": (lambda s, n, o: tk.tk_fill_u64(1, s, n, o), torch.int64),
    "f16_bits": (lambda s, n, o: tk.tk_fill_f16_bits(1, s, n, o), torch.int16),
    "f32": (lambda s, n, o: tk.tk_fill_f32(1, s, n, o), torch.int32),
    "f64": (lambda s, n, o: tk.tk_fill_f64(1, s, n, o), torch.int64),
    "bool": (lambda s, n, o: tk.tk_fill_bool(1, s, n, o), torch.uint8),
    "u32_below": (lambda s, n, o: tk.tk_fill_u32_below(1, s, n, 1000, o), torch.int32),
    "u64_below": (lambda s, n, o: tk.tk_fill_u64_below(1, s, n, (1 << 64) - 2, o), torch.int64),
    "i64_below32": (lambda s, n, o: tk.tk_fill_i64_below32(1, s, n, tk_inputs.LOW, tk_inputs.LOW_BOUND, o),
                    torch.int64),
    "normal_f64": (lambda s, n, o: tk.tk_fill_normal_f64(1, s, n, o), torch.int64),
    "normal_f32": (lambda s, n, o: tk.tk_fill_normal_f32(1, s, n, o), torch.int32),
    "normal_f32_half_turn": (lambda s, n, o: tk.tk_fill_normal_f32_half_turn(1, s, n, o), torch.int32),
    "randn_f32": (lambda s, n, o: tk.tk_fill_randn_f32(1, s, n, o), torch.int32),
    "exponential_f64": (lambda s, n, o: tk.tk_fill_exponential_f64(1, s, n, o), torch.int64),
    "exponential_f32": (lambda s, n, o: tk.tk_fill_exponential_f32(1, s, n, o), torch.int32),
    "choice_u32": (lambda s, n, o: tk.tk_fill_choice_u32(1, s, n, table(), o), torch.int32),
    "philox_u32": (lambda s, n, o: tk.tk_philox_fill_u32(1, s, n, o), torch.int32),
    "philox_u64_below": (lambda s, n, o: tk.tk_philox_fill_u64_below(1, s, n, 1000, o), torch.int64),
    "philox_normal_f32": (lambda s, n, o: tk.tk_philox_fill_normal_f32(1, s, n, o), torch.int32),
    "philox_normal_f64": (lambda s, n, o: tk.tk_philox_fill_normal_f64(1, s, n, o), torch.int64),
}


@pytest.mark.parametrize("name", list(FILLS) + ["dropout_f32"])
def test_cut_invariant_full_size(name):
    """fill(s + j, N - j) into out[1:] equals fill(s, N)[j:], bit for bit (shifting the
    output by one element changes which lane, tile and work-group computes each draw)."""
    if name == "dropout_f32":
        dt = torch.int32
    else:
        fill, dt = FILLS[name]
    isz = torch.empty(0, dtype=dt).element_size()
    start = 3
    whole = torch.empty(N, dtype=dt, device=DEV)
    part = torch.empty(N + 1, dtype=dt, device=DEV)
    log(f"{name}: whole fill at start {start}")
    if name == "dropout_f32":
        dropout(start, N, whole.data_ptr(), 0)
    else:
        fill(start, N, whole.data_ptr())
    for j in CUTS:
        log(f"{name}: cut at {j}")
        part.fill_(0x55 if isz == 1 else 0x5555)
        if name == "dropout_f32":
            dropout(start + j, N - j, part.data_ptr() + isz, j)
        else:
            fill(start + j, N - j, part.data_ptr() + isz)
        torch.cuda.synchronize()
        same = torch.eq(whole[j:], part[1:1 + N - j])
        if not bool(same.all()):
            k = int(torch.nonzero(~same)[0, 0])
            raise AssertionError(f"{name}: cut {j} differs first at element {j + k}")
        assert int(part[0]) == (0x55 if isz == 1 else 0x5555), f"{name}: cut {j} wrote before its output"
    del whole, part


def test_widths_share_one_stream():
    """u8, u16 and u64 fills are the bytes, halves and word pairs of the u32 fill; bool
    element i is bit i & 31 of word i >> 5; i32_below with a low bound is u32_below plus
    the bound; Philox u64 draws are pairs of Philox u32 words."""
    m = N // 4
    s = 5
    w = torch.empty(2 * m, dtype=torch.int32, device=DEV)
    log("widths: u32")
    tk.tk_fill_u32(2, s, 2 * m, w)
    b8 = torch.empty(4 * m, dtype=torch.uint8, device=DEV)
    tk.tk_fill_u8(2, 4 * s, 4 * m, b8)
    h16 = torch.empty(2 * m, dtype=torch.int16, device=DEV)
    tk.tk_fill_u16(2, 2 * s, 2 * m, h16)
    torch.cuda.synchronize()
    assert torch.equal(b8, w[:m].view(torch.uint8)), "u8 bytes"
    assert torch.equal(h16, w[:m].view(torch.int16)), "u16 halves"
    del b8, h16
    log("widths: u64")
    q = torch.empty(m, dtype=torch.int64, device=DEV)
    tk.tk_fill_u64(2, s // 2, m, q)
    w2 = torch.empty(2 * m, dtype=torch.int32, device=DEV)
    tk.tk_fill_u32(2, 2 * (s // 2), 2 * m, w2)
    torch.cuda.synchronize()
    assert torch.equal(q, w2.view(torch.int64)), "u64 word pairs"
    del q, w2
    log("widths: bool")
    nb = 32 * (m // 8)
    bb = torch.empty(nb, dtype=torch.uint8, device=DEV)
    tk.tk_fill_bool(2, 32 * s, nb, bb)
    torch.cuda.synchronize()
    words = w[: nb // 32].to(torch.int64) & 0xFFFFFFFF
    bits = (words[:, None] >> torch.arange(32, device=DEV)) & 1
    assert torch.equal(bb.view(-1, 32).to(torch.int64), bits), "bool bits"
    del bb, bits, words
    log("widths: bounded with a low bound")
    a = torch.empty(m, dtype=torch.int32, device=DEV)
    c = torch.empty(m, dtype=torch.int32, device=DEV)
    tk.tk_fill_u32_below(2, s, m, tk_inputs.LOW_BOUND, a)
    tk.tk_fill_i32_below(2, s, m, tk_inputs.LOW, tk_inputs.LOW_BOUND, c)
    torch.cuda.synchronize()
    assert torch.equal(c, a + tk_inputs.LOW), "i32_below = u32_below + low"
    del a, c
    log("widths: Philox u64")
    pq = torch.empty(m, dtype=torch.int64, device=DEV)
    pw = torch.empty(2 * m, dtype=torch.int32, device=DEV)
    tk.tk_philox_fill_u64(9, 7, m, pq)
    tk.tk_philox_fill_u32(9, 14, 2 * m, pw)
    torch.cuda.synchronize()
    assert torch.equal(pq, pw.view(torch.int64)), "Philox u64 word pairs"


def chi_square_p(values, edges):
    counts = torch.bincount(torch.bucketize(values, torch.from_numpy(edges).to(DEV)), minlength=edges.size + 1)
    return stats.chisquare(counts.cpu().numpy().astype(np.float64)).pvalue


def test_normal_f64_statistics_full_size():
    z = torch.empty(N, dtype=torch.float64, device=DEV)
    tk.tk_debug_set_normal_f64_mode(2)  # fused and counted
    try:
        log("normal_f64 statistics: fill")
        tk.tk_fill_normal_f64(1, 0, N, z)
        misses = tk.tk_debug_last_miss_count()
    finally:
        tk.tk_debug_set_normal_f64_mode(0)
    sd = np.sqrt(N * MISS_P * (1 - MISS_P))
    assert abs(misses - N * MISS_P) < 5 * sd, f"misses {misses}, expected {N * MISS_P:.0f} ± {sd:.0f}"
    mean, var = float(z.mean()), float(z.var())
    assert abs(mean) < 5 / np.sqrt(N), mean
    assert abs(var - 1) < 5 * np.sqrt(2 / N), var
    assert float(z.abs().max()) < 9.0  # the tail beyond r = 3.44 stays plausible at 2^28 draws
    p = chi_square_p(z, stats.norm.ppf(np.linspace(0, 1, 1001)[1:-1]))
    log(f"normal_f64: misses {misses}, mean {mean:.3e}, var {var:.6f}, chi-square p {p:.3g}")
    assert p > 1e-4


def test_exponential_f64_statistics_full_size():
    e = torch.empty(N, dtype=torch.float64, device=DEV)
    log("exponential_f64 statistics: fill")
    tk.tk_fill_exponential_f64(1, 0, N, e)
    mean = float(e.mean())
    assert float(e.min()) >= 0.0
    assert abs(mean - 1) < 5 / np.sqrt(N), mean
    p = chi_square_p(e, -np.log1p(-np.linspace(0, 1, 1001)[1:-1]))
    log(f"exponential_f64: mean {mean:.6f}, chi-square p {p:.3g}")
    assert p > 1e-4
