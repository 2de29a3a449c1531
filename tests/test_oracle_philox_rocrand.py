"""Pins the oracle's Philox4x32-10 words against an independent implementation: rocRAND's
Philox4x32-10 generator (ROCm's random-number library), run on the CPU through its host
generator.

Philox4x32-10 (Salmon et al., SC'11) is the cuRAND-comparable variant's word source; the
pages do not define it and no known-answer values are available here, so its oracle was
pinned only structurally (its blocks invert to their counters).  rocRAND's sequence for
seed s at offset o is word o, o+1, ... of the stream whose block b is Philox4x32-10 of
counter (lo32 b, hi32 b, 0, 0) under key (lo32 s, hi32 s), output lanes in order: the
layout the oracle reads (key, counter, rounds, multipliers, Weyl constants and lane
order).  Counter words 2 and 3, which the substreams use, stay zero here; the inverse-round
pin covers the round function at any counter.

Marked gpu: rocRAND sets up device state even for a host generator, so it needs a HIP
device, though the values compared are computed on the CPU by the oracle and by rocRAND.
Nothing from the library's kernels is involved."""
import ctypes as C
import os

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

ROCRAND = "/opt/rocm/lib/librocrand.so"
PHILOX4_32_10 = 404                      # rocrand_rng_type
ORDERINGS = (100, 101, 103)              # ROCRAND_ORDERING_PSEUDO_{BEST, DEFAULT, LEGACY}


@pytest.fixture(scope="module")
def rocrand():
    if not os.path.exists(ROCRAND):
        pytest.skip("rocRAND is not installed")
    import torch
    torch.cuda.init()  # the HIP runtime torch loaded serves rocRAND too
    lib = C.CDLL(ROCRAND)
    gen = C.c_void_p()
    assert lib.rocrand_create_generator_host_blocking(C.byref(gen), PHILOX4_32_10) == 0
    yield lib, gen
    lib.rocrand_destroy_generator(gen)


def rocrand_words(lib, gen, seed, offset, n, ordering):
    assert lib.rocrand_set_ordering(gen, ordering) == 0
    assert lib.rocrand_set_seed(gen, C.c_ulonglong(seed)) == 0
    assert lib.rocrand_set_offset(gen, C.c_ulonglong(offset)) == 0
    out = np.zeros(n, dtype=np.uint32)
    assert lib.rocrand_generate(gen, out.ctypes.data_as(C.c_void_p), C.c_size_t(n)) == 0
    return out


@pytest.mark.parametrize("seed", (0, 1, 7, 0x123456789ABCDEF0, 0xFFFFFFFFFFFFFFFF))
def test_philox_words_equal_rocrand(rocrand, seed):
    lib, gen = rocrand
    # offsets: aligned and unaligned to a block, and past 2^34 words (the counter's high word)
    for offset in (0, 1, 3, 4, 5, (1 << 34) + 6, (1 << 40) + 2):
        for ordering in ORDERINGS:
            n = 1 << 14
            got = rocrand_words(lib, gen, seed, offset, n, ordering)
            want = oracle.philox_fill_u32(seed, offset, n)
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, (f"seed {seed:#x} offset {offset} ordering {ordering}: {bad.size} words differ, "
                                   f"first at {bad[0]}: rocRAND {got[bad[0]]:#x} oracle {want[bad[0]]:#x}")
