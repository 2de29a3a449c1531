"""Pins the oracle's Philox4x32-10 word source against an independent implementation:
rocRAND's Philox4x32-10 (ROCm's random-number library).

Philox4x32-10 (Salmon et al., SC'11) is the cuRAND-comparable variant's word source; the
pages do not define it and no known-answer values are available here.  rocRAND's engine,
started with rocrand_init(seed, subsequence, offset), yields the words of the stream with
key (lo32 seed, hi32 seed) whose block b has counter (lo32 b, hi32 b, lo32 subsequence,
hi32 subsequence), output lanes in order, from word `offset`.  So:
  - the oracle's word w of key k (block w >> 2 at counter (lo32, hi32, 0, 0), lane w & 3)
    is rocRAND's word with seed k, subsequence 0, offset w;
  - the oracle's substream word j of draw i for purpose P (counter (lo32 i, hi32 i, P,
    j >> 2), lane j & 3) is rocRAND's first word with seed k, subsequence P + 2^32 (j >> 2),
    offset 4 i + (j & 3).
That covers the key and counter layout, the constants, the rounds and the output order, in
every counter word.

The CPU tests call rocRAND's header-only engine compiled for the host (tests/rocrand_ref.hip,
built by build()).  The gpu-marked test also checks rocRAND's generator API, whose host
generator computes on the CPU but needs a HIP device to set up; neither involves this
library's kernels."""
import ctypes as C
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
REF = os.path.join(HERE, "librocrand_ref.so")
SEEDS = (0, 1, 7, 0x0123456789ABCDEF, 0x123456789ABCDEF0, 0xFFFFFFFFFFFFFFFF)
# aligned and unaligned to a block, and past 2^34 words (the counter's high word)
OFFSETS = (0, 1, 3, 4, 5, (1 << 34) + 6, (1 << 40) + 2)


@pytest.fixture(scope="module")
def ref():
    if not os.path.exists(REF):
        import build_rocrand_ref
        if build_rocrand_ref.build() is None:
            pytest.skip("rocRAND's headers are not installed")
    lib = C.CDLL(REF)
    f = lib.rocrand_ref_philox_words
    f.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, C.c_uint64, C.c_void_p]
    f.restype = None

    def words(seed, subsequence, offset, n):
        out = np.zeros(n, dtype=np.uint32)
        f(seed, subsequence, offset, n, out.ctypes.data)
        return out
    return words


def first_mismatch(got, want):
    bad = np.flatnonzero(got != want)
    return None if bad.size == 0 else (int(bad[0]), int(got[bad[0]]), int(want[bad[0]]), int(bad.size))


@pytest.mark.parametrize("seed", SEEDS)
def test_primary_words_equal_rocrand(ref, seed):
    for offset in OFFSETS:
        n = 1 << 14
        m = first_mismatch(ref(seed, 0, offset, n), oracle.philox_fill_u32(seed, offset, n))
        assert m is None, f"seed {seed:#x} offset {offset}: (index, rocRAND, oracle, count) = {m}"


@pytest.mark.parametrize("seed", SEEDS)
def test_substream_words_equal_rocrand(ref, seed):
    # the purpose tags the Philox variants use ("NORM", "BL32", "BL64") and two others
    for purpose in (0x4E4F524D, 0x424C3332, 0x424C3634, 1, 0xFFFFFFFF):
        for i in (0, 1, 12345, (1 << 32) + 7, (1 << 61) + 3):  # 4 i + 3 < 2^64
            for j in (0, 1, 2, 3, 4, 7, 8, 4099, 65535):
                got = int(ref(seed, purpose + ((j >> 2) << 32), 4 * i + (j & 3), 1)[0])
                want = int(oracle.philox_sub_word(seed, i, purpose, j))
                assert got == want, f"seed {seed:#x} purpose {purpose:#x} draw {i} word {j}: {got:#x} != {want:#x}"


@pytest.mark.gpu
def test_generator_api_equals_oracle():
    """rocRAND's host generator (every pseudo-random output ordering) gives the same words."""
    lib_path = "/opt/rocm/lib/librocrand.so"
    if not os.path.exists(lib_path):
        pytest.skip("rocRAND is not installed")
    import torch
    torch.cuda.init()  # the HIP runtime torch loaded serves rocRAND too
    lib = C.CDLL(lib_path)
    gen = C.c_void_p()
    assert lib.rocrand_create_generator_host_blocking(C.byref(gen), 404) == 0  # PHILOX4_32_10
    try:
        for ordering in (100, 101, 103):  # ROCRAND_ORDERING_PSEUDO_{BEST, DEFAULT, LEGACY}
            for seed in (1, 0x123456789ABCDEF0):
                for offset in (0, 5, (1 << 34) + 6):
                    assert lib.rocrand_set_ordering(gen, ordering) == 0
                    assert lib.rocrand_set_seed(gen, C.c_ulonglong(seed)) == 0
                    assert lib.rocrand_set_offset(gen, C.c_ulonglong(offset)) == 0
                    n = 1 << 14
                    got = np.zeros(n, dtype=np.uint32)
                    assert lib.rocrand_generate(gen, got.ctypes.data_as(C.c_void_p), C.c_size_t(n)) == 0
                    m = first_mismatch(got, oracle.philox_fill_u32(seed, offset, n))
                    assert m is None, f"ordering {ordering} seed {seed:#x} offset {offset}: {m}"
    finally:
        lib.rocrand_destroy_generator(gen)
