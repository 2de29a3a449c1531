"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Holds none of the fills' arithmetic: only sizes, keys and start draws of the workloads,
host-side weights for the choice fill, the dropout input X, and index samples for
comparisons at full size.

Workloads (tandem-cuda, "Performance", §GPU: 2^28 elements into device memory; Phobos
stdlib, "Random numbers", §dropout: X of shape [M, 256]):
  - uniform fills of 2^28 elements, keys 1..3, start draws 0, 1 and 3;
  - bounded fills of 2^28 elements: bounds 1000 and 2^32-2 (32-bit), 1000 and 2^64-2
    (64-bit), and low = -500 with bound 1000 into int32 and int64;
  - f64 normals at 2^28 and 2^24 elements, starts 0, 1, 3; f32 normals at 2^28;
  - dropout over X = f32[2^20, 256] drawn as N(0, 1) with key 7, p = 0.1, key 8;
  - choice of 2^28 uint32 indices through an alias table over 1000 Zipf(1.1) weights.
"""
import numpy as np

FULL_N = 1 << 28          # elements per fill at the measured size
SMALL_N = 1 << 20         # the 4 MiB u32 case
NORMAL_F64_SIZES = (1 << 28, 1 << 24)
KEYS = (1, 2, 3)
STARTS = (0, 1, 3)
DROPOUT_ROWS, DROPOUT_COLS = 1 << 20, 256
DROPOUT_P = 0.1
DROPOUT_X_KEY = 7
DROPOUT_KEY = 8
ZIPF_N, ZIPF_S = 1000, 1.1
BOUNDS32 = (1000, (1 << 32) - 2)
BOUNDS64 = (1000, (1 << 64) - 2)
LOW, LOW_BOUND = -500, 1000


def zipf_weights(n=ZIPF_N, s=ZIPF_S):
    """Unnormalised Zipf weights (j + 1)^-s, j < n, as float64."""
    return (np.arange(n, dtype=np.float64) + 1.0) ** -s


def normal_x(n, seed=DROPOUT_X_KEY):
    """A seeded N(0, 1) float32 array (numpy's generator), for dropout inputs."""
    return np.random.default_rng(seed).standard_normal(n, dtype=np.float32)


def sample_indices(n, m=1 << 16, seed=0, edge=1024):
    """Sorted unique element indices in [0, n): the first and last `edge`, the elements
    around every power of two, and m seeded random ones."""
    rng = np.random.default_rng(seed)
    parts = [np.arange(min(edge, n)), np.arange(max(0, n - edge), n)]
    p = 1
    while p < n:
        parts.append(np.arange(max(0, p - 2), min(n, p + 2)))
        p <<= 1
    parts.append(rng.integers(0, n, size=min(m, n)))
    return np.unique(np.concatenate(parts)).astype(np.int64)
