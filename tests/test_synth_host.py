"""Host side of the input generator: published known-answer vectors and the
shape of the value distribution."""
import os

import numpy as np

from synth import gen, workloads as W

KAT = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers():
    n = 0
    for line in open(KAT):
        if line.startswith("#") or not line.strip():
            continue
        v = [int(x, 16) for x in line.split()]
        assert gen.philox4x32_10(v[0:4], v[4:6]) == v[6:10]
        n += 1
    assert n == 3


def test_values_are_deterministic_and_keyed():
    a = gen.host_fill(1, W.KIND_GRAD, 3, 10, 1000, 1e-3, gen.MODE_F32)
    b = gen.host_fill(1, W.KIND_GRAD, 3, 0, 1010, 1e-3, gen.MODE_F32)
    assert np.array_equal(a, b[10:])
    c = gen.host_fill(1, W.KIND_GRAD, 4, 10, 1000, 1e-3, gen.MODE_F32)
    assert not np.array_equal(a, c)
    idx = np.array([10, 500, 1009], np.int64)
    assert np.array_equal(gen.host_fill_idx(1, W.KIND_GRAD, 3, idx, 1e-3, gen.MODE_F32), b[idx])


def test_distribution_moments_and_modes():
    x = gen.host_fill(2, W.KIND_MASTER, 0, 0, 1 << 22, 0.02, gen.MODE_F32).astype(np.float64)
    assert abs(x.mean()) < 1e-4 and abs(x.std() / 0.02 - 1) < 2e-3
    k = ((x - x.mean()) ** 4).mean() / x.var() ** 2
    assert abs(k - (3 - 1.2 / 8)) < 0.01          # Irwin-Hall of 8 terms
    a = gen.host_fill(2, W.KIND_MASTER, 0, 0, 1000, 0.02, gen.MODE_ABS)
    assert np.array_equal(a, np.abs(x[:1000].astype(np.float32)))
    b = gen.host_fill(2, W.KIND_MASTER, 0, 0, 1000, 0.02, gen.MODE_BF16)
    u = x[:1000].astype(np.float32).view(np.uint32).astype(np.uint64)
    assert np.array_equal(b, ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16))
