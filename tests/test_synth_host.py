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


def test_normal_quantile_matches_an_independent_implementation():
    """The generator's normal quantile (Acklam's rational approximation, with
    its own log and square root) against scipy's ndtri (Cephes), over the
    centre, both tails and the extreme p the 52-bit uniform reaches: within
    the published 1.15e-9 relative error; odd about p = 1/2."""
    from scipy.special import ndtri
    p = np.concatenate([(np.arange(1 << 20) + 0.5) / (1 << 20),
                        (np.arange(1, 1 << 14) + 0.5) * 2.0 ** -52,
                        1 - (np.arange(1, 1 << 14) + 0.5) * 2.0 ** -52,
                        np.logspace(-16, np.log10(0.4999), 20000)])
    z, ref = gen.normal_quantile(p), ndtri(p)
    assert (np.abs(z - ref) <= 1.15e-9 * np.abs(ref) + 1e-300).all()
    assert gen.normal_quantile([0.5])[0] == 0.0
    q = np.linspace(0.001, 0.499, 997)
    np.testing.assert_allclose(gen.normal_quantile(q), -gen.normal_quantile(1 - q), rtol=2e-9)


def test_distribution_is_normal_and_modes_agree():
    from scipy import stats
    x = gen.host_fill(2, W.KIND_MASTER, 0, 0, 1 << 22, 0.02, gen.MODE_F32).astype(np.float64)
    assert abs(x.mean()) < 1e-4 and abs(x.std() / 0.02 - 1) < 2e-3
    k = ((x - x.mean()) ** 4).mean() / x.var() ** 2
    assert abs(k - 3) < 0.02                      # the normal's kurtosis
    assert stats.kstest(x[:1 << 20] / 0.02, "norm").pvalue > 1e-3
    assert np.abs(x).max() > 5 * 0.02             # tails past the old +-4.24 sigma support
    a = gen.host_fill(2, W.KIND_MASTER, 0, 0, 1000, 0.02, gen.MODE_ABS)
    assert np.array_equal(a, np.abs(x[:1000].astype(np.float32)))
    b = gen.host_fill(2, W.KIND_MASTER, 0, 0, 1000, 0.02, gen.MODE_BF16)
    u = x[:1000].astype(np.float32).view(np.uint32).astype(np.uint64)
    assert np.array_equal(b, ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16))
    # the value is fp32 of the quantile at p = (k + 1/2) 2^-52, times the fp32 std
    c = [gen.philox4x32_10([e, 0, 0, 0], [2026, gen.key1(2, W.KIND_MASTER, 0)]) for e in range(64)]
    p = np.array([((((w[1] << 32) | w[0]) >> 12) + 0.5) * 2.0 ** -52 for w in c])
    want = gen.normal_quantile(p).astype(np.float32) * np.float32(0.02)
    assert np.array_equal(want.view(np.uint32), x[:64].astype(np.float32).view(np.uint32))
