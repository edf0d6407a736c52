"""The statistics the GPU parity tests use, on synthetic logits (CPU only)."""
import numpy as np
import pytest
import scipy.stats

import parity_stats as ps


def test_poisson_binomial_quantile_equal_probabilities_is_binomial():
    for n, p in [(1, 0.3), (40, 0.05), (300, 0.01), (1000, 0.2)]:
        for q in (0.5, 0.9, 0.999):
            assert ps.poisson_binomial_quantile([p] * n, q) == int(scipy.stats.binom.ppf(q, n, p))


def test_poisson_binomial_quantile_mixed_probabilities_brute_force():
    rng = np.random.default_rng(3)
    p = rng.uniform(0, 0.6, size=10)
    # enumerate all 2^10 outcomes
    probs = np.zeros(11)
    for mask in range(1 << 10):
        bits = np.array([(mask >> i) & 1 for i in range(10)], dtype=bool)
        probs[bits.sum()] += np.prod(np.where(bits, p, 1 - p))
    cdf = np.cumsum(probs)
    for q in (0.1, 0.5, 0.9, 0.999):
        assert ps.poisson_binomial_quantile(p, q) == int(np.argmax(cdf >= q - 1e-12))
    assert ps.poisson_binomial_quantile([], 0.999) == 0
    assert ps.poisson_binomial_quantile([1.0, 1.0, 0.0], 0.5) == 2


def test_distance_statistics():
    a = np.zeros((3, 2000))
    b = np.zeros((3, 2000))
    b[0, :] = 0.5                  # rms 0.5
    b[1, :3] = 4.0                 # three spikes: p99.9 over 2000 values is the 3rd largest
    b[2, 0] = -1.0
    a += 1.0                       # cosine of a with b
    d = ps.distance(b, a)
    np.testing.assert_allclose(d.rms[0], 0.5)
    assert d.p999[1] == 3.0 and d.max[1] == 3.0
    assert d.p999[2] == 1.0 and d.max[2] == 2.0   # one spike is above the 99.9th percentile
    assert d.max_all == 3.0
    np.testing.assert_allclose(d.rms_all, np.sqrt(np.mean((b - a) ** 2)))
    assert d.cos[0] == pytest.approx(1.0)
    # pooled p99.9 over 6000 values: the 6th largest |d|
    flat = np.sort(np.abs(b - a).ravel())
    assert d.p999_all == flat[int(np.ceil(0.999 * flat.size)) - 1]


def test_normal_tail():
    x = np.array([0.0, 1.0, 2.5])
    np.testing.assert_allclose(ps.normal_tail(x), scipy.stats.norm.sf(x), rtol=1e-12)


def _noisy(rng, base, sigma):
    return base + rng.normal(0.0, sigma, size=base.shape)


def test_check_depth_regimes():
    rng = np.random.default_rng(5)
    plain = rng.normal(0.0, 1.3, size=(40, 4000))
    ref = _noisy(rng, plain, 0.05)
    alt = _noisy(rng, ref, 0.03)
    quiet = lambda *a, **k: None  # noqa: E731
    # a GPU result as noisy as a second correct evaluation passes (floor regime: alt's max > 3e-2)
    ps.check_depth(_noisy(rng, ref, 0.03), ref, alt, plain, 0.2, say=quiet)
    # a result 1.5x noisier fails
    with pytest.raises(AssertionError, match="pooled rms"):
        ps.check_depth(_noisy(rng, ref, 0.045), ref, alt, plain, 0.2, say=quiet)
    # one position far off fails on the worst position even if the pooled statistics pass
    g = _noisy(rng, ref, 0.03)
    g[7] = _noisy(rng, ref[7], 0.06)
    with pytest.raises(AssertionError, match="worst-position rms"):
        ps.check_depth(g, ref, alt, plain, 0.2, say=quiet)
    # stated regime: when a correct evaluation stays within 3e-2, so must the GPU
    alt_s = _noisy(rng, ref, 1e-3)
    ps.check_depth(_noisy(rng, ref, 2e-3), ref, alt_s, None, 0.2, say=quiet)
    with pytest.raises(AssertionError, match="stated"):
        ps.check_depth(_noisy(rng, ref, 8e-3), ref, alt_s, None, 0.2, say=quiet)


def test_greedy_check_forced_band_and_own_argmax():
    rng = np.random.default_rng(9)
    n, V = 400, 50
    ref = rng.normal(0.0, 1.0, size=(n, V))
    alt = _noisy(rng, ref, 0.02)
    gpu = _noisy(rng, ref, 0.02)
    tok = np.argmax(gpu, -1)
    rep = ps.greedy_check(tok, gpu, ref, alt, forced_margin=0.2)
    assert rep.checked == n and rep.band_mismatch <= rep.band_limit
    # a token that is not the argmax of the GPU's own logits
    bad = tok.copy()
    bad[3] = (bad[3] + 1) % V
    with pytest.raises(AssertionError, match="own logits"):
        ps.greedy_check(bad, gpu, ref, alt, forced_margin=0.2)
    # a flipped pick at a forced position (large margin)
    top, margin = ps.top2(ref)
    j = int(np.argmax(margin))
    g2 = gpu.copy()
    g2[j, top[j]] -= 10.0
    with pytest.raises(AssertionError, match="forced"):
        ps.greedy_check(np.argmax(g2, -1), g2, ref, alt, forced_margin=0.2)
    # many flips in the band, far more than the noise explains
    g3 = _noisy(rng, ref, 0.02)
    band = np.nonzero((margin > 0.1) & (margin <= 0.2))[0]
    assert band.size > 10
    second = np.argsort(ref, -1)[:, -2]
    for i in band:
        g3[i, second[i]] = ref[i, top[i]] + 0.5
    with pytest.raises(AssertionError, match="mismatches"):
        ps.greedy_check(np.argmax(g3, -1), g3, ref, alt, forced_margin=0.2)
