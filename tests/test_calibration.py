"""Pins for the calibration helpers of the benchmark's confidence-calibration
leg (freeaitool DSpark guide, section 4.1: per-position temperature scaling
from left to right against the empirical acceptance rate, reported as expected
calibration error): closed-form ECE cases and recovery of known over- and
under-confidence temperatures from Bernoulli labels."""
import numpy as np

import bench


def test_ece_closed_forms():
    # one bin, confidence 0.8, labels averaging 0.6 -> 0.2
    c = np.full(1000, 0.8)
    y = np.zeros(1000)
    y[:600] = 1
    assert abs(bench.ece(c, y) - 0.2) < 1e-12
    # two bins, each matching its label mean -> 0
    c = np.r_[np.full(100, 0.25), np.full(300, 0.75)]
    y = np.r_[np.r_[np.ones(25), np.zeros(75)], np.r_[np.ones(225), np.zeros(75)]]
    assert bench.ece(c, y) < 1e-12
    assert bench.ece([], []) == 0.0


def test_sts_recovers_known_temperatures():
    rng = np.random.default_rng(3)
    n, scales = 40000, np.array([1.5, 2.0, 3.0, 0.7])
    p = rng.uniform(0.05, 0.95, (n, 4))
    y = (rng.random((n, 4)) < p).astype(np.float64)
    lg = np.log(p) - np.log1p(-p)
    c_raw = 1.0 / (1.0 + np.exp(-scales[None, :] * lg))
    reached = np.ones((n, 4), bool)
    reached[: n // 2, 3] = False  # position 4 sees only half the samples
    taus = np.array(bench.sts_fit(c_raw, y, reached))
    np.testing.assert_allclose(taus, scales, rtol=0.1)
    cc = bench.sts_apply(c_raw, taus)
    for k in range(4):
        m = reached[:, k]
        raw, cal = bench.ece(c_raw[m, k], y[m, k]), bench.ece(cc[m, k], y[m, k])
        assert cal < 0.02
        assert cal < raw


def test_sparse_positions_inherit_the_previous_temperature():
    rng = np.random.default_rng(5)
    n = 5000
    p = rng.uniform(0.05, 0.95, (n, 3))
    y = (rng.random((n, 3)) < p).astype(np.float64)
    lg = np.log(p) - np.log1p(-p)
    c_raw = 1.0 / (1.0 + np.exp(-2.0 * lg))
    reached = np.ones((n, 3), bool)
    reached[10:, 1] = False  # position 2: 10 samples only
    reached[:, 2] = False    # position 3: none
    taus = bench.sts_fit(c_raw, y, reached)
    assert abs(taus[0] - 2.0) < 0.3
    assert taus[1] == taus[0] and taus[2] == taus[0]
