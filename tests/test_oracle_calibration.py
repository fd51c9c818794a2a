"""Pins of the calibrated- and static-scheduling oracle.

CPU only.  Sources: "UraionSpec", section "Sequential Temperature Scaling"
(c~ = c^(1/T), the left-to-right grid fit on the cumulative survival's ECE,
the static scheduler's fixed-length and threshold modes); "breaking down
dspark and its lineage", "Verify smarter, not longer" (threshold 0 is fixed
length).  A fit that ignores earlier positions, a wrong label index, an
inverted power or a threshold compared the wrong way fails at least one.
"""

import numpy as np
import pytest

from oracle import calibration as C
import workloads as W


def test_power_special_cases_and_order():
    c = np.array([0.0, 1.0, 0.25, 0.5, 0.9], np.float32)
    col = C.sts_apply(c[:, None], [2.0])[:, 0]
    assert col[0] == 0.0 and col[1] == 1.0 and col[2] == np.float32(0.5)
    g = np.random.default_rng(1).uniform(0, 1, (200, 3)).astype(np.float32)
    # T = 1 is the identity, bit for bit on float32 inputs
    np.testing.assert_array_equal(C.sts_apply(g, [1.0, 1.0, 1.0]), g)
    # T = 1/2 squares, T = 2 takes the square root (to float32 rounding)
    np.testing.assert_allclose(C.sts_apply(g, [0.5, 2.0, 0.25])[:, 0], g[:, 0].astype(np.float64) ** 2, rtol=2e-7)
    np.testing.assert_allclose(C.sts_apply(g, [0.5, 2.0, 0.25])[:, 1], np.sqrt(g[:, 1].astype(np.float64)), rtol=2e-7)
    # order preserving along a column
    s = np.sort(g[:, 2])
    assert np.all(np.diff(C.sts_apply(np.stack([s, s, s], 1), [3.0, 0.3, 1.7])[:, 0]) >= 0)


def test_grid_is_linear_with_one_on_it():
    t = C.grid()
    assert len(t) == 100 and t[0] == 0.1 and t[-1] == 10.0
    assert np.any(np.abs(t - 1.0) < 1e-12)


def test_ece_closed_forms():
    # all predictions 0.5, half the labels 1: perfectly calibrated
    assert C.ece(np.full(10, 0.5), np.r_[np.ones(5), np.zeros(5)]) == 0.0
    # predictions 0.9, labels 0: gap 0.9
    assert abs(C.ece(np.full(4, 0.9), np.zeros(4)) - 0.9) < 1e-15
    # two bins: {0.1, 0.1} labels {1, 0} -> |0.2 - 1| ; {0.8} label {1} -> |0.8 - 1|; / 3
    assert abs(C.ece([0.1, 0.1, 0.8], [1, 0, 1]) - (0.8 + 0.2) / 3) < 1e-15
    # 1.0 falls in the last bin, 0.0 in the first
    assert abs(C.ece([1.0, 0.0], [1, 0])) == 0.0


def test_fit_recovers_known_temperatures():
    conf, L, T = W.calibration(60000, G=6)
    fitted, table = C.sts_fit(conf, L, return_ece=True)
    assert np.all(np.abs(fitted - T) <= 0.25), (fitted, T)
    # the fitted point is the first minimum of each position's ECE row
    for k in range(6):
        assert fitted[k] == np.float64(np.float32(C.grid()[int(np.argmin(table[k]))]))
    # calibration never worsens a position against T = 1 given the same prefix
    one = int(np.argmin(np.abs(C.grid() - 1.0)))        # float32(1.0) is exact
    assert np.all(table[np.arange(6), [int(np.argmin(r)) for r in table]] <= table[:, one] + 1e-15)


def test_fit_on_calibrated_data_stays_near_one():
    conf, L, _ = W.calibration(60000, G=4, true_temps=[1.0, 1.0, 1.0, 1.0])
    fitted = C.sts_fit(conf, L)
    assert np.all(np.abs(fitted - 1.0) <= 0.2), fitted


def test_fit_is_sequential():
    """Position k's fit uses the calibrated earlier positions, not the raw ones."""
    conf, L, T = W.calibration(60000, G=3, true_temps=[0.5, 1.0, 1.0])
    fitted = C.sts_fit(conf, L)
    # with the first position corrected, the later ones need no correction
    assert abs(fitted[0] - 0.5) <= 0.1 and np.all(np.abs(fitted[1:] - 1.0) <= 0.2), fitted


def test_static_modes():
    assert C.static_fixed(4, 15, 7).tolist() == [7] * 4
    assert C.static_fixed(3, 5, 9).tolist() == [5] * 3 and C.static_fixed(2, 5, -1).tolist() == [0, 0]
    c = np.array([[0.9, 0.8, 0.3, 0.9], [0.2, 0.9, 0.9, 0.9], [0.95, 0.95, 0.95, 0.95]], np.float32)
    assert C.static_threshold(c, 0.5).tolist() == [2, 0, 4]
    assert C.static_threshold(c, 0.0).tolist() == [4, 4, 4]          # threshold 0: fixed full length
    assert C.static_threshold(c, 0.95).tolist() == [0, 0, 0]         # strictly above
    assert C.static_threshold(c, 1.0).tolist() == [0, 0, 0]
