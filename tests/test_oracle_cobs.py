"""Pins of the oracle's second-order block scores (CPU only): hand-computed
values, causality, and the cumulant expansion the score truncates."""
import math

import numpy as np

from oracle import cobs


def test_equal_keys_have_no_second_order_term():
    # one pooled row (p = 1), one block of 4 identical keys: variance 0
    q = np.array([[[1.0, 2.0]]])
    k = np.tile(np.array([[[0.5, -1.0]]]), (4, 1, 1))
    P2 = cobs.cobs_scores(q, k, 0.5, 4, 1, 1, 4)
    assert P2.shape == (1, 1, 1)
    assert abs(P2[0, 0, 0] - 0.5 * (0.5 - 2.0)) < 1e-15


def test_two_keys_by_hand():
    # scores a = 3 and b = -1 (scale 1): mean 1, variance 4 -> 1 + 2 = 3
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[3.0, 7.0]], [[-1.0, 2.0]]])
    P2 = cobs.cobs_scores(q, k, 1.0, 2, 1, 1, 2)
    assert abs(P2[0, 0, 0] - 3.0) < 1e-15


def test_causality_uses_only_visible_keys():
    # Lq = Lk = 4, B = 2, p = 2: pooled row 0 (tokens 0, 1) sees keys 0, 1;
    # pooled row 1 sees all four. Key scores (scale 1): 1, 3, 10, 20.
    k = np.array([1.0, 3.0, 10.0, 20.0]).reshape(4, 1, 1)
    qt = np.ones((2, 1, 1))
    P2 = cobs.cobs_scores(qt, k, 1.0, 2, 2, 4, 4)
    assert abs(P2[0, 0, 0] - (2.0 + 0.5 * 1.0)) < 1e-15   # keys 1, 3
    assert P2[0, 0, 1] == -np.inf                         # block 1 unseen by row 0
    assert abs(P2[0, 1, 1] - (15.0 + 0.5 * 25.0)) < 1e-15  # keys 10, 20
    # chunked offset: Lq = 2 queries at positions 2, 3 of Lk = 4; p = 1, B = 2
    P2 = cobs.cobs_scores(np.ones((2, 1, 1)), k, 1.0, 2, 1, 2, 4)
    assert abs(P2[0, 0, 1] - 10.0) < 1e-15                # row 0 sees key 2 only in block 1
    assert abs(P2[0, 1, 1] - 27.5) < 1e-15


def test_second_order_truncation_of_the_log_mass():
    # scores mu +- delta in equal numbers: ln(mean e^s) = mu + ln cosh(delta)
    # = mu + delta^2/2 - delta^4/12 + ..., so P2 = mu + delta^2/2 is off by
    # at most delta^4/12
    for mu, delta in [(0.3, 0.1), (-2.0, 0.25), (5.0, 0.5)]:
        k = np.array([mu + delta, mu - delta] * 8).reshape(16, 1, 1)
        P2 = cobs.cobs_scores(np.ones((1, 1, 1)), k, 1.0, 16, 1, 1, 16)[0, 0, 0]
        exact = mu + math.log(math.cosh(delta))
        assert abs(P2 - (mu + delta ** 2 / 2)) < 1e-12
        assert abs(P2 - exact) <= delta ** 4 / 12 + 1e-12
