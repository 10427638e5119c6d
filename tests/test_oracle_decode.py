"""Pins of the oracle's split decode walk (CPU only): the textbook softmax over
the listed keys when skipping is off, agreement with the prefill walk's own
oracle for one segment, a hand-built case where splitting changes the skip
count, and the segment bounds."""
import math

import numpy as np

from oracle import decode as od, osk as oosk


def _inputs(seed, Lk, Hq=4, Hkv=2, d=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, d))
    k = rng.standard_normal((Lk, Hkv, d))
    v = rng.standard_normal((Lk, Hkv, d))
    return q, k, v


def test_segment_bounds():
    assert od.segment_bounds(10, 3) == [(0, 3), (3, 6), (6, 10)]
    assert od.segment_bounds(2, 4) == [(0, 0), (0, 1), (1, 1), (1, 2)]
    assert od.segment_bounds(0, 2) == [(0, 0), (0, 0)]


def test_no_skip_is_softmax_over_listed_keys():
    B, Lk, G = 8, 75, 2
    q, k, v = _inputs(1, Lk)
    order = np.array([[9, 0, 4, 2, -1, -1], [3, 1, 8, 5, 0, 7]])  # block 9 is the partial last block
    count = np.array([4, 6])
    scale = 0.3
    for S in (1, 2, 3, 7):
        out = od.decode_sequence(q, k, v, order, count, scale, 0.0, G, B, S)
        for h in range(4):
            g = h // G
            keys = np.concatenate([np.arange(kb * B, min(kb * B + B, Lk)) for kb in order[g, : count[g]]])
            s = scale * (k[keys, g] @ q[0, h])
            p = np.exp(s - s.max())
            want = (p / p.sum()) @ v[keys, g]
            np.testing.assert_allclose(out["O"][h], want, rtol=1e-12, atol=1e-12)
            assert abs(out["lse"][h] - (s.max() + math.log(p.sum()))) < 1e-12
            assert out["visited"][h] == count[g] and out["skipped"][h] == 0


def test_one_segment_equals_the_prefill_walk():
    B, Lk, G = 8, 64, 2
    q, k, v = _inputs(2, Lk)
    k[3, :, :] *= 12.0  # a dominant key so that later blocks get skipped
    order = np.array([[0, 5, 2, 7, 1], [0, 3, 6, 4, 2]])
    count = np.array([5, 4])
    tau = math.exp(-4.0)
    out = od.decode_sequence(q, k, v, order, count, 0.5, tau, G, B, 1)
    ref = oosk.osk_sequence(q, k, v, order[:, None, :], count[:, None], 0.5, tau, G, B)
    np.testing.assert_allclose(out["O"], ref["O"][0], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(out["visited"], ref["visited"][:, 0])
    np.testing.assert_array_equal(out["skipped"], ref["skipped"][:, 0])
    assert out["skipped"].sum() > 0


def test_splitting_changes_the_skip_count_by_hand():
    # one head, B = 2: block 0 holds a key scoring 30, block 1 keys scoring 0;
    # with one segment block 1 sits 30 nats below the running max (skipped at
    # tau = e^-16); as the first block of a second segment it is computed
    d = 2
    q = np.array([[[1.0, 0.0]]])
    k = np.zeros((4, 1, d))
    k[1, 0, 0] = 30.0
    v = np.arange(8.0).reshape(4, 1, 2)
    order = np.array([[0, 1]])
    count = np.array([2])
    tau = math.exp(-16.0)
    one = od.decode_sequence(q, k, v, order, count, 1.0, tau, 1, 2, 1)
    two = od.decode_sequence(q, k, v, order, count, 1.0, tau, 1, 2, 2)
    assert (one["visited"][0], one["skipped"][0]) == (2, 1)
    assert (two["visited"][0], two["skipped"][0]) == (2, 0)
    # one segment: only block 0 counts: weights e^0 (key 0) and e^30 (key 1)
    w = np.array([math.exp(-30.0), 1.0])
    np.testing.assert_allclose(one["O"][0], (w / w.sum()) @ v[:2, 0], rtol=1e-14)
    # two segments: every key counts
    w = np.array([math.exp(-30.0), 1.0, math.exp(-30.0), math.exp(-30.0)])
    np.testing.assert_allclose(two["O"][0], (w / w.sum()) @ v[:, 0], rtol=1e-14)
