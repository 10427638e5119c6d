"""Pins of the oracle's binary-mask and attention-mass functions (CPU only).

Each function is checked against values fixed by hand, closed forms or brute
force, never against a retyped copy of itself.
"""
import itertools

import numpy as np

from oracle import masks


def test_mask_of_a_hand_written_list():
    # row 0: 5 causal blocks, list [3, 0, 2, 9] (9 is not causal, ignored) + pad
    # row 1: past the sequence end (n = 0): nothing survives
    order = np.array([[3, 0, 2, 9, -1], [1, 2, -1, -1, -1]])
    count = np.array([4, 2])
    m = masks.mask_from_order(order, count, np.array([5, 0]), 70)
    assert m[0].nonzero()[0].tolist() == [0, 2, 3]
    assert not m[1].any()
    w = masks.pack_words(m, 2)
    assert w[0].tolist() == [13, 0] and w[1].tolist() == [0, 0]


def test_corrupt_count_is_clamped():
    order = np.array([[4, 1, 0]])
    m = masks.mask_from_order(order, np.array([7]), np.array([6]), 6)  # count > kmax
    assert m[0].nonzero()[0].tolist() == [0, 1, 4]
    m = masks.mask_from_order(order, np.array([-2]), np.array([6]), 6)
    assert not m.any()


def test_ascending_list_of_a_hand_written_mask():
    mask = np.zeros((2, 10), dtype=bool)
    mask[0, [7, 1, 4, 9]] = True
    mask[1, [0, 8]] = True
    order, count = masks.order_from_mask(mask, np.array([8, 10]), 3)
    # row 0: block 9 is not causal (n = 8), so 1, 4, 7; row 1 fits
    assert order.tolist() == [[1, 4, 7], [0, 8, -1]]
    assert count.tolist() == [3, 2]
    order, count = masks.order_from_mask(None, np.array([5, 0]), 3)  # every causal block, truncated
    assert order.tolist() == [[0, 1, 2], [-1, -1, -1]] and count.tolist() == [3, 0]


def test_list_mask_list_round_trip_sorts():
    rng = np.random.default_rng(5)
    for _ in range(50):
        n = int(rng.integers(1, 200))
        c = int(rng.integers(1, n + 1))
        lst = rng.choice(n, c, replace=False)
        order = np.full((1, c + 3), -1)
        order[0, :c] = lst
        m = masks.mask_from_order(order, np.array([c]), np.array([n]), 256)
        back, cnt = masks.order_from_mask(m, np.array([n]), c + 3)
        assert cnt[0] == c
        assert back[0, :c].tolist() == sorted(lst.tolist())


def test_pack_unpack_bit_positions():
    m = np.zeros((1, 130), dtype=bool)
    m[0, [0, 63, 64, 129]] = True
    w = masks.pack_words(m, 3)
    assert w[0].tolist() == [1 | (1 << 63), 1, 2]
    assert np.array_equal(masks.unpack_words(w, 130), m)


def _rows(Lq, B):
    return [min(B, Lq - qb * B) for qb in range(-(-Lq // B))]


def test_block_mass_rows_sum_to_row_count():
    rng = np.random.default_rng(1)
    Lq, Lk, B, G = 150, 300, 32, 2
    q = rng.standard_normal((Lq, 4, 16))
    k = rng.standard_normal((Lk, 2, 16))
    M = masks.block_mass_sequence(q, k, 0.3, G, B)
    np.testing.assert_allclose(M.sum(axis=2), np.array([_rows(Lq, B)] * 4), rtol=0, atol=1e-12)


def test_block_mass_closed_form_for_equal_scores():
    # q = 0: every visible key of row i has probability 1 / (pos_i + 1), so the
    # mass of block kb is sum_i |keys of kb visible to i| / (pos_i + 1)
    Lq, Lk, B = 70, 100, 16
    q = np.zeros((Lq, 1, 8))
    k = np.random.default_rng(2).standard_normal((Lk, 1, 8))
    M = masks.block_mass_sequence(q, k, 1.0, 1, B)
    off = Lk - Lq
    for qb in range(M.shape[1]):
        for kb in range(M.shape[2]):
            want = 0.0
            for i in range(qb * B, min(qb * B + B, Lq)):
                pos = off + i
                seen = min(max(pos - kb * B + 1, 0), min(B, Lk - kb * B))
                want += seen / (pos + 1)
            assert abs(M[0, qb, kb] - want) < 1e-12, (qb, kb)


def test_block_mass_of_a_dominant_key():
    # key 5 scores 60 nats above every other key for every row that sees it
    Lq = Lk = 64
    B = 16
    q = np.zeros((Lq, 1, 2))
    q[:, 0, 0] = 1.0
    k = np.zeros((Lk, 1, 2))
    k[5, 0, 0] = 60.0
    M = masks.block_mass_sequence(q, k, 1.0, 1, B)
    # rows 0..4 do not see key 5: their mass spreads over the keys they see
    assert abs(M[0, 0, 0] - 16.0) < 1e-12  # block 0 holds all keys of rows 0..15
    for qb in range(1, 4):
        # every other key carries at most e^-60 of a row: 16 rows x 64 keys of it
        assert abs(M[0, qb, 0] - 16.0) < 1e-12
        assert M[0, qb, 1:].sum() < 1e-20


def test_recall_and_oracle_selection_by_brute_force():
    rng = np.random.default_rng(3)
    M = rng.random((4, 6))
    M[3] = 0.0  # a row with no mass
    k = np.array([2, 3, 1, 2])
    best = masks.oracle_recall(M, k)
    for r in range(3):
        tot = M[r].sum()
        brute = max(M[r, list(s)].sum() / tot for s in itertools.combinations(range(6), int(k[r])))
        assert abs(best[r] - brute) < 1e-15
        for s in itertools.combinations(range(6), int(k[r])):
            order = np.array([list(s) + [-1] * (6 - len(s))])
            got = masks.recall(M[r : r + 1], order, np.array([len(s)]))[0]
            assert got <= best[r] + 1e-15
    assert np.isnan(best[3])
    full = masks.recall(M[:1], np.array([[5, 4, 3, 2, 1, 0]]), np.array([6]))
    assert abs(full[0] - 1.0) < 1e-15


def test_union_lists_by_hand():
    # one sequence, one KV group, three query blocks with 2, 4 and 5 causal blocks
    order = np.array([[[[1, 0, -1], [3, 0, -1], [4, 9, 2]]]])  # 9 is not causal for qb 2: ignored
    count = np.array([[[2, 2, 3]]])
    n = np.array([[[2, 4, 5]]])
    out, cnt = masks.union_lists(order, count, n, 5)
    # union {0, 1, 2, 3, 4}, cut causally per query block
    assert out[0, 0].tolist() == [[0, 1, -1, -1, -1], [0, 1, 2, 3, -1], [0, 1, 2, 3, 4]]
    assert cnt[0, 0].tolist() == [2, 4, 5]
    out, cnt = masks.union_lists(order, count, n, 3)  # truncation keeps the lowest blocks
    assert out[0, 0, 2].tolist() == [0, 1, 2] and cnt[0, 0].tolist() == [2, 3, 3]


def test_union_lists_cover_and_stay_minimal():
    rng = np.random.default_rng(11)
    nb, hkv, nq, kmax = 2, 3, 6, 4
    n = np.tile(np.arange(3, 3 + nq), (nb, hkv, 1))
    order = np.full((nb, hkv, nq, kmax), -1)
    count = np.minimum(rng.integers(1, kmax + 1, size=(nb, hkv, nq)), n)
    for idx in np.ndindex(nb, hkv, nq):
        order[idx][: count[idx]] = rng.choice(n[idx], count[idx], replace=False)
    out, cnt = masks.union_lists(order, count, n, 16)
    for b in range(nb):
        for g in range(hkv):
            listed = {int(x) for qb in range(nq) for x in order[b, g, qb, : count[b, g, qb]]}
            for qb in range(nq):
                got = out[b, g, qb, : cnt[b, g, qb]].tolist()
                assert got == sorted(got) and all(kb < n[b, g, qb] for kb in got)
                # coverage: what this row listed survives; minimality: nothing unlisted appears
                assert set(order[b, g, qb, : count[b, g, qb]].tolist()) <= set(got)
                assert set(got) <= listed
                assert set(got) == {kb for kb in listed if kb < n[b, g, qb]}
