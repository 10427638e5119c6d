"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test ties the oracle to something other than its own code: a library
routine (torch SDPA), a closed form, a hand-worked example under
``tests/golden/`` (derivations inside the files), brute force on tiny inputs,
or an invariant the CoSA summary states (order invariance §2.1, unselected
blocks never touched §2.3, per-tile skip veto and running-max lower bound §1).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import cases, dense, exp32 as ex, kap, layout, osk
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- exp32 ----

def test_exp32_special_values():
    assert ex.exp32(np.float32(0.0)) == np.float32(1.0)
    for x in [-87.0001, -88.0, -1e30, -np.inf, np.nan]:
        assert ex.exp32(np.float32(x)) == 0.0
    assert ex.exp32(np.float32(-87.0)) > 0.0


def test_exp32_constants_are_the_spec_bits():
    # fp32(log2 e) and fp32(ln2^k / k!), k = 0..7, as IEEE bit patterns.
    want = [0x3F800000, 0x3F317218, 0x3E75FDF0, 0x3D635847,
            0x3C1D955B, 0x3AAEC3FF, 0x39218489, 0x377FE5FE]
    got = [int(np.float32(c).view(np.uint32)) for c in ex.COEFFS]
    assert got == want
    assert int(ex.LOG2E.view(np.uint32)) == 0x3FB8AA3B


def test_exp32_accuracy_and_monotone():
    x = np.linspace(-87.0, 0.0, 2_000_001, dtype=np.float32)
    y = ex.exp32(x)
    ref = np.exp(x.astype(np.float64))
    rel = np.abs(y.astype(np.float64) - ref) / ref
    assert rel.max() < 4e-6
    assert np.all(np.diff(y.astype(np.float64)) >= 0.0)
    # normal results only
    assert y.min() >= np.finfo(np.float32).tiny


# ---------------------------------------------------------------- dense ----

def _sdpa_reference(q, k, v, scale):
    """torch SDPA in fp64 on the CPU with an explicit causal mask (GQA expanded)."""
    Lq, Hq, d = q.shape
    Lk, Hkv, _ = k.shape
    G = Hq // Hkv
    off = Lk - Lq
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1).permute(1, 0, 2)[None].contiguous()
    mask = torch.arange(Lk)[None, :] <= (torch.arange(Lq)[:, None] + off)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_dense_matches_torch_sdpa_chunked_gqa():
    rng = np.random.default_rng(0)
    Lq, Lk, Hq, Hkv, d = 300, 437, 4, 2, 16
    q = rng.standard_normal((Lq, Hq, d))
    k = rng.standard_normal((Lk, Hkv, d))
    v = rng.standard_normal((Lk, Hkv, d))
    o, lse = dense.dense_sequence(q, k, v, 0.25, row_chunk=77)
    ref = _sdpa_reference(q, k, v, 0.25)
    assert np.abs(o - ref).max() < 1e-12
    # lse by its definition for one row
    i, h = 123, 3
    s = 0.25 * (k[: i + (Lk - Lq) + 1, h // 2] @ q[i, h])
    assert abs(lse[h, i] - math.log(np.exp(s).sum())) < 1e-12


def test_dense_bruteforce_tiny():
    rng = np.random.default_rng(1)
    Lq, Lk, d = 5, 7, 3
    q = rng.standard_normal((Lq, 1, d))
    k = rng.standard_normal((Lk, 1, d))
    v = rng.standard_normal((Lk, 1, d))
    o, _ = dense.dense_sequence(q, k, v, 0.7)
    for i in range(Lq):
        w = [math.exp(0.7 * sum(q[i, 0, t] * k[j, 0, t] for t in range(d))) for j in range(i + 2 + 1)]
        z = sum(w)
        for c in range(d):
            want = sum(w[j] * v[j, 0, c] for j in range(len(w))) / z
            assert abs(o[i, 0, c] - want) < 1e-12


# ---------------------------------------------------------------- OSK ------

def _small_case(seed=7, lq=700, lk=None, hq=4, hkv=2, d=32, B=64, p=8, budget=0.3, dtype="f32"):
    return synthetic.lowrank_case(seed, [lq], None if lk is None else [lk], h_q=hq, h_kv=hkv,
                                  head_dim=d, block=B, pool=p, budget=budget, dtype=dtype)


def _all_blocks_order(case, rng=None):
    """Every causal block of every row, ascending or randomly permuted."""
    B = case.block
    Lq, Lk = case.seqlens_q[0], int(case.seqlens_k[0])
    nq = layout.cdiv(Lq, B)
    nmax = layout.n_causal_blocks(nq - 1, B, Lq, Lk)
    order = np.full((1, case.h_kv, nq, nmax), -1, dtype=np.int32)
    count = np.zeros((1, case.h_kv, nq), dtype=np.int32)
    for g in range(case.h_kv):
        for qb in range(nq):
            n = layout.n_causal_blocks(qb, B, Lq, Lk)
            lst = np.arange(n)
            if rng is not None:
                lst = rng.permutation(n)
            order[0, g, qb, :n] = lst
            count[0, g, qb] = n
    return order, count


def test_osk_full_budget_no_skip_equals_dense():
    case = _small_case(lk=900)
    ref = cases.dense_case(case)["O"]
    order, count = _all_blocks_order(case, np.random.default_rng(3))
    out = cases.osk_case(case, order, count, tau=0.0)
    assert np.abs(out["O"] - ref).max() < 1e-12
    assert np.abs(out["lse"] - cases.dense_case(case)["lse"]).max() < 1e-12
    assert out["skipped"].sum() == 0
    # the proxy at budget 1 lists every causal block, in its own order
    ko = cases.kap_case(case, budget=1.0)
    out2 = cases.osk_case(case, ko["order"], ko["count"], tau=0.0)
    assert np.abs(out2["O"] - ref).max() < 1e-12


def test_osk_order_invariance():
    case = _small_case(seed=8, budget=0.4)
    ko = cases.kap_case(case)
    a = cases.osk_case(case, ko["order"], ko["count"], tau=0.0)["O"]
    rng = np.random.default_rng(5)
    perm = ko["order"].copy()
    for g in range(case.h_kv):
        for qb in range(perm.shape[2]):
            c = ko["count"][0, g, qb]
            perm[0, g, qb, :c] = rng.permutation(perm[0, g, qb, :c])
    b = cases.osk_case(case, perm, ko["count"], tau=0.0)["O"]
    assert np.abs(a - b).max() < 1e-12


def test_osk_equals_block_masked_softmax():
    """Unselected blocks are never touched: O equals dense softmax with the
    unlisted blocks' scores set to -inf (computed here from the full matrix)."""
    case = _small_case(seed=9, lq=500, lk=777, budget=0.25)
    ko = cases.kap_case(case)
    out = cases.osk_case(case, ko["order"], ko["count"], tau=0.0)
    q, k, v = cases.sequence_inputs(case, 0)
    Lq, Lk, B, G = q.shape[0], k.shape[0], case.block, case.h_q // case.h_kv
    off = Lk - Lq
    for h in range(case.h_q):
        g = h // G
        s = case.scale * q[:, h] @ k[:, g].T
        allowed = np.zeros((Lq, Lk), dtype=bool)
        for qb in range(layout.cdiv(Lq, B)):
            for kb in ko["order"][0, g, qb, : ko["count"][0, g, qb]]:
                allowed[qb * B : qb * B + B, kb * B : kb * B + B] = True
        allowed &= np.arange(Lk)[None, :] <= (np.arange(Lq)[:, None] + off)
        s = np.where(allowed, s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        want = (w @ v[:, g]) / w.sum(axis=1, keepdims=True)
        assert np.abs(out["O"][:, h] - want).max() < 1e-12


def _peaked_case():
    """Small fp32 case with aligned sinks, so that tiles are skipped in-kernel."""
    return synthetic.lowrank_case(synthetic.CONFIG_SEEDS[1], [1024], h_q=2, h_kv=1, head_dim=64,
                                  block=64, pool=8, budget=0.25, dtype="f32", sink_logit=24.0,
                                  name="sinks-small")


def test_osk_skip_soundness_and_effect_bound():
    """Every in-kernel skipped block holds less than B*tau of the row's softmax
    mass under the dense normaliser and under the computed-blocks normaliser,
    for every valid row; the output moves by at most 2 max|v| times the
    skipped mass."""
    case = _peaked_case()
    ko = cases.kap_case(case)
    on = cases.osk_case(case, ko["order"], ko["count"])
    off_ = cases.osk_case(case, ko["order"], ko["count"], tau=0.0)
    assert on["skipped"].sum() > 0 and (on["skip_bits"] == 0).sum() > on["visited"][0, 0].size
    q, k, v = cases.sequence_inputs(case, 0)
    B, tau = case.block, case.tau
    Lq = q.shape[0]
    vmax = np.abs(v).max()
    for h, qb in [(h, qb) for h in range(case.h_q) for qb in range(layout.cdiv(Lq, B))]:
        s_full = case.scale * q[:, h] @ k[:, 0].T
        s_full = np.where(np.arange(Lq)[None, :] <= np.arange(Lq)[:, None], s_full, -np.inf)
        rows = np.arange(qb * B, min(qb * B + B, Lq))
        lst = ko["order"][0, 0, qb, : ko["count"][0, 0, qb]]
        bits = on["skip_bits"][0, h, qb, : len(lst)]
        comp = [kb for kb, b_ in zip(lst, bits) if b_ == 0]
        skip = [kb for kb, b_ in zip(lst, bits) if b_ == 1]
        M = s_full[rows].max(axis=1, keepdims=True)
        dense_den = np.exp(s_full[rows] - M).sum(axis=1)
        cols_c = np.concatenate([np.arange(kb * B, kb * B + B) for kb in comp])
        Mc = s_full[rows][:, cols_c].max(axis=1, keepdims=True)
        vis_den = np.exp(s_full[rows][:, cols_c] - Mc).sum(axis=1)
        skipped_mass = np.zeros(len(rows))
        for kb in skip:
            cols = np.arange(kb * B, kb * B + B)
            m1 = np.exp(s_full[rows][:, cols] - M).sum(axis=1) / dense_den
            m2 = np.exp(s_full[rows][:, cols] - Mc).sum(axis=1) / vis_den
            assert np.all(m1 < B * tau) and np.all(m2 < B * tau)
        # effect bound against the tau=0 run (mass under the listed normaliser)
        cols_l = np.concatenate([np.arange(kb * B, kb * B + B) for kb in lst])
        Ml = s_full[rows][:, cols_l].max(axis=1, keepdims=True)
        den_l = np.exp(s_full[rows][:, cols_l] - Ml).sum(axis=1)
        for kb in skip:
            cols = np.arange(kb * B, kb * B + B)
            skipped_mass += np.exp(s_full[rows][:, cols] - Ml).sum(axis=1) / den_l
        dlt = np.abs(on["O"][rows, h] - off_["O"][rows, h]).max(axis=1)
        assert np.all(dlt <= 2 * vmax * skipped_mass + 1e-12)


def test_osk_hand_example():
    with open(os.path.join(GOLDEN, "osk_hand_example.json")) as f:
        ex_ = json.load(f)
    pr = ex_["params"]
    q = np.array(ex_["q"], dtype=np.float64).reshape(-1, 1, 1)
    k = np.array(ex_["k"], dtype=np.float64).reshape(-1, 1, 1)
    v = np.array(ex_["v"], dtype=np.float64).reshape(-1, 1, 1)
    order = np.array([[[0, -1], ex_["order_qb1"]]], dtype=np.int32)
    count = np.array([[1, 2]], dtype=np.int32)
    out = osk.osk_sequence(q, k, v, order, count, pr["scale"], pr["tau"], 1, pr["block"])
    want = ex_["expected"]
    assert np.allclose(out["O"][2:4, 0, 0], want["O_rows_2_3"], rtol=0, atol=1e-12)
    assert list(out["skip_bits"][0, 1]) == want["skip_bits_qb1"]
    assert out["skipped"][0, 1] == want["skipped_qb1"]
    q2 = q.copy()
    q2[3, 0, 0] = want["variant_q3"]
    out2 = osk.osk_sequence(q2, k, v, order, count, pr["scale"], pr["tau"], 1, pr["block"])
    assert list(out2["skip_bits"][0, 1]) == want["variant_skip_bits_qb1"]


def test_osk_first_block_never_skipped_and_tau0_never_skips():
    case = _peaked_case()
    ko = cases.kap_case(case)
    on = cases.osk_case(case, ko["order"], ko["count"])
    assert np.all(on["skip_bits"][..., 0] == 0)
    off_ = cases.osk_case(case, ko["order"], ko["count"], tau=0.0)
    assert off_["skipped"].sum() == 0
    np.testing.assert_array_equal(on["visited"][0, 0], ko["count"][0, 0])


# ---------------------------------------------------------------- KAP ------

def test_kap_hand_example():
    with open(os.path.join(GOLDEN, "kap_hand_example.json")) as f:
        ex_ = json.load(f)
    pr = ex_["params"]
    qh = np.array(ex_["q_heads"], dtype=np.float64)  # [H, L]
    q = qh.T[:, :, None]
    k = np.array(ex_["k"], dtype=np.float64)[:, None, None]
    for budget, want in ex_["expected"].items():
        if budget.startswith("block"):
            continue
        kmax = max(len(o) for o in want["order"])
        for prec in ("fp64", "fp32"):
            out = kap.kap_sequence(q, k, pr["scale"], pr["block"], pr["pool"], float(budget), kmax, prec)
            for qb, (o, h) in enumerate(zip(want["order"], want["hrm"])):
                assert out["count"][0, qb] == len(o)
                assert list(out["order"][0, qb, : len(o)]) == o
                assert list(out["hrm"][0, qb, : len(o)]) == h
    out = kap.kap_sequence(q, k, 1.0, 2, 1, 0.5, 2, "fp64")
    assert np.allclose(out["s"][0, 3], ex_["expected"]["block_scores_qb3"], atol=1e-4)
    assert np.allclose(out["s"][0, 2, :3], ex_["expected"]["block_scores_qb2"], atol=1e-4)


def test_kap_hrm_exact_ties_only():
    """HRM means the block attains the row max exactly: an exact tie flags both
    blocks, a block one part in 1e7 below the max is not flagged."""
    B = 2
    q = np.ones((4, 1, 1))
    for k_vals, want in [([3.0, 0.0, 3.0, 1.0], {0, 1}),
                         ([3.0, 0.0, 3.0 - 3e-7, 1.0], {0}),
                         ([3.0 - 3e-7, 0.0, 3.0, 1.0], {1})]:
        k = np.array(k_vals)[:, None, None]
        for prec in ("fp64", "fp32"):
            out = kap.kap_sequence(q, k, 1.0, B, 1, 1.0, 2, prec)
            assert set(np.nonzero(out["hrm_full"][0, 1])[0].tolist()) == want


def test_kap_hrm_bruteforce_pool1():
    """At p=1 the HRM set of (g, qb) is exactly the set of blocks that hold the
    argmax key of some row of qb for some head of g (dot products by loops)."""
    rng = np.random.default_rng(11)
    L, Hq, Hkv, d, B = 256, 4, 2, 8, 16
    q = rng.standard_normal((L, Hq, d))
    k = rng.standard_normal((L, Hkv, d))
    out = kap.kap_sequence(q, k, 0.5, B, 1, 1.0, L // B, "fp64")
    G = Hq // Hkv
    for g in range(Hkv):
        for qb in range(L // B):
            want = set()
            for h in range(g * G, (g + 1) * G):
                for i in range(qb * B, qb * B + B):
                    sc = [sum(q[i, h, t] * k[j, g, t] for t in range(d)) for j in range(i + 1)]
                    want.add(int(np.argmax(sc)) // B)
            got = set(np.nonzero(out["hrm_full"][g, qb])[0].tolist())
            assert got == want


def test_kap_closed_form_pool_equals_block():
    """p = B, G = 1: P[qb, kb] = scale * mean(Q of qb) . mean(K of kb) for
    kb <= qb and -inf above the diagonal (ragged tails average what exists)."""
    rng = np.random.default_rng(12)
    L, d, B = 200, 8, 32
    q = rng.standard_normal((L, 1, d))
    k = rng.standard_normal((L, 1, d))
    qt = kap.pool_tokens(q, B)
    kt = kap.pool_tokens(k, B)
    P = kap.proxy_scores(qt, kt, 0.3, B, B, L, L)
    nb = layout.cdiv(L, B)
    for a in range(nb):
        for b in range(nb):
            if b > a:
                assert P[0, a, b] == -np.inf
                continue
            mq = q[a * B : min(a * B + B, L), 0].sum(axis=0) / len(range(a * B, min(a * B + B, L)))
            mk = k[b * B : min(b * B + B, L), 0].sum(axis=0) / len(range(b * B, min(b * B + B, L)))
            assert abs(P[0, a, b] - 0.3 * float(mq @ mk)) < 1e-12


def test_pool_identity_and_tail():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((10, 2, 3))
    assert np.array_equal(kap.pool_tokens(x, 1), x)
    t = kap.pool_tokens(x, 4)
    assert t.shape == (3, 2, 3)
    assert np.allclose(t[2], x[8:10].mean(axis=0), atol=1e-15)


def _check_selection(out, B, Lq, Lk, budget):
    s, hfull = out["s"], out["hrm_full"]
    for g in range(out["order"].shape[0]):
        for qb in range(out["order"].shape[1]):
            n = layout.n_causal_blocks(qb, B, Lq, Lk)
            cnt = int(out["count"][g, qb])
            assert cnt == layout.budget_count(n, budget)
            sel = out["order"][g, qb, :cnt].tolist()
            assert len(set(sel)) == cnt and all(0 <= kb < n for kb in sel)
            assert np.all(out["order"][g, qb, cnt:] == -1)
            keys = [(int(hfull[g, qb, kb]), float(s[g, qb, kb]), -kb) for kb in range(n)]
            got = [keys[kb] for kb in sel]
            assert all(got[i] > got[i + 1] for i in range(cnt - 1))  # strictly descending
            rest = [keys[kb] for kb in range(n) if kb not in sel]
            if rest:
                assert min(got) > max(rest)  # the kept ones are the top-k
            flags = out["hrm"][g, qb, :cnt].tolist()
            assert flags == sorted(flags, reverse=True)  # HRM entries first
            assert flags == [int(hfull[g, qb, kb]) for kb in sel]


@pytest.mark.parametrize("precision", ["fp64", "fp32"])
def test_kap_selection_properties(precision):
    case = _small_case(seed=21, lq=900, lk=1300, budget=0.2)
    q, k, _ = cases.sequence_inputs(case, 0)
    kmax = layout.kmax(case.block, case.seqlens_q, case.seqlens_k.tolist(), case.budget)
    out = kap.kap_sequence(q, k, case.scale, case.block, case.pool, case.budget, kmax, precision)
    _check_selection(out, case.block, 900, 1300, case.budget)


def test_kap_fp32_spec_tracks_fp64():
    case = _small_case(seed=22, lq=640, budget=0.3)
    q, k, _ = cases.sequence_inputs(case, 0)
    a = kap.kap_sequence(q, k, case.scale, case.block, case.pool, 0.3, 10, "fp64")
    b = kap.kap_sequence(q, k, case.scale, case.block, case.pool, 0.3, 10, "fp32")
    assert np.allclose(b["s"], a["s"], rtol=2e-5, atol=1e-30)


def test_budget_closed_forms():
    """Per-row counts k = ceil(beta*n) summed over a causal triangle of N blocks
    equal the arithmetic-series closed form (B=128, aligned prefill)."""
    def total(N, beta_num, beta_den, off_blocks=0):
        tot = 0
        for qb in range(N):
            n = off_blocks + qb + 1
            tot += -(-n * beta_num // beta_den)
        return tot

    def via_oracle(Lq, Lk, B, beta):
        return sum(layout.budget_count(layout.n_causal_blocks(qb, B, Lq, Lk), beta)
                   for qb in range(layout.cdiv(Lq, B)))

    # tiny case: 16 blocks at 25% -> 1,1,1,1,2,2,2,2,3,3,3,3,4,4,4,4 = 40 of 136
    assert [layout.budget_count(n, 0.25) for n in range(1, 17)] == [1] * 4 + [2] * 4 + [3] * 4 + [4] * 4
    assert via_oracle(1024, 1024, 64, 0.25) == 40
    # 32K at 10%: sum_{n=1}^{256} ceil(n/10) = 10*(1+..+25) + 6*26 = 3406 of 32896
    assert via_oracle(32768, 32768, 128, 0.1) == 10 * 25 * 26 // 2 + 6 * 26 == 3406
    assert total(256, 1, 10) == 3406
    # 128K at 5/10/25%
    assert via_oracle(131072, 131072, 128, 0.05) == total(1024, 1, 20) == 26728
    assert via_oracle(131072, 131072, 128, 0.10) == total(1024, 1, 10) == 52942
    assert via_oracle(131072, 131072, 128, 0.25) == total(1024, 1, 4) == 131584
    # 4K chunk over 64K cache at 10%: n = 481..512
    assert via_oracle(4096, 65536, 128, 0.1) == total(32, 1, 10, off_blocks=480) == 1604
    # kmax
    assert layout.kmax(128, [131072], [131072], 0.1) == 103


# ---------------------------------------------------------------- inputs ---

def test_generator_determinism():
    a = synthetic.config_case(2, scale_down=64)
    b = synthetic.config_case(2, scale_down=64)
    for name in ("q", "k_pages", "v_pages"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    c = synthetic.config_case(4, scale_down=16)
    assert torch.isnan(c.k_pages.float()).any()  # spare pages are poisoned
    used = set(c.block_table[0].tolist())
    assert len(used) == c.block_table.shape[1]
    for pg in range(c.k_pages.shape[0]):
        if pg not in used:
            assert torch.isnan(c.k_pages[pg].float()).all()


# ------------------------------------------- hand pins: paging, R4, R7, R9 ---

def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_gather_pages_hand_example():
    """Logical KV blocks come from the pages the block table names, in table
    order (KV-head-major pages, CompactAttention page, execution stage)."""
    ex_ = _load("gather_pages_hand_example.json")
    P, H, B = ex_["num_pages"], ex_["h_kv"], ex_["block"]
    pages = np.zeros((P, H, B, 1))
    for p_ in range(P):
        for h in range(H):
            for r in range(B):
                pages[p_, h, r, 0] = 100 * p_ + 10 * h + r
    got = layout.gather_pages(pages, np.array(ex_["table_row"], dtype=np.int32), ex_["seqlen_k"])
    assert got.shape == (ex_["seqlen_k"], H, 1)
    assert got[:, 0, 0].tolist() == ex_["expected"]["head0"]
    assert got[:, 1, 0].tolist() == ex_["expected"]["head1"]


def test_shuffled_pages_give_the_same_oracle_results():
    """The page pool's arrangement is not part of the method: the same logical
    K/V in a shuffled, NaN-padded pool gives the same proxy lists and the same
    attention output as in an identity-ordered pool."""
    kw = dict(h_q=4, h_kv=2, head_dim=16, block=64, pool=8, budget=0.3, dtype="f32")
    a = synthetic.lowrank_case(31, [300], [700], **kw)
    b = synthetic.lowrank_case(31, [300], [700], shuffle_pages=True, spare_pages=3, **kw)
    assert not np.array_equal(a.block_table.numpy(), b.block_table.numpy())
    ka, kb_ = cases.kap_case(a), cases.kap_case(b)
    for name in ("order", "hrm", "count"):
        np.testing.assert_array_equal(ka[name], kb_[name])
    oa = cases.osk_case(a, ka["order"], ka["count"])
    ob = cases.osk_case(b, ka["order"], ka["count"])
    assert np.isfinite(ob["O"]).all()
    np.testing.assert_array_equal(oa["O"], ob["O"])
    np.testing.assert_array_equal(cases.dense_case(a)["O"], cases.dense_case(b)["O"])


@pytest.mark.parametrize("precision", ["fp64", "fp32"])
def test_kap_chunk_offset_not_multiple_of_pool(precision):
    """R4 at a chunked offset (7) that the pool factor (2) does not divide: the
    last token of a pooled query window decides which pooled keys it sees."""
    ex_ = _load("kap_chunk_offset_hand_example.json")
    pr = ex_["params"]
    q = np.array(ex_["q"], dtype=np.float64)[:, None, None]
    k = np.array(ex_["k"], dtype=np.float64)[:, None, None]
    out = kap.kap_sequence(q, k, pr["scale"], pr["block"], pr["pool"], 1.0, 3, precision)
    assert out["P"][0].tolist() == ex_["expected"]["P"]
    for qb in range(2):
        assert out["count"][0, qb] == 3
        assert out["order"][0, qb].tolist() == ex_["expected"]["order"][qb]
        assert out["hrm"][0, qb].tolist() == ex_["expected"]["hrm"][qb]
    assert np.allclose(out["s"][0, 0], ex_["expected"]["s_qb0"], rtol=0, atol=1e-7)
    assert np.allclose(out["s"][0, 1], ex_["expected"]["s_qb1"], rtol=0, atol=1e-7)


@pytest.mark.parametrize("precision", ["fp64", "fp32"])
def test_kap_tie_break_order(precision):
    """R9: equal block scores are ordered by ascending KV block index, inside
    the HRM group and inside the rest, and the budget cut respects it."""
    ex_ = _load("kap_tie_break_hand_example.json")
    pr = ex_["params"]
    q = np.array(ex_["q"], dtype=np.float64)[:, None, None]
    k = np.array(ex_["k"], dtype=np.float64)[:, None, None]
    for budget, want in ex_["expected"].items():
        kmax = len(want["qb3"])
        out = kap.kap_sequence(q, k, pr["scale"], pr["block"], pr["pool"], float(budget), kmax, precision)
        assert out["s"][0, 3, 1] == out["s"][0, 3, 2]  # an exact tie
        assert out["order"][0, 3].tolist() == want["qb3"]
        assert out["hrm"][0, 3].tolist() == want["qb3_hrm"]
        if "qb2" in want:
            assert out["order"][0, 2, :3].tolist() == want["qb2"]
            assert out["hrm"][0, 2, :3].tolist() == want["qb2_hrm"]


def _sum_order_P(ex_, part):
    d24 = np.array([int(ex_["D24_bits"], 16)], dtype=np.uint32).view(np.float32)[0]
    tok = {"0": np.float32(0.0), "-100": np.float32(-100.0), "-inf": np.float32(-np.inf), "D24": d24}
    return np.array([[[tok[x] for x in row] for row in head] for head in part["P"]], dtype=np.float32)


def test_kap_sum_order_bits():
    """R7: the block score is a sequential fp32 sum, heads outer and pooled
    rows inner, each add rounded to nearest even; three blocks whose bits each
    expose a different summation order."""
    ex_ = _load("kap_sum_order_hand_example.json")
    pr = ex_["params"]
    P = _sum_order_P(ex_, ex_)
    assert ex32(np.float32(P[0, 2, 0])) == np.float32(2.0 ** -24)
    out = kap.kap_from_scores(P, pr["h_q"] // pr["h_kv"], pr["block"], pr["pool"], pr["Lq"], pr["Lk"],
                              pr["budget"], 3, "fp32")
    bits = lambda x: [f"0x{int(v):08x}" for v in np.asarray(x, dtype=np.float32).view(np.uint32)]
    assert bits(out["s"][0, 1]) == ex_["expected"]["s_qb1_bits"]
    assert bits(out["s"][0, 0]) == ex_["expected"]["s_qb0_bits"]
    assert out["order"][0].tolist() == ex_["expected"]["order"]
    assert out["hrm"][0].tolist() == ex_["expected"]["hrm"]
    assert out["count"][0].tolist() == ex_["expected"]["count"]
    # eight terms per block: pairwise and blocked sums differ from the sequential one
    pb = ex_["part_b"]
    prb = pb["params"]
    out = kap.kap_from_scores(_sum_order_P(ex_, pb), prb["h_q"] // prb["h_kv"], prb["block"], prb["pool"],
                              prb["Lq"], prb["Lk"], prb["budget"], 2, "fp32")
    assert bits(out["s"][0, 0]) == pb["expected"]["s_bits"]
    assert out["order"][0, 0].tolist() == pb["expected"]["order"]
    assert out["hrm"][0, 0].tolist() == pb["expected"]["hrm"]
    assert out["count"][0, 0] == pb["expected"]["count"]


def ex32(x):
    return ex.exp32(np.asarray([x], dtype=np.float32))[0]
