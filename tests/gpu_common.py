"""Helpers shared by the GPU tests: move a synthetic case to the device, run
the library through its C ABI, and compare with the oracle."""
import math
import sys

import numpy as np
import torch

import block_sparse_attention_26_amd as cosa
from oracle import cases as oc, kap as okap, layout, osk as oosk

# bf16 inputs: max-abs 2e-2 and mean-abs 2e-3 against the fp64 oracle; fp32 inputs: 1e-4.
TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-4)}
# skip decisions whose fp64 margin is within this many nats of the threshold
# may legitimately differ between fp32 GPU arithmetic and the fp64 oracle
AMBIGUOUS_NATS = 1e-3


def say(*args):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[gpu]", *args, file=sys.stderr, flush=True)


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cosa.load()


class OnDevice:
    def __init__(self, case):
        self.case = case
        self.q = case.q.cuda()
        self.k = case.k_pages.cuda()
        self.v = case.v_pages.cuda()
        self.problem = cosa.Problem.from_case(case)


def check_output(O_gpu, O_ref, dtype, what=""):
    """Element-wise comparison of the GPU output with the oracle's."""
    o = O_gpu.float().cpu().numpy().astype(np.float64)
    err = np.abs(o - O_ref)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    mx, mean = TOL[dtype]
    assert err.max() <= mx, f"{what}: max abs err {err.max():.3e} > {mx}"
    assert err.mean() <= mean, f"{what}: mean abs err {err.mean():.3e} > {mean}"
    return float(err.max()), float(err.mean())


def check_skip_sets(gpu, ref, count, G):
    """visited identical; skip bits identical outside the ambiguity band."""
    vis = gpu["visited"].cpu().numpy()
    nb, hq, nq = vis.shape
    want_vis = np.repeat(count, G, axis=1)  # [b, h_kv, nq] -> [b, h_q, nq]
    np.testing.assert_array_equal(vis, want_vis)
    np.testing.assert_array_equal(vis, ref["visited"])
    bits = gpu["skip_bits"].cpu().numpy()
    rb = ref["skip_bits"]
    amb = np.abs(ref["margin"]) < AMBIGUOUS_NATS
    diff = (bits != rb) & ~amb
    assert not diff.any(), f"{int(diff.sum())} skip decisions differ outside the ambiguity band"
    sk = gpu["skipped"].cpu().numpy()
    np.testing.assert_array_equal(sk, (bits == 1).sum(axis=3))
    return int(amb.sum()), int((bits == 1).sum())


# ---- full-size checks (bench launch configuration, sampled where the oracle is slow) ----

def sample_qbs(nq, n_mid=12):
    mid = np.linspace(2, nq - 3, n_mid).round().astype(int).tolist() if nq > 4 else []
    return sorted(set([0, 1, nq - 2, nq - 1] + mid) & set(range(nq)))


def run_gpu(case, budget=None, tau=None):
    """Bench configuration plus a diagnostic run; returns host arrays."""
    budget = case.budget if budget is None else budget
    tau = case.tau if tau is None else tau
    q, k, v = case.q.cuda(), case.k_pages.cuda(), case.v_pages.cuda()
    pr = cosa.Problem.from_case(case)
    say(case.name, "proxy (workspace mode) + walk (bench configuration)")
    ka = cosa.kap_order(pr, q, k, case.pool, budget)
    oa = cosa.osk_attention(pr, q, k, v, ka["order"], ka["count"], tau)
    say(case.name, "proxy (scores exported) + walk (skip bits)")
    kx = cosa.kap_order(pr, q, k, case.pool, budget, export_scores=True, export_block_scores=True)
    ox = cosa.osk_attention(pr, q, k, v, ka["order"], ka["count"], tau, skip_bits=True, lse=True)
    torch.cuda.synchronize()
    for name in ("order", "hrm", "count"):
        assert torch.equal(ka[name], kx[name]), name
    assert torch.equal(oa["O"].view(torch.int16), ox["O"].view(torch.int16)), "O differs between the two runs"
    for name in ("visited", "skipped"):
        assert torch.equal(oa[name], ox[name]), name
    out = {name: ka[name].cpu().numpy() for name in ("order", "hrm", "count")}
    out["P"] = kx["P"].cpu().numpy()
    out["s"] = kx["s"].cpu().numpy()
    out["O"] = ox["O"].float().cpu().numpy()  # compared in fp64 (upcast per slice)
    out["walk"] = {"visited": ox["visited"], "skipped": ox["skipped"], "skip_bits": ox["skip_bits"]}
    out["dev"] = (pr, q, k, v)
    return out


def check_lists(case, g, budget, rows=None):
    """Every (or the listed) (b, g, qb) row: order, HRM flags, count and block
    scores bit-exact against the oracle fed the same fp32 proxy scores."""
    B, p = case.block, case.pool
    G = case.h_q // case.h_kv
    per = B // p
    n_rows = 0
    for b in range(case.batch):
        Lq, Lk = case.seqlens_q[b], int(case.seqlens_k[b])
        nq, nr = layout.cdiv(Lq, B), layout.cdiv(Lq, p)
        for kvh in range(case.h_kv):
            for qb in (range(nq) if rows is None else [x for x in rows[b] if x < nq]):
                n = layout.n_causal_blocks(qb, B, Lq, Lk)
                P = g["P"][b, kvh * G:(kvh + 1) * G, qb * per:min(qb * per + per, nr), :n]
                s, fl = okap.rank_row(P, "fp32")
                lst, flags = okap.select_row(s, fl, n, budget)
                where = (b, kvh, qb)
                assert g["count"][where] == len(lst), where
                assert g["order"][where][:len(lst)].tolist() == lst, where
                assert np.all(g["order"][where][len(lst):] == -1), where
                assert g["hrm"][where][:len(lst)].tolist() == flags, where
                assert np.array_equal(g["s"][where][:n].view(np.uint32), s.view(np.uint32)), where
                n_rows += 1
    return n_rows


def check_proxy_scores(case, g):
    """P upstream of the bit-exact contract: visibility pattern exact, finite
    entries within 1e-2 of the largest magnitude of the fp64 oracle's."""
    P64 = oc.kap_case(case, precision="fp64")["P"]
    fin = np.isfinite(P64)
    assert np.array_equal(np.isfinite(g["P"]), fin), "visibility pattern of P"
    assert np.abs(g["P"][fin] - P64[fin]).max() <= 1e-2 * np.abs(P64[fin]).max()


def check_walk(case, g, qbs_per_seq=None, tau=None, groups=None):
    """Output of the listed query blocks (all when None) of the listed KV
    groups (all when None) against the oracle's ordered walk over the same
    lists, per KV group; skip sets identical outside the ambiguity band."""
    tau = case.tau if tau is None else tau
    B, G = case.block, case.h_q // case.h_kv
    mx, mean = TOL[case.dtype]
    cu = case.cu_seqlens_q.tolist()
    bits = g["walk"]["skip_bits"].cpu().numpy()
    vis = g["walk"]["visited"].cpu().numpy()
    skp = g["walk"]["skipped"].cpu().numpy()
    errs, n_amb, n_skip = [], 0, 0
    for b in range(case.batch):
        q, k, v = oc.sequence_inputs(case, b)
        Lq = q.shape[0]
        nq = layout.cdiv(Lq, B)
        qbs = list(range(nq)) if qbs_per_seq is None else [x for x in qbs_per_seq[b] if x < nq]
        rows = np.concatenate([np.arange(qb * B, min(qb * B + B, Lq)) for qb in qbs])
        for kvh in (range(case.h_kv) if groups is None else groups):
            hs = slice(kvh * G, (kvh + 1) * G)
            ref = oosk.osk_sequence(q[:, hs], k[:, kvh:kvh + 1], v[:, kvh:kvh + 1], g["order"][b, kvh:kvh + 1],
                                    g["count"][b, kvh:kvh + 1], case.scale, tau, G, B, query_blocks=qbs)
            got = g["O"][cu[b] + rows][:, hs]
            err = np.abs(got - ref["O"][rows])
            assert np.isfinite(got).all(), (b, kvh)
            assert err.max() <= mx, (b, kvh, err.max())
            errs.append(err)
            amb = np.abs(ref["margin"]) < AMBIGUOUS_NATS
            for qb in qbs:
                c = g["count"][b, kvh, qb]
                np.testing.assert_array_equal(vis[b, hs, qb], c)
                gb, rb = bits[b, hs, qb, :c], ref["skip_bits"][:, qb, :c]
                assert not ((gb != rb) & ~amb[:, qb, :c]).any(), (b, kvh, qb)
                np.testing.assert_array_equal(skp[b, hs, qb], (gb == 1).sum(axis=1))
                n_amb += int(amb[:, qb, :c].sum())
                n_skip += int((gb == 1).sum())
            say(case.name, f"sequence {b}, KV group {kvh}: walk checked on {len(qbs)} query blocks")
    allerr = np.concatenate([e.ravel() for e in errs])
    assert allerr.mean() <= mean, allerr.mean()
    return float(allerr.max()), float(allerr.mean()), n_amb, n_skip


def check_dense(case, dev, qbs_per_seq):
    """The dense kernel against the fp64 oracle on sampled query blocks."""
    pr, q, k, v = dev
    de = cosa.dense_attention(pr, q, k, v)
    torch.cuda.synchronize()
    O = de["O"].float().cpu().numpy().astype(np.float64)
    B = case.block
    mx, mean = TOL[case.dtype]
    rows_per_seq = []
    for b in range(case.batch):
        Lq = case.seqlens_q[b]
        qbs = [x for x in qbs_per_seq[b] if x * B < Lq]
        rows_per_seq.append(np.concatenate([np.arange(qb * B, min(qb * B + B, Lq)) for qb in qbs]))
    ref = oc.dense_case(case, rows_per_seq=rows_per_seq)["O"]
    cu = case.cu_seqlens_q.tolist()
    idx = np.concatenate([cu[b] + r for b, r in enumerate(rows_per_seq)])
    err = np.abs(O[idx] - ref[idx])
    assert err.max() <= mx and err.mean() <= mean, (err.max(), err.mean())
    return O
