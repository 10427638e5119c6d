"""Run the oracle over a whole packed batch, in the library's output layouts.

Inputs are a ``synthetic.Case`` (CPU torch tensors); bf16 values are widened
exactly to fp64. Outputs use the same shapes the C-ABI writes:

    order, hrm      [batch, h_kv, max_nq, kmax]   (int32 -1 pad, uint8 0 pad)
    count           [batch, h_kv, max_nq]
    P               [batch, h_q, max_nr, max_nk]  (fp32 or fp64, -inf pad)
    s               [batch, h_kv, max_nq, max_nk] (block scores, 0 pad)
    O               [total_q, h_q, d]
    lse             [h_q, total_q]
    visited/skipped [batch, h_q, max_nq]
    skip_bits       [batch, h_q, max_nq, kmax]    (255 pad)
"""
from __future__ import annotations

import numpy as np

from . import dense as _dense
from . import kap as _kap
from . import masks as _masks
from . import osk as _osk
from .layout import cdiv, gather_pages, kmax as _kmax, n_causal_blocks


def _f64(t) -> np.ndarray:
    return t.float().numpy().astype(np.float64)


def sequence_inputs(case, b: int):
    """(q, k, v) of sequence b as fp64 arrays [L, H, d]."""
    cu = case.cu_seqlens_q.tolist()
    Lk = int(case.seqlens_k[b])
    table = case.block_table[b].numpy()
    q = _f64(case.q[cu[b] : cu[b + 1]])
    k = gather_pages(_f64(case.k_pages), table, Lk)
    v = gather_pages(_f64(case.v_pages), table, Lk)
    return q, k, v


def dims(case):
    lq = case.seqlens_q
    lk = case.seqlens_k.tolist()
    B, p = case.block, case.pool
    return {
        "max_nq": max(cdiv(x, B) for x in lq),
        "max_nk": max(cdiv(x, B) for x in lk),
        "max_nr": max(cdiv(x, p) for x in lq),
        "kmax": _kmax(B, lq, lk, case.budget),
    }


def kap_case(case, precision: str = "fp64", P_given=None, budget=None):
    """The proxy over the batch. With ``P_given`` ([batch, h_q, max_nr, max_nk]
    fp32, e.g. the GPU's exported scores) only the ranking, flagging and sort
    run (parity mode)."""
    dm = dims(case)
    budget = case.budget if budget is None else budget
    B, p = case.block, case.pool
    Hq, Hkv = case.h_q, case.h_kv
    nb = case.batch
    kmax = _kmax(B, case.seqlens_q, case.seqlens_k.tolist(), budget)
    fdt = np.float32 if precision == "fp32" else np.float64
    order = np.full((nb, Hkv, dm["max_nq"], kmax), -1, dtype=np.int32)
    hrm = np.zeros((nb, Hkv, dm["max_nq"], kmax), dtype=np.uint8)
    count = np.zeros((nb, Hkv, dm["max_nq"]), dtype=np.int32)
    P = np.full((nb, Hq, dm["max_nr"], dm["max_nk"]), -np.inf, dtype=fdt)
    s = np.zeros((nb, Hkv, dm["max_nq"], dm["max_nk"]), dtype=fdt)
    for b in range(nb):
        Lq = case.seqlens_q[b]
        Lk = int(case.seqlens_k[b])
        if Lq == 0:
            continue
        nq, nk, nr = cdiv(Lq, B), cdiv(Lk, B), cdiv(Lq, p)
        if P_given is not None:
            Pb = np.asarray(P_given[b, :, :nr, :nk])
            out = _kap.kap_from_scores(Pb, Hq // Hkv, B, p, Lq, Lk, budget, kmax, precision)
            out["P"] = Pb
        else:
            q, k, _ = sequence_inputs(case, b)
            out = _kap.kap_sequence(q, k, case.scale, B, p, budget, kmax, precision)
        order[b, :, :nq] = out["order"]
        hrm[b, :, :nq] = out["hrm"]
        count[b, :, :nq] = out["count"]
        P[b, :, :nr, :nk] = out["P"]
        s[b, :, :nq, :nk] = out["s"]
    return {"order": order, "hrm": hrm, "count": count, "P": P, "s": s, "kmax": kmax}


def osk_case(case, order, count, tau=None, query_blocks=None):
    """Ordered walk with skips over the batch, given the order lists."""
    dm = dims(case)
    tau = case.tau if tau is None else tau
    B, Hq, Hkv, d = case.block, case.h_q, case.h_kv, case.head_dim
    G = Hq // Hkv
    nb = case.batch
    kmax = order.shape[3]
    cu = case.cu_seqlens_q.tolist()
    O = np.zeros((cu[-1], Hq, d))
    lse = np.full((Hq, cu[-1]), -np.inf)
    visited = np.zeros((nb, Hq, dm["max_nq"]), dtype=np.int32)
    skipped = np.zeros((nb, Hq, dm["max_nq"]), dtype=np.int32)
    bits = np.full((nb, Hq, dm["max_nq"], kmax), 255, dtype=np.uint8)
    margin = np.full((nb, Hq, dm["max_nq"], kmax), np.nan)
    for b in range(nb):
        Lq = case.seqlens_q[b]
        if Lq == 0:
            continue
        nq = cdiv(Lq, B)
        q, k, v = sequence_inputs(case, b)
        qbs = None if query_blocks is None else [x for x in query_blocks[b] if x < nq]
        out = _osk.osk_sequence(q, k, v, order[b, :, :nq], count[b, :, :nq],
                                case.scale, tau, G, B, qbs)
        O[cu[b] : cu[b + 1]] = out["O"]
        lse[:, cu[b] : cu[b + 1]] = out["lse"]
        visited[b, :, :nq] = out["visited"]
        skipped[b, :, :nq] = out["skipped"]
        bits[b, :, :nq] = out["skip_bits"]
        margin[b, :, :nq] = out["margin"]
    return {"O": O, "lse": lse, "visited": visited, "skipped": skipped,
            "skip_bits": bits, "margin": margin}


def dense_case(case, rows_per_seq=None):
    """Dense causal attention over the batch (optionally only some rows)."""
    Hq, d = case.h_q, case.head_dim
    cu = case.cu_seqlens_q.tolist()
    O = np.zeros((cu[-1], Hq, d))
    lse = np.full((Hq, cu[-1]), -np.inf)
    for b in range(case.batch):
        if cu[b + 1] == cu[b]:
            continue
        q, k, v = sequence_inputs(case, b)
        rows = None if rows_per_seq is None else rows_per_seq[b]
        o, ls = _dense.dense_sequence(q, k, v, case.scale, rows=rows)
        idx = np.arange(cu[b + 1] - cu[b]) if rows is None else np.asarray(rows)
        O[cu[b] + idx] = o
        lse[:, cu[b] + idx] = ls
    return {"O": O, "lse": lse}


def n_causal_rows(case) -> np.ndarray:
    """Causal KV blocks of every row [batch, h_kv, max_nq] (0 past a sequence's end)."""
    dm = dims(case)
    B = case.block
    n = np.zeros((case.batch, case.h_kv, dm["max_nq"]), dtype=np.int64)
    for b in range(case.batch):
        Lq, Lk = case.seqlens_q[b], int(case.seqlens_k[b])
        for qb in range(cdiv(Lq, B)):
            n[b, :, qb] = n_causal_blocks(qb, B, Lq, Lk)
    return n


def block_mass_case(case) -> np.ndarray:
    """Exact block mass [batch, h_q, max_nq, max_nk] over the batch (fp64)."""
    dm = dims(case)
    M = np.zeros((case.batch, case.h_q, dm["max_nq"], dm["max_nk"]))
    G = case.h_q // case.h_kv
    for b in range(case.batch):
        Lq, Lk = case.seqlens_q[b], int(case.seqlens_k[b])
        if Lq == 0:
            continue
        q, k, _ = sequence_inputs(case, b)
        M[b, :, : cdiv(Lq, case.block), : cdiv(Lk, case.block)] = _masks.block_mass_sequence(
            q, k, case.scale, G, case.block)
    return M
