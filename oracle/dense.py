"""Dense causal softmax attention in fp64: the baseline every speedup is
measured against (CoSA summary §4, Experimental Results, efficiency).

Textbook definition, one sequence at a time:
    O_i = sum_j softmax_j(scale * q_i . k_j  over j <= off + i) v_j
with GQA: query head h reads KV head h // G, G = h_q / h_kv. Also returns the
natural-log sum-exp lse_i = log sum_j exp(scale * q_i . k_j).
"""
from __future__ import annotations

import numpy as np


def dense_sequence(q, k, v, scale: float, row_chunk: int = 1024, rows=None):
    """q [Lq, Hq, d], k/v [Lk, Hkv, d] (any float; computed in fp64).

    ``rows`` optionally restricts the computation to a subset of query rows
    (returned outputs are then [len(rows), Hq, d] and [Hq, len(rows)]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, Hq, d = q.shape
    Lk, Hkv, _ = k.shape
    G = Hq // Hkv
    off = Lk - Lq
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), Hq, d))
    lse = np.full((Hq, len(rows)), -np.inf)
    for h in range(Hq):
        g = h // G
        for c0 in range(0, len(rows), row_chunk):
            r = rows[c0 : c0 + row_chunk]
            hi = int(r.max()) + off + 1  # keys any of these rows can see
            s = scale * (q[r, h, :] @ k[:hi, g, :].T)
            vis = np.arange(hi)[None, :] <= (r[:, None] + off)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            den = p.sum(axis=1, keepdims=True)
            out[c0 : c0 + len(r), h, :] = (p @ v[:hi, g, :]) / den
            lse[h, c0 : c0 + len(r)] = (m + np.log(den))[:, 0]
    return out, lse
