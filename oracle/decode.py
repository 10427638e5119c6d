"""Decode-stage ordered walk with a split list (test infrastructure only).

The CoSA pages name decoding as future work and give no method for it. The
reading taken here (R30) keeps every rule of the prefill walk (CoSA summary
§2.3, §1) and adds only what a split-KV decode kernel needs:

R30 A decode step is a prefill chunk of one token per sequence (query at
    absolute position Lk - 1). The list of (sequence, KV group) is cut into
    n_splits contiguous segments, entries [floor(s n / S), floor((s+1) n / S)).
    Each segment is walked on its own, in list order, from m = -inf, l = 0,
    acc = 0, with the skip rule of R11 applied per query head (the tile is
    that head's single row). The segments' results are merged exactly:
        m* = max_s m_s,  O = sum_s e^(m_s - m*) acc_s / sum_s e^(m_s - m*) l_s,
    lse = m* + ln(sum_s e^(m_s - m*) l_s). visited / skipped add over the
    segments. With skipping off the result is softmax attention over the
    listed keys for any n_splits (order invariance, CoSA summary §2.1);
    with skipping on, a segment's first block is never skipped, so the skip
    count depends on n_splits.
"""
from __future__ import annotations

import math

import numpy as np

from .layout import cdiv


def segment_bounds(n: int, n_splits: int):
    """[t0, t1) of every segment of an n-entry list."""
    return [((s * n) // n_splits, ((s + 1) * n) // n_splits) for s in range(n_splits)]


def decode_sequence(q, k, v, order, count, scale: float, tau: float, G: int, B: int, n_splits: int):
    """Split decode walk for one sequence with a single query token.

    q [1, Hq, d], k/v [Lk, Hkv, d], order [Hkv, kmax], count [Hkv].
    Returns O [Hq, d], lse [Hq], visited / skipped [Hq] and the per-decision
    margin [Hq, kmax] (max(m_loc - m) - ln tau, nan where no decision)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, d = q.shape[1], q.shape[2]
    Lk = k.shape[0]
    pos = Lk - 1
    ln_tau = math.log(tau) if tau > 0 else -math.inf
    kmax = order.shape[1]
    O = np.zeros((Hq, d))
    lse = np.full(Hq, -np.inf)
    visited = np.zeros(Hq, dtype=np.int32)
    skipped = np.zeros(Hq, dtype=np.int32)
    margin = np.full((Hq, kmax), np.nan)
    for h in range(Hq):
        g = h // G
        n = int(count[g])
        parts = []
        for t0, t1 in segment_bounds(n, n_splits):
            m, l, acc = -np.inf, 0.0, np.zeros(d)
            for t in range(t0, t1):
                kb = int(order[g, t])
                keys = np.arange(kb * B, min(kb * B + B, Lk))
                keys = keys[keys <= pos]
                s = scale * (k[keys, g, :] @ q[0, h, :])
                m_loc = s.max() if len(s) else -np.inf
                diff = m_loc - m if m_loc != -np.inf else -np.inf
                margin[h, t] = diff - ln_tau
                visited[h] += 1
                if tau > 0 and diff < ln_tau:
                    skipped[h] += 1
                    continue
                m_new = max(m, m_loc)
                alpha = 0.0 if m == -np.inf else math.exp(m - m_new)
                p = np.exp(s - m_new)
                l = alpha * l + p.sum()
                acc = alpha * acc + p @ v[keys, g, :]
                m = m_new
            parts.append((m, l, acc))
        m_star = max(p[0] for p in parts) if parts else -np.inf
        if m_star == -np.inf:
            continue
        lt = sum(math.exp(m_s - m_star) * l_s for m_s, l_s, _ in parts if m_s != -np.inf)
        at = sum(math.exp(m_s - m_star) * a_s for m_s, _, a_s in parts if m_s != -np.inf)
        if lt > 0:
            O[h] = at / lt
            lse[h] = m_star + math.log(lt)
    return {"O": O, "lse": lse, "visited": visited, "skipped": skipped, "margin": margin}


def decode_case(case, order, count, n_splits: int, tau=None):
    """Split decode walk over a packed batch of single-token queries.

    order [batch, h_kv, max_nq, kmax] and count [batch, h_kv, max_nq] in the
    library's layout (max_nq is 1). Returns O [total_q, h_q, d], lse
    [h_q, total_q], visited / skipped [batch, h_q] and margin [batch, h_q, kmax]."""
    from .cases import sequence_inputs

    tau = case.tau if tau is None else tau
    G = case.h_q // case.h_kv
    cu = case.cu_seqlens_q.tolist()
    kmax = order.shape[3]
    O = np.zeros((cu[-1], case.h_q, case.head_dim))
    lse = np.full((case.h_q, cu[-1]), -np.inf)
    visited = np.zeros((case.batch, case.h_q), dtype=np.int32)
    skipped = np.zeros((case.batch, case.h_q), dtype=np.int32)
    margin = np.full((case.batch, case.h_q, kmax), np.nan)
    for b in range(case.batch):
        if cu[b + 1] == cu[b]:
            continue
        q, k, v = sequence_inputs(case, b)
        out = decode_sequence(q, k, v, order[b, :, 0], count[b, :, 0], case.scale, tau, G, case.block, n_splits)
        O[cu[b]] = out["O"]
        lse[:, cu[b]] = out["lse"]
        visited[b] = out["visited"]
        skipped[b] = out["skipped"]
        margin[b] = out["margin"]
    return {"O": O, "lse": lse, "visited": visited, "skipped": skipped, "margin": margin}
