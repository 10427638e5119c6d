"""Ordered-Skipping Kernel (OSK) semantics in fp64.

CoSA summary §2.3 ("Stage 2: Ordered-Skipping Kernel") names three fates for
a KV block of a query block: mask-skipped (not in the order list, never
touched), in-kernel skipped (decided from the local and the running row max),
computed (full online-softmax update). §2.1 gives order invariance of the
online-softmax accumulation; §1 fixes the veto granularity (one outlier row
blocks the skip for the whole tile) and notes the running max is a lower bound
of the global max.

Readings:

R8  Query head h uses the order list of its KV group g = h // G; the skip
    decision is taken per query head over all valid rows of the query block.
R11 With tau in (0, 1), block t of the list is skipped iff
        max over valid rows i with a visible key in the block of
            (m_loc_i - m_i)  <  ln(tau)
    where m_loc_i is the row's max scaled score in the block and m_i the
    running max before the block (m_i = -inf gives +inf, so the first block a
    row can see is never skipped). A skip leaves m, l, acc untouched.
    tau = 0 disables skipping.
R12 visited = every listed block (its QK^T is paid), skipped = in-kernel
    skipped, computed = visited - skipped.
R14 Rows past the sequence end do not exist; a row with no visible key in any
    computed block gets O = 0 and lse = -inf.

Besides O and lse the oracle records each decision's margin
mu = max_i(m_loc_i - m_i) - ln(tau) in nats, so a comparison can set aside
decisions that are within rounding of the threshold.
"""
from __future__ import annotations

import math

import numpy as np

from .layout import cdiv


def osk_sequence(q, k, v, order, count, scale: float, tau: float, G: int, B: int,
                 query_blocks=None):
    """Ordered walk with skips for one sequence.

    q [Lq, Hq, d], k/v [Lk, Hkv, d], order [Hkv, Nq, kmax] (int), count
    [Hkv, Nq]. ``query_blocks`` optionally restricts the work to some qb.
    Returns dict with O [Lq, Hq, d] (rows of untouched blocks stay 0),
    lse [Hq, Lq], visited/skipped [Hq, Nq], skip_bits [Hq, Nq, kmax]
    (0 computed, 1 skipped, 255 pad) and margin [Hq, Nq, kmax] (nan pad).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, Hq, d = q.shape
    Lk = k.shape[0]
    off = Lk - Lq
    Nq = cdiv(Lq, B)
    kmax = order.shape[2]
    ln_tau = math.log(tau) if tau > 0 else -math.inf
    O = np.zeros((Lq, Hq, d))
    lse = np.full((Hq, Lq), -np.inf)
    visited = np.zeros((Hq, Nq), dtype=np.int32)
    skipped = np.zeros((Hq, Nq), dtype=np.int32)
    bits = np.full((Hq, Nq, kmax), 255, dtype=np.uint8)
    margin = np.full((Hq, Nq, kmax), np.nan)
    qbs = range(Nq) if query_blocks is None else query_blocks
    with np.errstate(invalid="ignore", divide="ignore"):
        for h in range(Hq):
            g = h // G
            for qb in qbs:
                rows = np.arange(qb * B, min(qb * B + B, Lq))
                pos = rows + off
                m = np.full(len(rows), -np.inf)
                l = np.zeros(len(rows))
                acc = np.zeros((len(rows), d))
                n_list = int(count[g, qb])
                visited[h, qb] = n_list
                for t in range(n_list):
                    kb = int(order[g, qb, t])
                    keys = np.arange(kb * B, min(kb * B + B, Lk))
                    s = scale * (q[rows, h, :] @ k[keys, g, :].T)
                    vis = keys[None, :] <= pos[:, None]
                    s = np.where(vis, s, -np.inf)
                    m_loc = s.max(axis=1)
                    diff = np.where(m_loc == -np.inf, -np.inf, m_loc - m)
                    worst = diff.max()
                    margin[h, qb, t] = worst - ln_tau
                    if tau > 0 and worst < ln_tau:
                        skipped[h, qb] += 1
                        bits[h, qb, t] = 1
                        continue
                    bits[h, qb, t] = 0
                    m_new = np.maximum(m, m_loc)
                    alpha = np.where(m == -np.inf, 0.0, np.exp(m - m_new))
                    pexp = np.where(vis, np.exp(s - m_new[:, None]), 0.0)
                    l = alpha * l + pexp.sum(axis=1)
                    acc = alpha[:, None] * acc + pexp @ v[keys, g, :]
                    m = m_new
                ok = l > 0
                O[rows[ok], h, :] = acc[ok] / l[ok, None]
                lse[h, rows[ok]] = m[ok] + np.log(l[ok])
    return {"O": O, "lse": lse, "visited": visited, "skipped": skipped,
            "skip_bits": bits, "margin": margin}
