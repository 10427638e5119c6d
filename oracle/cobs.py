"""Second-order block scores (COBS page) as an alternative proxy ranking
(test infrastructure only).

The COBS page expands the log attention mass of a block in cumulants,
ln m_b = ln L + q.k_mean + (1/2) q^T Sigma q + ..., and ranks blocks by the
first two terms, q.k_mean + (1/2) q^T Sigma q (its §2.2-2.3), where k_mean and
Sigma are the mean and covariance of the block's keys; its own selector stores
compressed statistics (low rank, a query subspace, fp4) for a single decode
query. The reading used here for prefill:

R31 For pooled query row r (R1) and KV block kb, with
    s_j = scale * q_pooled[r] . k_j over the raw keys j of the block that the
    row's window may see (j <= off + min(r*p + p - 1, Lq - 1), j < Lk):
        P2[h, r, kb] = mean_j s_j + 1/2 var_j s_j
    (population variance; -inf when no key is visible). With k_mean and Sigma
    the mean and covariance of those keys this is exactly
    scale q.k_mean + (scale^2 / 2) q^T Sigma q: the page's score with the
    exact per-block covariance, no compression. MaxNorm, HRM flags, the sort
    and the budget then run unchanged on P2 (R5-R10).
"""
from __future__ import annotations

import numpy as np

from .kap import pool_tokens
from .layout import cdiv


def cobs_scores(qt, k, scale: float, B: int, p: int, Lq: int, Lk: int) -> np.ndarray:
    """P2 [Hq, R, Nk] in fp64 from pooled queries qt [R, Hq, d] and raw keys k [Lk, Hkv, d]."""
    qt = np.asarray(qt, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    R, Hq, _ = qt.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    off = Lk - Lq
    Nk = cdiv(Lk, B)
    jmax = off + np.minimum(np.arange(R) * p + p - 1, Lq - 1)
    keys = np.arange(Lk)
    vis = keys[None, :] <= jmax[:, None]  # [R, Lk]
    P2 = np.full((Hq, R, Nk), -np.inf)
    for h in range(Hq):
        s = scale * (qt[:, h, :] @ k[:, h // G, :].T)  # [R, Lk]
        for kb in range(Nk):
            cols = slice(kb * B, min(kb * B + B, Lk))
            for r in range(R):
                x = s[r, cols][vis[r, cols]]
                if x.size:
                    mu = x.mean()
                    P2[h, r, kb] = mu + 0.5 * ((x - mu) ** 2).mean()
    return P2


def cobs_case(case) -> np.ndarray:
    """P2 over a packed batch in the library layout [batch, h_q, max_nr, max_nk] (-inf pad)."""
    from .cases import dims, sequence_inputs

    dm = dims(case)
    out = np.full((case.batch, case.h_q, dm["max_nr"], dm["max_nk"]), -np.inf)
    for b in range(case.batch):
        Lq, Lk = case.seqlens_q[b], int(case.seqlens_k[b])
        if Lq == 0:
            continue
        q, k, _ = sequence_inputs(case, b)
        qt = pool_tokens(q, case.pool)
        out[b, :, : qt.shape[0], : cdiv(Lk, case.block)] = cobs_scores(qt, k, case.scale, case.block, case.pool,
                                                                      Lq, Lk)
    return out
