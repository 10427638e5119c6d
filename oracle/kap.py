"""Kernel-Aware Proxy (KAP): from Q and K to a computation-order mask.

Follows the CoSA summary §2.2 ("Stage 1: Kernel-Aware Proxy") in the order the
page lists the steps: Block Ranking (downsample, approximate scores, MaxPool
over keys, MaxNorm), HRM Flag Generation, Flag-Grouped Sorting under a budget;
§2.1 defines the output as an order, not a binary mask.

Readings of steps the pages leave open (the plainest the text supports):

R1  Downsampling is the mean over p consecutive tokens, for Q and for K, per
    head; p divides the block size B; a ragged final window averages only the
    tokens that exist.
R2  "MaxPool over keys" acts on the pooled score matrix along the key axis,
    inside each KV block (B/p pooled keys -> one value): P[h, r, kb].
R3  Scores carry the attention softmax scale.
R4  Pooled causality: pooled key j is visible to pooled row r iff
    j*p <= off + min(r*p + p - 1, Lq - 1) (the diagonal pooled pair counts).
    P is -inf where no pooled key of the block is visible.
R5  MaxNorm divides each row's exp-scores by the row's largest exp-score:
    c = exp(P - rowmax(P)), a contribution in (0, 1].
R6  HRM: block kb is flagged for query block qb of KV group g when P attains
    the row maximum exactly for any pooled row of qb of any query head of g.
R7  Block score s[g, qb, kb] = sum of c over the group's heads (ascending) and
    the block's pooled rows (ascending), a sequential sum.
R8  One order per (sequence, KV head, query block), shared by the G query
    heads of the group (the intra-group union of the CompactAttention page,
    selection stage).
R9  Sort key: HRM first, then s descending, then kb ascending (a strict total
    order, so the result is unique).
R10 Sort, then keep the first k = clamp(ceil(beta*n - 1e-9), 1, n) entries of
    the n causal blocks; HRM blocks compete for the budget like the rest.

Two precisions:
* ``precision="fp64"``: everything in float64 with numpy's exp.
* ``precision="fp32"``: the bit-exact contract. Given fp32 proxy scores P,
  m, D = P - m, c = exp32(D), HRM = (D == 0) and the sequential fp32 sum s
  are each single rounded binary32 operations; the GPU must reproduce order,
  HRM flags and s bit for bit from the same P.
"""
from __future__ import annotations

import numpy as np

from .exp32 import exp32
from .layout import budget_count, cdiv, n_causal_blocks


def pool_tokens(x, p: int) -> np.ndarray:
    """R1: mean of x [L, H, d] over windows [r*p, min(r*p+p, L)) -> [ceil(L/p), H, d]."""
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[0]
    R = cdiv(L, p)
    out = np.empty((R,) + x.shape[1:])
    for r in range(R):
        lo, hi = r * p, min(r * p + p, L)
        out[r] = x[lo:hi].sum(axis=0) / (hi - lo)
    return out


def proxy_scores(qt, kt, scale: float, B: int, p: int, Lq: int, Lk: int) -> np.ndarray:
    """R2-R4: P[h, r, kb] = max over visible pooled keys j of block kb of
    scale * qt[r, h] . kt[j, h // G]  (fp64), -inf where none is visible."""
    qt = np.asarray(qt, dtype=np.float64)
    kt = np.asarray(kt, dtype=np.float64)
    R, Hq, _ = qt.shape
    Rk, Hkv, _ = kt.shape
    G = Hq // Hkv
    off = Lk - Lq
    Nk = cdiv(Lk, B)
    per = B // p
    r_last = np.minimum(np.arange(R) * p + p - 1, Lq - 1)
    vis = (np.arange(Rk)[None, :] * p) <= (off + r_last[:, None])
    P = np.empty((Hq, R, Nk))
    for h in range(Hq):
        s = scale * (qt[:, h, :] @ kt[:, h // G, :].T)
        s = np.where(vis, s, -np.inf)
        pad = np.full((R, Nk * per), -np.inf)
        pad[:, :Rk] = s
        P[h] = pad.reshape(R, Nk, per).max(axis=2)
    return P


def rank_row(P_rows, precision: str = "fp32"):
    """R5-R7 for one list row (b, g, qb).

    P_rows [G, nrow, nk]: the proxy scores of the group's query heads
    (ascending) for the pooled rows of qb (ascending), over the sequence's KV
    blocks. Returns (s [nk], hrm [nk])."""
    dt = np.float32 if precision == "fp32" else np.float64
    P_rows = np.asarray(P_rows, dtype=dt)
    with np.errstate(invalid="ignore"):
        m = P_rows.max(axis=2, keepdims=True)  # row max (exact in any precision)
        D = (P_rows - m).astype(dt)
        if precision == "fp32":
            c = exp32(D)
        else:
            c = np.nan_to_num(np.exp(D), nan=0.0)  # exp(-inf) = 0, NaN -> 0
    flag = D == 0
    nk = P_rows.shape[2]
    s = np.zeros(nk, dtype=dt)
    hrm = np.zeros(nk, dtype=bool)
    for h in range(P_rows.shape[0]):
        for r in range(P_rows.shape[1]):
            s = (s + c[h, r]).astype(dt)  # one rounded add per term, per block
            hrm |= flag[h, r]
    return s, hrm


def select_row(s, hrm, n: int, budget: float):
    """R9-R10 for one list row: sort the n causal blocks, keep k of them.
    Returns (order list, HRM flags of the listed blocks)."""
    ranked = sorted(range(n), key=lambda kb: (not hrm[kb], -s[kb], kb))
    k = budget_count(n, budget)
    return ranked[:k], [1 if hrm[kb] else 0 for kb in ranked[:k]]


def row_inputs(P, G: int, g: int, qb: int, B: int, p: int):
    """The slice of P [Hq, R, Nk] that list row (g, qb) ranks."""
    per = B // p
    R = P.shape[1]
    return P[g * G : (g + 1) * G, qb * per : min(qb * per + per, R), :]


def rank(P, G: int, B: int, p: int, Lq: int, precision: str = "fp32"):
    """R5-R8 over a whole sequence. P [Hq, R, Nk] -> (s, hrm) [Hkv, Nq, Nk]."""
    dt = np.float32 if precision == "fp32" else np.float64
    Hq, R, Nk = P.shape
    Hkv = Hq // G
    Nq = cdiv(Lq, B)
    s = np.zeros((Hkv, Nq, Nk), dtype=dt)
    hrm = np.zeros((Hkv, Nq, Nk), dtype=bool)
    for g in range(Hkv):
        for qb in range(Nq):
            s[g, qb], hrm[g, qb] = rank_row(row_inputs(P, G, g, qb, B, p), precision)
    return s, hrm


def select(s, hrm, B: int, Lq: int, Lk: int, budget: float, kmax: int):
    """R9-R10 over a whole sequence.

    Returns order [Hkv, Nq, kmax] int32 (-1 padded), hrm_sel [Hkv, Nq, kmax]
    uint8 and count [Hkv, Nq] int32."""
    Hkv, Nq, _ = s.shape
    order = np.full((Hkv, Nq, kmax), -1, dtype=np.int32)
    hsel = np.zeros((Hkv, Nq, kmax), dtype=np.uint8)
    count = np.zeros((Hkv, Nq), dtype=np.int32)
    for g in range(Hkv):
        for qb in range(Nq):
            n = n_causal_blocks(qb, B, Lq, Lk)
            lst, flags = select_row(s[g, qb], hrm[g, qb], n, budget)
            order[g, qb, : len(lst)] = lst
            hsel[g, qb, : len(lst)] = flags
            count[g, qb] = len(lst)
    return order, hsel, count


def kap_from_scores(P, G: int, B: int, p: int, Lq: int, Lk: int, budget: float,
                    kmax: int, precision: str = "fp32"):
    """Steps after the proxy scores, given P (parity mode when fp32)."""
    s, hrm = rank(P, G, B, p, Lq, precision)
    order, hsel, count = select(s, hrm, B, Lq, Lk, budget, kmax)
    return {"order": order, "hrm": hsel, "count": count, "s": s, "hrm_full": hrm}


def kap_sequence(q, k, scale: float, B: int, p: int, budget: float, kmax: int,
                 precision: str = "fp64"):
    """The whole proxy for one sequence: q [Lq, Hq, d], k [Lk, Hkv, d]."""
    Lq, Hq, _ = q.shape
    Lk, Hkv, _ = k.shape
    qt = pool_tokens(q, p)
    kt = pool_tokens(k, p)
    P = proxy_scores(qt, kt, scale, B, p, Lq, Lk)
    if precision == "fp32":
        P = P.astype(np.float32)
    out = kap_from_scores(P, Hq // Hkv, B, p, Lq, Lk, budget, kmax, precision)
    out["P"] = P
    out["q_pooled"] = qt
    out["k_pooled"] = kt
    return out
