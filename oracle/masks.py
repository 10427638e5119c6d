"""Binary block masks, block-union tables and exact attention mass (test
infrastructure only).

The CoSA summary contrasts its computation-order list with the binary masks
of earlier proxies (§2.1, "Computation-Order Mask"; §1, proxy-driven methods)
and its page-remapped walk with the control-flow skipping of standard sparse
kernels (§2.3, "Mask-Skipped"); its ablation (§4) separates ordered
selection, in-kernel skipping and remapping. The COBS page describes an
oracle selector that keeps the blocks holding the most exact attention mass
(its "Oracle Sparse Attention"), an upper bound for any proxy at the same
budget.

Readings:

R24 The mask of a list is the set of its listed causal blocks; the visit
    order is dropped. Entries that are not causal blocks of the row are
    ignored.
R25 The list of a mask is its selected causal blocks in ascending kb (the
    order a fixed-order kernel visits them in), truncated to kmax entries.
    Without a mask every causal block is selected.
R26 Exact block mass of (head h, query block qb, KV block kb): the dense
    causal softmax probabilities of the valid rows of qb summed over the
    visible keys of kb. The mass of a KV group sums its query heads. Each row
    contributes 1 in total, so a group row's masses add to G x (valid rows).
R27 Recall of a selection for row (g, qb): its share of the row's group
    mass. The oracle selector at the same list length k keeps the k blocks of
    largest mass, so its recall bounds every selection of k blocks.
R29 Block union (CompactAttention page, selection stage): the per-group lists
    are already a union over the group's query heads; the Q-block union joins
    the lists of all query blocks of a sequence into one table per (sequence,
    KV group). Execution (the same page, zero-copy paged attention) walks the
    table for every query block, each block cut to what is causal for it, in
    ascending order.
"""
from __future__ import annotations

import numpy as np

from .layout import cdiv


def mask_from_order(order, count, n_causal, max_nk: int) -> np.ndarray:
    """Boolean mask [..., max_nk] of the listed causal blocks (R24).

    order [..., kmax] int, count [...] int, n_causal [...] int (0 for rows
    past a sequence's end)."""
    order = np.asarray(order)
    lead = order.shape[:-1]
    kmax = order.shape[-1]
    mask = np.zeros(lead + (max_nk,), dtype=bool)
    for idx in np.ndindex(*lead):
        n = int(n_causal[idx])
        c = max(0, min(int(count[idx]), kmax))
        for t in range(c):
            kb = int(order[idx + (t,)])
            if 0 <= kb < n:
                mask[idx + (kb,)] = True
    return mask


def order_from_mask(mask, n_causal, kmax: int):
    """Ascending lists of the selected causal blocks (R25); mask None selects
    every causal block. Returns (order [..., kmax] int32 with -1 pad, count)."""
    n_causal = np.asarray(n_causal)
    lead = n_causal.shape
    order = np.full(lead + (kmax,), -1, dtype=np.int32)
    count = np.zeros(lead, dtype=np.int32)
    for idx in np.ndindex(*lead):
        n = int(n_causal[idx])
        sel = [kb for kb in range(n) if mask is None or mask[idx + (kb,)]]
        sel = sel[:kmax]
        order[idx + (slice(0, len(sel)),)] = sel
        count[idx] = len(sel)
    return order, count


def union_lists(order, count, n_causal, kmax_out: int):
    """Block-union lists (R29): for every (sequence, KV group) the union of the
    causal blocks listed by its query blocks; each query block gets the union's
    blocks that are causal for it, ascending, truncated to kmax_out.

    order [batch, h_kv, nq, kmax], count / n_causal [batch, h_kv, nq].
    Returns (order [batch, h_kv, nq, kmax_out] int32 with -1 pad, count)."""
    order = np.asarray(order)
    nb, hkv, nq, kmax = order.shape
    out = np.full((nb, hkv, nq, kmax_out), -1, dtype=np.int32)
    cnt = np.zeros((nb, hkv, nq), dtype=np.int32)
    for b in range(nb):
        for g in range(hkv):
            union = set()
            for qb in range(nq):
                n = int(n_causal[b, g, qb])
                c = max(0, min(int(count[b, g, qb]), kmax))
                union.update(int(kb) for kb in order[b, g, qb, :c] if 0 <= kb < n)
            for qb in range(nq):
                n = int(n_causal[b, g, qb])
                sel = sorted(kb for kb in union if kb < n)[:kmax_out]
                out[b, g, qb, : len(sel)] = sel
                cnt[b, g, qb] = len(sel)
    return out, cnt


def pack_words(mask, mask_words: int) -> np.ndarray:
    """Boolean [..., n] -> uint64 words [..., mask_words]: bit i of word w is
    block 64 w + i."""
    mask = np.asarray(mask, dtype=bool)
    words = np.zeros(mask.shape[:-1] + (mask_words,), dtype=np.uint64)
    for kb in range(mask.shape[-1]):
        words[..., kb // 64] |= mask[..., kb].astype(np.uint64) << np.uint64(kb % 64)
    return words


def unpack_words(words, n: int) -> np.ndarray:
    """uint64 words [..., mask_words] -> boolean [..., n]."""
    words = np.asarray(words, dtype=np.uint64)
    out = np.zeros(words.shape[:-1] + (n,), dtype=bool)
    for kb in range(n):
        out[..., kb] = ((words[..., kb // 64] >> np.uint64(kb % 64)) & np.uint64(1)) == 1
    return out


def block_mass_sequence(q, k, scale: float, G: int, B: int) -> np.ndarray:
    """Exact block mass (R26) of one sequence in fp64.

    q [Lq, Hq, d], k [Lk, Hkv, d] -> M [Hq, Nq, Nk]; non-causal blocks 0."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    Lq, Hq, _ = q.shape
    Lk = k.shape[0]
    off = Lk - Lq
    Nq, Nk = cdiv(Lq, B), cdiv(Lk, B)
    M = np.zeros((Hq, Nq, Nk))
    pos = np.arange(Lq) + off
    keys = np.arange(Lk)
    for h in range(Hq):
        s = scale * (q[:, h, :] @ k[:, h // G, :].T)  # [Lq, Lk]
        vis = keys[None, :] <= pos[:, None]
        s = np.where(vis, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        for qb in range(Nq):
            rows = slice(qb * B, min(qb * B + B, Lq))
            col = p[rows].sum(axis=0)  # mass of each key over the query block's rows
            for kb in range(Nk):
                M[h, qb, kb] = col[kb * B : min(kb * B + B, Lk)].sum()
    return M


def recall(M_group, order, count) -> np.ndarray:
    """Share of each row's group mass held by its listed blocks (R27).

    M_group [..., Nk], order [..., kmax], count [...] -> [...] (nan for rows
    with no mass)."""
    M_group = np.asarray(M_group, dtype=np.float64)
    lead = M_group.shape[:-1]
    out = np.full(lead, np.nan)
    for idx in np.ndindex(*lead):
        tot = M_group[idx].sum()
        if tot <= 0:
            continue
        c = int(count[idx])
        sel = [int(x) for x in order[idx + (slice(0, c),)]]
        out[idx] = M_group[idx][sel].sum() / tot
    return out


def oracle_recall(M_group, k) -> np.ndarray:
    """Recall of the k largest-mass blocks of each row (R27); k [...] int."""
    M_group = np.asarray(M_group, dtype=np.float64)
    lead = M_group.shape[:-1]
    out = np.full(lead, np.nan)
    for idx in np.ndindex(*lead):
        tot = M_group[idx].sum()
        if tot <= 0:
            continue
        top = np.sort(M_group[idx])[::-1][: int(k[idx])]
        out[idx] = top.sum() / tot
    return out
