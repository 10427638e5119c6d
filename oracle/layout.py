"""Causal block arithmetic and page gathering for the oracle.

Readings (the CoSA pages define none of this):

* Chunked-prefill positions (CompactAttention page, problem statement: chunks
  attend to the accumulated KV cache): a sequence has Lq queries and Lk >= Lq
  keys; local query i sits at absolute position off + i with off = Lk - Lq,
  and sees key j iff j <= off + i.
* Blocks: query block qb holds local rows [qb*B, min(qb*B+B, Lq)); KV block kb
  holds keys [kb*B, min(kb*B+B, Lk)). kb is causal for qb iff some valid row
  of qb sees its first key, i.e. kb*B <= off + last_row(qb).
* Budget: a row keeps k = clamp(ceil(beta*n - 1e-9), 1, n) of its n causal
  blocks, evaluated in IEEE double (the 1e-9 absorbs the binary rounding of
  decimal budgets such as 0.1).
"""
from __future__ import annotations

import math

import numpy as np


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def last_row(qb: int, B: int, Lq: int) -> int:
    return min(qb * B + B - 1, Lq - 1)


def n_causal_blocks(qb: int, B: int, Lq: int, Lk: int) -> int:
    """Number of KV blocks causal for query block qb (they are kb = 0..n-1)."""
    off = Lk - Lq
    return (off + last_row(qb, B, Lq)) // B + 1


def budget_count(n: int, budget: float) -> int:
    """Blocks a row of n causal blocks keeps under budget beta in (0, 1]."""
    k = math.ceil(float(budget) * n - 1e-9)
    return max(1, min(n, k))


def kmax(B: int, seqlens_q, seqlens_k, budget: float) -> int:
    """Widest order list over all rows of all sequences."""
    best = 1
    for Lq, Lk in zip(seqlens_q, seqlens_k):
        if Lq == 0:
            continue
        nq = cdiv(Lq, B)
        best = max(best, budget_count(n_causal_blocks(nq - 1, B, Lq, Lk), budget))
    return best


def gather_pages(pages: np.ndarray, table_row: np.ndarray, Lk: int) -> np.ndarray:
    """[num_pages, h_kv, B, d] pages + one block-table row -> [Lk, h_kv, d]."""
    B = pages.shape[2]
    nb = cdiv(Lk, B)
    x = pages[np.asarray(table_row[:nb], dtype=np.int64)]  # [nb, h_kv, B, d]
    x = np.transpose(x, (0, 2, 1, 3)).reshape(nb * B, pages.shape[1], pages.shape[3])
    return np.ascontiguousarray(x[:Lk])
