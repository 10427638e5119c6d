"""Seeded synthetic inputs for the CoSA prefill path.

This module only draws random tensors and lays them out in memory. It holds
none of the attention, proxy or ordering arithmetic, so both the CPU oracle and
the HIP path can consume what it produces without sharing any of the method.

The shapes follow the long-context prefill workloads the CoSA pages evaluate
(4K-128K tokens, Llama-3-8B-style GQA heads of dimension 128). The pages
evaluate on RULER and LongBench-v2; neither dataset is used here: these
generators stand in for the context shapes only.

Recipes (all draws from ``torch.Generator`` on the CPU, float32 math, then a
round-to-nearest-even cast to the case's dtype):

* ``iid_case`` (tiny CPU-checkable case): Q, K, V iid N(0,1)/sqrt(d); a few
  planted keys set to ``planted_norm`` times the unit direction of a random
  later query row.
* ``lowrank_case`` (long-context cases): per KV head g a factor
  F_g ~ N(0, 1/16)^{rank x d}; K_g = Z F_g + 0.3 E and, per query head h of
  the group, Q_h = Z' F_g + 0.3 E' with Z, Z', E, E' ~ N(0,1); rotate-half RoPE
  (theta 500000) at the tokens' absolute positions; the first ``sinks`` keys of
  each sequence multiplied by ``sink_mult`` after RoPE; V ~ N(0,1). Optional
  "needle" blocks overwrite every key of a random KV block with
  4*kappa*u + 0.3*eps, where u is the unit direction of a random later query
  row of the group and kappa the RMS key norm (sinks excluded).
* aligned sinks (``sink_logit``, off in the named workloads): the sinks
  become keys every query of the group answers with a logit of about
  ``sink_logit`` nats. A tile can only be skipped in-kernel when every one of
  its rows sits far below its running max, which needs such a shared sink;
  without it, skips essentially never happen.

K and V are stored in KV-head-major pages ``[num_pages, h_kv, block, d]``;
``block_table[b, kb]`` names the page that holds logical KV block kb of
sequence b. Key slots past a sequence's end and spare pages are filled with
NaN, so a kernel that reads them poisons its output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

__all__ = ["Case", "iid_case", "lowrank_case", "config_case", "CONFIG_SEEDS"]

# Query component along the aligned-sink direction (see _lowrank_sequence).
SINK_QUERY = 4.0

# Seed per named workload (config N uses 1000 + N).
CONFIG_SEEDS = {1: 1001, 2: 1002, 3: 1003, 4: 1004, 5: 1005}


@dataclass
class Case:
    """One prefill problem: packed queries, paged K/V and the call parameters."""

    name: str
    q: torch.Tensor  # [total_q, h_q, d]
    k_pages: torch.Tensor  # [num_pages, h_kv, block, d]
    v_pages: torch.Tensor  # [num_pages, h_kv, block, d]
    block_table: torch.Tensor  # int32 [batch, max_blocks_k]
    cu_seqlens_q: torch.Tensor  # int32 [batch + 1]
    seqlens_k: torch.Tensor  # int32 [batch]
    h_q: int
    h_kv: int
    head_dim: int
    block: int
    pool: int
    budget: float
    tau: float
    dtype: str  # "f32" or "bf16"
    scale: float = 0.0
    meta: dict = field(default_factory=dict)

    def __post_init__(self):
        if self.scale == 0.0:
            self.scale = 1.0 / math.sqrt(self.head_dim)

    @property
    def batch(self) -> int:
        return int(self.seqlens_k.numel())

    @property
    def seqlens_q(self) -> List[int]:
        cu = self.cu_seqlens_q.tolist()
        return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]

    def kv_contiguous(self, b: int, which: str = "k") -> torch.Tensor:
        """Logical [Lk, h_kv, d] view of sequence b's keys or values (a copy)."""
        pages = self.k_pages if which == "k" else self.v_pages
        lk = int(self.seqlens_k[b])
        nb = -(-lk // self.block)
        idx = self.block_table[b, :nb].long()
        x = pages[idx]  # [nb, h_kv, B, d]
        x = x.permute(0, 2, 1, 3).reshape(nb * self.block, self.h_kv, self.head_dim)
        return x[:lk].clone()


def _torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def _rope(x: torch.Tensor, positions: torch.Tensor, theta: float) -> torch.Tensor:
    """Rotate-half rotary embedding of x [T, d] at integer positions [T]."""
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-(torch.arange(half, dtype=torch.float64) * 2.0 / d))
    ang = positions.to(torch.float64)[:, None] * inv[None, :]
    cos = torch.cos(ang).to(torch.float32)
    sin = torch.sin(ang).to(torch.float32)
    x1, x2 = x[:, :half], x[:, half:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=1)


def _page(
    k_seqs: List[torch.Tensor],
    v_seqs: List[torch.Tensor],
    block: int,
    dtype: torch.dtype,
    spare_pages: int,
    shuffle_seed: Optional[int],
):
    """Scatter per-sequence [Lk, h_kv, d] K/V into NaN-poisoned pages."""
    h_kv, d = k_seqs[0].shape[1], k_seqs[0].shape[2]
    nbs = [-(-k.shape[0] // block) for k in k_seqs]
    used = sum(nbs)
    total = used + spare_pages
    if shuffle_seed is not None:
        g = torch.Generator().manual_seed(shuffle_seed)
        perm = torch.randperm(total, generator=g)
    else:
        perm = torch.arange(total)
    kp = torch.full((total, h_kv, block, d), float("nan"), dtype=dtype)
    vp = torch.full((total, h_kv, block, d), float("nan"), dtype=dtype)
    max_nb = max(nbs)
    table = torch.zeros((len(k_seqs), max_nb), dtype=torch.int32)
    pos = 0
    for b, (k, v) in enumerate(zip(k_seqs, v_seqs)):
        lk = k.shape[0]
        for kb in range(nbs[b]):
            page = int(perm[pos])
            pos += 1
            table[b, kb] = page
            lo, hi = kb * block, min((kb + 1) * block, lk)
            kp[page, :, : hi - lo, :] = k[lo:hi].permute(1, 0, 2).to(dtype)
            vp[page, :, : hi - lo, :] = v[lo:hi].permute(1, 0, 2).to(dtype)
    return kp, vp, table


def iid_case(
    seed: int,
    seqlen: int = 1024,
    h_q: int = 1,
    h_kv: int = 1,
    head_dim: int = 64,
    block: int = 64,
    pool: int = 8,
    budget: float = 0.25,
    tau: float = math.exp(-16.0),
    dtype: str = "f32",
    planted: int = 4,
    planted_norm: float = 6.0,
    q_mult: float = 1.0,
    name: str = "iid",
) -> Case:
    """Tiny case: iid N(0,1)/sqrt(d) Q/K/V plus planted keys (one sequence)."""
    g = torch.Generator().manual_seed(seed)
    T, d = seqlen, head_dim
    s = 1.0 / math.sqrt(d)
    q = torch.randn((T, h_q, d), generator=g) * s
    k = torch.randn((T, h_kv, d), generator=g) * s
    v = torch.randn((T, h_kv, d), generator=g) * s
    if planted > 0:
        pos = torch.randperm(T, generator=g)[:planted].sort().values
        for t in pos.tolist():
            i = int(torch.randint(t, T, (1,), generator=g))
            for hk in range(h_kv):
                qi = q[i, hk * (h_q // h_kv)]
                k[t, hk] = planted_norm * qi / qi.norm()
    q = q * q_mult
    tdt = _torch_dtype(dtype)
    kp, vp, table = _page([k], [v], block, tdt, 0, None)
    return Case(
        name=name,
        q=q.to(tdt).contiguous(),
        k_pages=kp,
        v_pages=vp,
        block_table=table,
        cu_seqlens_q=torch.tensor([0, T], dtype=torch.int32),
        seqlens_k=torch.tensor([T], dtype=torch.int32),
        h_q=h_q,
        h_kv=h_kv,
        head_dim=d,
        block=block,
        pool=pool,
        budget=budget,
        tau=tau,
        dtype=dtype,
        meta={"seed": seed, "q_mult": q_mult},
    )


def _lowrank_sequence(
    g: torch.Generator,
    lq: int,
    lk: int,
    h_q: int,
    h_kv: int,
    d: int,
    rank: int,
    noise: float,
    theta: float,
    sinks: int,
    sink_mult: float,
    sink_logit=None,
):
    """One sequence's fp32 Q [lq, h_q, d], K and V [lk, h_kv, d] (post-RoPE).

    With ``sink_logit`` set, the sinks are aligned: each group draws a unit
    direction u in its four lowest-frequency rotary pairs; every query of the
    group has its component along u replaced by ``SINK_QUERY`` * u, and the
    first ``sinks`` keys are c*u + noise with c chosen so that the scaled
    logit of a query with a sink is about ``sink_logit`` nats (before the slow
    rotary decay). Without it, sinks are the first keys times ``sink_mult``.
    """
    grp = h_q // h_kv
    off = lk - lq
    pos_k = torch.arange(lk)
    pos_q = torch.arange(off, lk)
    q = torch.empty((lq, h_q, d))
    k = torch.empty((lk, h_kv, d))
    v = torch.empty((lk, h_kv, d))
    for gi in range(h_kv):
        f = torch.randn((rank, d), generator=g) * (1.0 / math.sqrt(rank))
        zk = torch.randn((lk, rank), generator=g)
        ek = torch.randn((lk, d), generator=g)
        kpre = zk @ f + noise * ek
        u = None
        if sink_logit is not None:
            half = d // 2
            idx = list(range(half - 4, half)) + list(range(d - 4, d))
            u = torch.zeros(d)
            u[idx] = torch.randn(8, generator=g)
            u = u / u.norm()
            c = sink_logit * math.sqrt(d) / SINK_QUERY
            kpre[:sinks] = c * u + noise * torch.randn((min(sinks, lk), d), generator=g)
        kg = _rope(kpre, pos_k, theta)
        if sink_logit is None:
            kg[:sinks] *= sink_mult
        k[:, gi] = kg
        for hi in range(grp):
            zq = torch.randn((lq, rank), generator=g)
            eq = torch.randn((lq, d), generator=g)
            qpre = zq @ f + noise * eq
            if u is not None:
                qpre = qpre - (qpre @ u)[:, None] * u[None, :] + SINK_QUERY * u[None, :]
            q[:, gi * grp + hi] = _rope(qpre, pos_q, theta)
        v[:, gi] = torch.randn((lk, d), generator=g)
    return q, k, v


def _plant_needles(
    g: torch.Generator,
    q: torch.Tensor,
    k: torch.Tensor,
    block: int,
    per_head: int,
    sinks: int,
    noise: float,
):
    """Overwrite `per_head` KV blocks per KV head with keys aligned to a later query."""
    lq, h_q, d = q.shape
    lk, h_kv, _ = k.shape
    off = lk - lq
    grp = h_q // h_kv
    nblk = -(-lk // block)
    planted = []
    for gi in range(h_kv):
        kappa = k[sinks:, gi].pow(2).sum(dim=1).mean().sqrt()
        cand = torch.randperm(max(nblk - 2, 0), generator=g)[:per_head] + 1
        for kb in cand.tolist():
            lo = max((kb + 1) * block - off, 0)
            if lo >= lq:
                continue
            i = int(torch.randint(lo, lq, (1,), generator=g))
            h = gi * grp + int(torch.randint(0, grp, (1,), generator=g))
            u = q[i, h] / q[i, h].norm()
            hi_t = min((kb + 1) * block, lk)
            eps = torch.randn((hi_t - kb * block, d), generator=g)
            k[kb * block : hi_t, gi] = 4.0 * kappa * u + noise * eps
            planted.append((gi, kb, i, h))
    return planted


def lowrank_case(
    seed: int,
    seqlens_q: List[int],
    seqlens_k: Optional[List[int]] = None,
    h_q: int = 32,
    h_kv: int = 8,
    head_dim: int = 128,
    block: int = 128,
    pool: int = 16,
    budget: float = 0.1,
    tau: float = math.exp(-16.0),
    dtype: str = "bf16",
    rank: int = 16,
    noise: float = 0.3,
    theta: float = 500000.0,
    sinks: int = 4,
    sink_mult: float = 8.0,
    needles_per_head: int = 0,
    sink_logit=None,
    spare_pages: int = 0,
    shuffle_pages: bool = False,
    per_sequence_seeds: bool = False,
    name: str = "lowrank",
) -> Case:
    """Long-context case: rank-16 factors + noise, RoPE, sinks, optional needles."""
    if seqlens_k is None:
        seqlens_k = list(seqlens_q)
    tdt = _torch_dtype(dtype)
    qs, ks, vs = [], [], []
    needles = []
    base = torch.Generator().manual_seed(seed)
    for b, (lq, lk) in enumerate(zip(seqlens_q, seqlens_k)):
        g = torch.Generator().manual_seed(seed + 10 + b) if per_sequence_seeds else base
        q, k, v = _lowrank_sequence(
            g, lq, lk, h_q, h_kv, head_dim, rank, noise, theta, sinks, sink_mult, sink_logit
        )
        if needles_per_head > 0:
            gn = torch.Generator().manual_seed(seed + 1 + 100 * b)
            needles += [(b,) + t for t in _plant_needles(gn, q, k, block, needles_per_head, sinks, noise)]
        qs.append(q.to(tdt))
        ks.append(k)
        vs.append(v)
    kp, vp, table = _page(
        ks, vs, block, tdt, spare_pages, (seed + 3) if shuffle_pages else None
    )
    cu = [0]
    for lq in seqlens_q:
        cu.append(cu[-1] + lq)
    return Case(
        name=name,
        q=torch.cat(qs, dim=0).contiguous(),
        k_pages=kp,
        v_pages=vp,
        block_table=table,
        cu_seqlens_q=torch.tensor(cu, dtype=torch.int32),
        seqlens_k=torch.tensor(seqlens_k, dtype=torch.int32),
        h_q=h_q,
        h_kv=h_kv,
        head_dim=head_dim,
        block=block,
        pool=pool,
        budget=budget,
        tau=tau,
        dtype=dtype,
        meta={"seed": seed, "needles": needles, "sink_logit": sink_logit},
    )


def ragged_lengths(seed: int, n: int, lo: int, hi: int) -> List[int]:
    """n sequence lengths uniform in [lo, hi] (inclusive), seeded."""
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, (n,), generator=g).tolist()


def config_case(n: int, scale_down: int = 1, budget: Optional[float] = None, **kw) -> Case:
    """The five named workloads; ``scale_down`` shrinks sequence lengths for tests.

    1: tiny iid fp32 prefill, T=1024, d=64, block 64, pool 8, budget 25%.
    2: Llama-3-8B-shaped layer, T=32768, 32/8 heads, d=128, bf16, block 128,
       pool 16, budget 10%.
    3: as 2 at T=131072 with 32 needle blocks per KV head, budget 10%
       (5% and 25% are the sweep).
    4: chunked prefill, a 4096-token chunk against 65536 cached tokens held in
       a shuffled pool of 640 pages (128 spare, NaN-filled), budget 10%.
    5: ragged batch of 8 sequences, lengths uniform in [4096, 32768],
       64/8 heads (GQA 8), budget 10% (5%, 25%, 100% are the sweep).
    """
    seed = CONFIG_SEEDS[n]
    sd = max(1, int(scale_down))
    if n == 1:
        c = iid_case(seed, seqlen=1024 // sd, name="cfg1", **kw)
    elif n == 2:
        c = lowrank_case(seed, [32768 // sd], name="cfg2", **kw)
    elif n == 3:
        c = lowrank_case(seed, [131072 // sd], needles_per_head=32, name="cfg3", **kw)
    elif n == 4:
        lk = 65536 // sd
        lq = 4096 // sd
        kw.setdefault("spare_pages", 128 // sd)
        c = lowrank_case(
            seed, [lq], [lk], shuffle_pages=True, name="cfg4", **kw
        )
    elif n == 5:
        lens = ragged_lengths(seed + 2, 8, 4096 // sd, 32768 // sd)
        kw.setdefault("h_q", 64)
        c = lowrank_case(seed, lens, per_sequence_seeds=True, name="cfg5", **kw)
    else:
        raise ValueError(f"unknown workload {n}")
    if budget is not None:
        c.budget = budget
    return c
