"""Strided query and output tensors through the C ABI.

The library reads q and writes o through element strides per token and per
head (zero-copy access to the caller's tensors, CompactAttention page,
execution stage), so a query slice of a fused QKV projection or a heads-major
layout needs no copy. Every entry point that reads q or writes o must give,
for such views, exactly the bits it gives for the contiguous tensors: the
kernels do the same arithmetic, only the addresses differ.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_26_amd as cosa
import synthetic
from gpu_common import OnDevice, require_gpu, say

pytestmark = pytest.mark.gpu


def _views(q):
    """(fused-QKV slice, heads-major) views holding q's values."""
    T, Hq, D = q.shape
    h_kv = 2
    qkv = torch.full((T, Hq + 2 * h_kv, D), float("nan"), dtype=q.dtype, device=q.device)
    qkv[:, :Hq] = q
    fused = qkv[:, :Hq]                                   # strides ((Hq + 2 h_kv) D, D, 1)
    heads_major = q.permute(1, 0, 2).contiguous().permute(1, 0, 2)  # strides (D, T D, 1)
    assert not fused.is_contiguous() and not heads_major.is_contiguous()
    return {"fused": fused, "heads-major": heads_major}


def _heads_major_out(q):
    T, Hq, D = q.shape
    return torch.full((Hq, T, D), float("nan"), dtype=q.dtype, device=q.device).permute(1, 0, 2)


def _same(a, b, what):
    assert a.shape == b.shape, what
    x = a.contiguous().view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32)
    y = b.contiguous().view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
    assert torch.equal(x, y), what


CASES = {
    "bf16-gqa4-varlen": lambda: synthetic.lowrank_case(91, [700, 1300], [900, 1300], h_q=8, h_kv=2, head_dim=128,
                                                       block=128, pool=16, budget=0.3, sink_logit=24.0,
                                                       per_sequence_seeds=True, spare_pages=3,
                                                       shuffle_pages=True, name="bf16-gqa4-varlen"),
    "bf16-d64-b64": lambda: synthetic.lowrank_case(92, [1000], h_q=4, h_kv=2, head_dim=64, block=64, pool=8,
                                                   budget=0.3, name="bf16-d64-b64"),
    "f32-tiny": lambda: synthetic.lowrank_case(93, [600], h_q=2, h_kv=2, head_dim=64, block=64, pool=8,
                                               budget=0.3, dtype="f32", name="f32-tiny"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_strided_q_and_o(name):
    require_gpu()
    case = CASES[name]()
    dev = OnDevice(case)
    pr = dev.problem
    say(name, "contiguous reference")
    k0 = cosa.kap_order(pr, dev.q, dev.k, case.pool, case.budget, export_scores=True)
    o0 = cosa.osk_attention(pr, dev.q, dev.k, dev.v, k0["order"], k0["count"], case.tau, skip_bits=True, lse=True)
    d0 = cosa.dense_attention(pr, dev.q, dev.k, dev.v, lse=True)
    for vname, qv in _views(dev.q).items():
        say(name, "q view", vname, tuple(qv.stride()))
        k1 = cosa.kap_order(pr, qv, dev.k, case.pool, case.budget, export_scores=True)
        for f in ("order", "hrm", "count", "P"):
            assert torch.equal(k1[f], k0[f]), (vname, f)
        for out in (None, _heads_major_out(dev.q)):
            o1 = cosa.osk_attention(pr, qv, dev.k, dev.v, k0["order"], k0["count"], case.tau, skip_bits=True,
                                    lse=True, out=out)
            _same(o1["O"], o0["O"], (vname, "walk O"))
            for f in ("visited", "skipped", "skip_bits", "lse"):
                assert torch.equal(o1[f], o0[f]), (vname, f)
            d1 = cosa.dense_attention(pr, qv, dev.k, dev.v, lse=True, out=out)
            _same(d1["O"], d0["O"], (vname, "dense O"))
            assert torch.equal(d1["lse"], d0["lse"]), vname
    torch.cuda.synchronize()
    if case.dtype == "bf16":
        say(name, "block mass and second-order scores on a fused-QKV slice")
        qv = _views(dev.q)["fused"]
        _same(cosa.block_mass(pr, qv, dev.k, d0["lse"]), cosa.block_mass(pr, dev.q, dev.k, d0["lse"]), "mass")
        _same(cosa.cobs_scores(pr, qv, dev.k, case.pool), cosa.cobs_scores(pr, dev.q, dev.k, case.pool), "cobs")
        mask = cosa.mask_from_order(pr, k0["order"], k0["count"])
        m0 = cosa.osk_attention_masked(pr, dev.q, dev.k, dev.v, mask, case.tau)
        m1 = cosa.osk_attention_masked(pr, qv, dev.k, dev.v, mask, case.tau, out=_heads_major_out(dev.q))
        _same(m1["O"], m0["O"], "mask walk O")


def test_decode_strided_q_and_o():
    require_gpu()
    case = synthetic.lowrank_case(94, [1, 1, 1], [3000, 5000, 777], h_q=8, h_kv=2, head_dim=128, block=128,
                                  pool=16, budget=0.2, per_sequence_seeds=True, spare_pages=2,
                                  shuffle_pages=True, name="decode-strided")
    dev = OnDevice(case)
    pr = dev.problem
    say("decode", "contiguous reference")
    k0 = cosa.kap_order(pr, dev.q, dev.k, case.pool, case.budget)
    g0 = cosa.osk_decode(pr, dev.q, dev.k, dev.v, k0["order"], k0["count"], case.tau, 3, lse=True)
    for vname, qv in _views(dev.q).items():
        say("decode", "q view", vname)
        k1 = cosa.kap_order(pr, qv, dev.k, case.pool, case.budget)
        for f in ("order", "hrm", "count"):
            assert torch.equal(k1[f], k0[f]), (vname, f)
        g1 = cosa.osk_decode(pr, qv, dev.k, dev.v, k0["order"], k0["count"], case.tau, 3, lse=True,
                             out=_heads_major_out(dev.q))
        _same(g1["O"], g0["O"], (vname, "decode O"))
        for f in ("visited", "skipped", "lse"):
            assert torch.equal(g1[f], g0[f]), (vname, f)
    torch.cuda.synchronize()
