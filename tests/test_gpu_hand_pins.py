"""The rank pass on the GPU against hand-derived expectations.

The hand-worked proxy examples under ``tests/golden/`` use tiny blocks; the
library's blocks are 64 or 128 tokens. Each example is carried over to a
problem with the same number of pooled rows per query block, causal blocks per
row and visibility pattern (block 64, with the pool factor chosen so that B/p
and the chunk offset in pooled rows match), and its proxy scores P are fed to
``cosa_kap_rank`` directly. The lists, HRM flags, counts and, where the hand
derivation fixes them, the bits of the block scores must come out as derived
(CoSA summary §2.2: MaxNorm, HRM flags, flag-grouped sort, budget).
"""
import json
import os

import numpy as np
import pytest
import torch

import block_sparse_attention_26_amd as cosa
from gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _problem(lq, lk, h_q, h_kv, block=64):
    require_gpu()
    nb = -(-lk // block)
    dev = torch.device("cuda")
    return cosa.Problem(h_q=h_q, h_kv=h_kv, head_dim=128, block=block, dtype=cosa.COSA_BF16,
                        softmax_scale=1.0, num_pages=nb,
                        cu_seqlens_q=torch.tensor([0, lq], dtype=torch.int32, device=dev),
                        seqlens_k=torch.tensor([lk], dtype=torch.int32, device=dev),
                        block_table=torch.arange(nb, dtype=torch.int32, device=dev)[None],
                        host_cu_seqlens_q=[0, lq], host_seqlens_k=[lk])


def _rank(pr, P, pool, budget):
    scores = torch.from_numpy(np.ascontiguousarray(P[None].astype(np.float32))).cuda()
    out = cosa.kap_rank(pr, scores, pool, budget, export_block_scores=True)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in out.items()}


def _bits(x):
    return [f"0x{int(v):08x}" for v in np.asarray(x, dtype=np.float32).view(np.uint32)]


def _sum_order_P(ex_, part):
    d24 = np.array([int(ex_["D24_bits"], 16)], dtype=np.uint32).view(np.float32)[0]
    tok = {"0": np.float32(0.0), "-100": np.float32(-100.0), "-inf": np.float32(-np.inf), "D24": d24}
    return np.array([[[tok[x] for x in row] for row in head] for head in part["P"]], dtype=np.float32)


def test_rank_sum_order_bits():
    """Sequential fp32 block-score sums (heads outer, rows inner): the hand
    bits of both parts of the sum-order example."""
    ex_ = _load("kap_sum_order_hand_example.json")
    say("hand pin", "sum order, part A")
    # part A: 2 pooled rows per query block, chunk offset of one block, 3 KV blocks
    pr = _problem(128, 192, 2, 1)
    out = _rank(pr, _sum_order_P(ex_, ex_), 32, 1.0)
    want = ex_["expected"]
    assert _bits(out["s"][0, 0, 1]) == want["s_qb1_bits"]
    assert _bits(out["s"][0, 0, 0]) == want["s_qb0_bits"]
    assert out["order"][0, 0].tolist() == want["order"]
    assert out["hrm"][0, 0].tolist() == want["hrm"]
    assert out["count"][0, 0].tolist() == want["count"]
    say("hand pin", "sum order, part B")
    pb = ex_["part_b"]
    pr = _problem(64, 128, 2, 1)
    out = _rank(pr, _sum_order_P(ex_, pb), 16, 1.0)
    assert _bits(out["s"][0, 0, 0]) == pb["expected"]["s_bits"]
    assert out["order"][0, 0, 0].tolist() == pb["expected"]["order"]
    assert out["hrm"][0, 0, 0].tolist() == pb["expected"]["hrm"]
    assert out["count"][0, 0, 0] == pb["expected"]["count"]


def test_rank_tie_break():
    """Exactly tied block scores are listed by ascending block index."""
    ex_ = _load("kap_tie_break_hand_example.json")
    say("hand pin", "tie break")
    # one pooled row per query block (pool = block), 4 query and 4 KV blocks;
    # P[r, kb] = max of the block's one pooled key 0, 1, 1, 3 where visible
    keys = [0.0, 1.0, 1.0, 3.0]
    P = np.full((1, 4, 4), -np.inf, dtype=np.float32)
    for r in range(4):
        for kb in range(r + 1):
            P[0, r, kb] = keys[kb]
    pr = _problem(256, 256, 1, 1)
    for budget, want in ex_["expected"].items():
        out = _rank(pr, P, 64, float(budget))
        k = len(want["qb3"])
        assert out["order"][0, 0, 3, :k].tolist() == want["qb3"]
        assert out["hrm"][0, 0, 3, :k].tolist() == want["qb3_hrm"]
        assert out["s"][0, 0, 3, 1] == out["s"][0, 0, 3, 2]
        if "qb2" in want:
            assert out["order"][0, 0, 2, :3].tolist() == want["qb2"]
            assert out["hrm"][0, 0, 2, :3].tolist() == want["qb2_hrm"]


def test_rank_chunk_offset():
    """The chunked-offset example's proxy scores (3 pooled rows, offset of
    3.5 pooled rows) give the hand order for both query blocks."""
    ex_ = _load("kap_chunk_offset_hand_example.json")
    say("hand pin", "chunk offset")
    P = np.array(ex_["expected"]["P"], dtype=np.float32)[None]
    # Lq = 80, Lk = 192, pool 32: pooled windows [0,32), [32,64), [64,80), off = 112
    pr = _problem(80, 192, 1, 1)
    out = _rank(pr, P, 32, 1.0)
    for qb in range(2):
        assert out["count"][0, 0, qb] == 3
        assert out["order"][0, 0, qb].tolist() == ex_["expected"]["order"][qb]
        assert out["hrm"][0, 0, qb].tolist() == ex_["expected"]["hrm"][qb]
    assert np.allclose(out["s"][0, 0, 0], ex_["expected"]["s_qb0"], rtol=0, atol=1e-6)
    assert np.allclose(out["s"][0, 0, 1], ex_["expected"]["s_qb1"], rtol=0, atol=1e-6)
