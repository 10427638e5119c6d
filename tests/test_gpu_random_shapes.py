"""GPU parity over seeded random shapes (through the C ABI).

Each case draws block size, head dim, pool, KV-head count (including counts
that are not a multiple of the attention walk's four-group launch phases),
GQA group, a ragged batch with chunked offsets, budget and optionally aligned
sinks, then checks the proxy's lists bit-exact against the oracle fed the
GPU's fp32 proxy scores, the ordered walk (output, visited and skip sets) and
the dense kernel against the fp64 oracle, to the same bars as the fixed cases.
Decode cases draw contexts up to 9000 tokens, sequences without a new token
and a segment count of 1 to 8, and check the split walk against the oracle's.
"""
import random

import numpy as np
import pytest
import torch

import block_sparse_attention_26_amd as cosa
import synthetic
from oracle import cases as oc, decode as odec
from gpu_common import AMBIGUOUS_NATS, OnDevice, check_output, check_skip_sets, require_gpu, say

pytestmark = pytest.mark.gpu

N_CASES = 16
N_DECODE = 8


def _draw(i):
    rng = random.Random(5000 + i)
    B = rng.choice([64, 128])
    d = rng.choice([64, 128])
    p = rng.choice([4, 8, 16, 32, B])
    hkv = rng.choice([1, 2, 3, 5, 6, 7, 9])
    G = rng.choice([1, 2, 3, 4, 8])
    nseq = rng.choice([1, 1, 2, 3])
    lq = [rng.randint(1, 1400) for _ in range(nseq)]
    lk = [q + rng.choice([0, 0, rng.randint(1, 1500)]) for q in lq]
    budget = rng.choice([0.1, 0.25, 0.5])
    sink = rng.choice([None, None, 24.0])
    return dict(B=B, d=d, p=p, hkv=hkv, G=G, lq=lq, lk=lk, budget=budget, sink=sink)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_parity(i):
    require_gpu()
    c = _draw(i)
    say("random case", i, c)
    kw = {} if c["sink"] is None else {"sink_logit": c["sink"]}
    case = synthetic.lowrank_case(7000 + i, c["lq"], c["lk"], h_q=c["G"] * c["hkv"], h_kv=c["hkv"],
                                  head_dim=c["d"], block=c["B"], pool=c["p"], budget=c["budget"],
                                  per_sequence_seeds=True, name=f"random{i}", **kw)
    dev = OnDevice(case)
    tag = f"random case {i} {c}"

    k = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, case.budget, export_scores=True)
    torch.cuda.synchronize()
    ref = oc.kap_case(case, precision="fp32", P_given=k["P"].cpu().numpy())
    for name in ("order", "hrm", "count"):
        np.testing.assert_array_equal(k[name].cpu().numpy(), ref[name], err_msg=f"{tag}: {name}")

    ko = oc.kap_case(case)
    order = torch.from_numpy(ko["order"]).cuda()
    count = torch.from_numpy(ko["count"]).cuda()
    g = cosa.osk_attention(dev.problem, dev.q, dev.k, dev.v, order, count, case.tau, skip_bits=True)
    torch.cuda.synchronize()
    r = oc.osk_case(case, ko["order"], ko["count"])
    check_output(g["O"], r["O"], case.dtype, tag)
    check_skip_sets(g, r, ko["count"], c["G"])

    gd = cosa.dense_attention(dev.problem, dev.q, dev.k, dev.v)
    torch.cuda.synchronize()
    check_output(gd["O"], oc.dense_case(case)["O"], case.dtype, tag + " dense")


def _draw_decode(i):
    rng = random.Random(6000 + i)
    B = rng.choice([64, 128])
    d = rng.choice([64, 128])
    p = rng.choice([4, 8, 16, 32])
    hkv = rng.choice([1, 2, 3, 5])
    G = rng.choice([1, 2, 4, 8])
    nseq = rng.choice([1, 2, 3, 4])
    lk = [rng.randint(1, 9000) for _ in range(nseq)]
    lq = [1 if rng.random() > 0.15 else 0 for _ in range(nseq)]
    if sum(lq) == 0:
        lq[0] = 1
    budget = rng.choice([0.1, 0.25, 0.5])
    sink = rng.choice([None, 24.0])
    S = rng.randint(1, 8)
    return dict(B=B, d=d, p=p, hkv=hkv, G=G, lq=lq, lk=lk, budget=budget, sink=sink, S=S)


@pytest.mark.parametrize("i", range(N_DECODE))
def test_random_decode_parity(i):
    require_gpu()
    c = _draw_decode(i)
    say("random decode case", i, c)
    kw = {} if c["sink"] is None else {"sink_logit": c["sink"]}
    case = synthetic.lowrank_case(8000 + i, c["lq"], c["lk"], h_q=c["G"] * c["hkv"], h_kv=c["hkv"],
                                  head_dim=c["d"], block=c["B"], pool=c["p"], budget=c["budget"],
                                  per_sequence_seeds=True, name=f"random-decode{i}", **kw)
    dev = OnDevice(case)
    tag = f"random decode case {i} {c}"

    k = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, case.budget, export_scores=True)
    torch.cuda.synchronize()
    ref = oc.kap_case(case, precision="fp32", P_given=k["P"].cpu().numpy())
    for name in ("order", "hrm", "count"):
        np.testing.assert_array_equal(k[name].cpu().numpy(), ref[name], err_msg=f"{tag}: {name}")

    ko = oc.kap_case(case)
    order = torch.from_numpy(ko["order"]).cuda()
    count = torch.from_numpy(ko["count"]).cuda()
    g = cosa.osk_decode(dev.problem, dev.q, dev.k, dev.v, order, count, case.tau, c["S"])
    torch.cuda.synchronize()
    r = odec.decode_case(case, ko["order"], ko["count"], c["S"])
    check_output(g["O"], r["O"], case.dtype, tag)
    np.testing.assert_array_equal(g["visited"].cpu().numpy()[:, :, 0], r["visited"])
    clear = ~(np.abs(r["margin"]) < AMBIGUOUS_NATS).any(axis=2)
    np.testing.assert_array_equal(g["skipped"].cpu().numpy()[:, :, 0][clear], r["skipped"][clear])
