"""GPU parity of the second-order block scores and of the rank pass over given
scores, through the C ABI.

* second-order scores: the pattern of -inf entries identical to the fp64
  oracle's, finite entries within 1e-2 of the largest magnitude (pooled
  queries are rounded to bf16 on the GPU, as for the max-pooled scores);
* rank pass over the GPU's second-order scores: order, HRM flags, counts and
  block scores bit-exact against the oracle fed the same fp32 scores;
* rank pass over the max-pooled scores exported by cosa_kap_order: the same
  lists as the fused proxy, bit for bit.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_26_amd as cosa
import synthetic
from oracle import cases as oc, cobs as ocobs
from gpu_common import OnDevice, require_gpu, say

pytestmark = pytest.mark.gpu


def _lr(name, seed, lq, lk=None, hq=8, hkv=2, d=128, B=128, p=16, budget=0.25, **kw):
    return lambda: synthetic.lowrank_case(seed, lq, lk, h_q=hq, h_kv=hkv, head_dim=d, block=B, pool=p,
                                          budget=budget, name=name, **kw)


CASES = {
    "gqa4-ragged": _lr("gqa4-ragged", 61, [2000]),
    "chunk-paged": _lr("chunk-paged", 62, [1000], [8192], budget=0.1, spare_pages=16, shuffle_pages=True),
    "varlen-gqa8": _lr("varlen-gqa8", 63, [700, 1500, 333], [700, 1700, 1333], hq=16, hkv=2,
                       per_sequence_seeds=True, spare_pages=3, shuffle_pages=True),
    "d64-b64-p8": _lr("d64-b64-p8", 64, [1100], hq=4, hkv=2, d=64, B=64, p=8, sink_logit=26.0),
    "d128-b64-p4": _lr("d128-b64-p4", 65, [1300], [1400], hq=4, hkv=4, d=128, B=64, p=4),
    "b128-p32": _lr("b128-p32", 66, [900], hq=4, hkv=2, d=128, B=128, p=32),
}


@pytest.fixture(scope="module", params=list(CASES))
def run(request):
    require_gpu()
    case = CASES[request.param]()
    say("case", request.param, "q", tuple(case.q.shape), "pages", tuple(case.k_pages.shape))
    return {"name": request.param, "case": case, "dev": OnDevice(case)}


def test_second_order_scores(run):
    case, dev = run["case"], run["dev"]
    say(run["name"], "second-order scores")
    P2 = cosa.cobs_scores(dev.problem, dev.q, dev.k, case.pool)
    torch.cuda.synchronize()
    got = P2.cpu().numpy()
    ref = ocobs.cobs_case(case)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), "pattern of -inf entries"
    assert np.all(got[~fin] == -np.inf)
    err = np.abs(got[fin] - ref[fin]).max()
    assert err <= 1e-2 * np.abs(ref[fin]).max(), f"max err {err:.3e}"
    run["P2"] = P2


def test_rank_over_second_order_scores(run):
    case, dev = run["case"], run["dev"]
    P2 = run.get("P2")
    if P2 is None:
        P2 = cosa.cobs_scores(dev.problem, dev.q, dev.k, case.pool)
    say(run["name"], "rank over second-order scores")
    k = cosa.kap_rank(dev.problem, P2, case.pool, case.budget, export_block_scores=True)
    torch.cuda.synchronize()
    ref = oc.kap_case(case, precision="fp32", P_given=P2.cpu().numpy())
    for name in ("order", "hrm", "count"):
        np.testing.assert_array_equal(k[name].cpu().numpy(), ref[name], err_msg=name)
    s = k["s"].cpu().numpy()
    assert np.array_equal(s.view(np.uint32), ref["s"].astype(np.float32).view(np.uint32)), "block scores"


def test_rank_pass_equals_fused_proxy(run):
    case, dev = run["case"], run["dev"]
    say(run["name"], "rank pass over exported scores")
    fused = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, case.budget, export_scores=True,
                           export_block_scores=True)
    k = cosa.kap_rank(dev.problem, fused["P"], case.pool, case.budget, export_block_scores=True)
    torch.cuda.synchronize()
    for name in ("order", "hrm", "count", "s"):
        assert torch.equal(k[name], fused[name]), name
