"""GPU parity of the decode step (one new query token per sequence) against the
oracle's split walk, through the C ABI.

* proxy lists on decode problems bit-exact against the oracle fed the GPU's
  fp32 proxy scores;
* decode walk for 1, 3 and 8 segments: O within the bf16 tolerance of the
  fp64 oracle, lse within 1e-2, visited exact, skipped exact for every head
  whose decisions all sit outside the 1e-3-nat ambiguity band;
* skipping off: every segment count gives the same result as the oracle;
  full budget with skipping off equals dense attention of the last row;
* an empty list gives O = 0 and lse = -inf, a corrupt entry NaN for its
  group only.
Cases cover GQA 4 and 8, ragged contexts, a shuffled NaN-poisoned page pool,
a sequence with no new token, d = 64 with B = 64, and aligned sinks (skips).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_26_amd as cosa
import synthetic
from oracle import cases as oc, decode as odec
from gpu_common import AMBIGUOUS_NATS, OnDevice, check_output, require_gpu, say

pytestmark = pytest.mark.gpu


def _dc(name, seed, lk, lq=None, hq=8, hkv=2, d=128, B=128, p=16, budget=0.25, **kw):
    lq = [1] * len(lk) if lq is None else lq
    return lambda: synthetic.lowrank_case(seed, lq, lk, h_q=hq, h_kv=hkv, head_dim=d, block=B, pool=p,
                                          budget=budget, name=name, **kw)


CASES = {
    "g4-ragged-paged": _dc("g4-ragged-paged", 51, [5000, 700, 9000, 130], spare_pages=4, shuffle_pages=True,
                           per_sequence_seeds=True),
    "g8-sinks": _dc("g8-sinks", 52, [6000, 3000], hq=16, hkv=2, sink_logit=24.0, per_sequence_seeds=True),
    "d64-b64-sinks": _dc("d64-b64-sinks", 53, [2000, 65, 4100], hq=4, hkv=1, d=64, B=64, p=8, sink_logit=24.0,
                         per_sequence_seeds=True),
    "no-token": _dc("no-token", 54, [3000, 200, 1500], lq=[1, 0, 1], per_sequence_seeds=True),
}


@pytest.fixture(scope="module", params=list(CASES))
def run(request):
    require_gpu()
    case = CASES[request.param]()
    say("case", request.param, "q", tuple(case.q.shape), "pages", tuple(case.k_pages.shape))
    dev = OnDevice(case)
    ko = oc.kap_case(case)
    return {"name": request.param, "case": case, "dev": dev, "ko": ko,
            "order": torch.from_numpy(ko["order"]).cuda(), "count": torch.from_numpy(ko["count"]).cuda()}


def test_decode_proxy_lists(run):
    case, dev = run["case"], run["dev"]
    say(run["name"], "decode proxy")
    k = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, case.budget, export_scores=True)
    torch.cuda.synchronize()
    ref = oc.kap_case(case, precision="fp32", P_given=k["P"].cpu().numpy())
    for name in ("order", "hrm", "count"):
        np.testing.assert_array_equal(k[name].cpu().numpy(), ref[name], err_msg=name)


@pytest.mark.parametrize("n_splits", [1, 3, 8])
def test_decode_parity(run, n_splits):
    case, dev = run["case"], run["dev"]
    say(run["name"], "decode, segments", n_splits)
    g = cosa.osk_decode(dev.problem, dev.q, dev.k, dev.v, run["order"], run["count"], case.tau, n_splits,
                        lse=True)
    torch.cuda.synchronize()
    ref = odec.decode_case(case, run["ko"]["order"], run["ko"]["count"], n_splits)
    check_output(g["O"], ref["O"], case.dtype, f"{run['name']} S={n_splits}")
    lse = g["lse"].cpu().numpy()
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - ref["lse"][fin]).max() < 1e-2
    vis = g["visited"].cpu().numpy()[:, :, 0]
    skp = g["skipped"].cpu().numpy()[:, :, 0]
    np.testing.assert_array_equal(vis, ref["visited"])
    clear = ~(np.abs(ref["margin"]) < AMBIGUOUS_NATS).any(axis=2)
    np.testing.assert_array_equal(skp[clear], ref["skipped"][clear])
    if "sinks" in run["name"] and n_splits < 8:
        assert skp.sum() > 0  # the case exercises both fates


def test_decode_no_skip_any_split(run):
    case, dev = run["case"], run["dev"]
    say(run["name"], "decode without skipping")
    ref = odec.decode_case(case, run["ko"]["order"], run["ko"]["count"], 1, tau=0.0)
    for n_splits in (1, 5):
        g = cosa.osk_decode(dev.problem, dev.q, dev.k, dev.v, run["order"], run["count"], 0.0, n_splits)
        torch.cuda.synchronize()
        check_output(g["O"], ref["O"], case.dtype, f"{run['name']} tau=0 S={n_splits}")
        assert int(g["skipped"].sum()) == 0


def test_decode_full_budget_is_dense(run):
    case, dev = run["case"], run["dev"]
    say(run["name"], "decode, budget 1")
    full = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, 1.0)
    g = cosa.osk_decode(dev.problem, dev.q, dev.k, dev.v, full["order"], full["count"], 0.0, 4)
    torch.cuda.synchronize()
    check_output(g["O"], oc.dense_case(case)["O"], case.dtype, run["name"] + " dense")


def test_decode_empty_and_corrupt_lists(run):
    case, dev = run["case"], run["dev"]
    say(run["name"], "decode, empty and corrupt lists")
    order = run["ko"]["order"].copy()
    count = run["ko"]["count"].copy()
    G = case.h_q // case.h_kv
    cu = case.cu_seqlens_q.tolist()
    live = [b for b in range(case.batch) if cu[b + 1] > cu[b]]
    b0 = live[0]
    count[b0, 0, 0] = 0
    order[b0, 0, 0, :] = 1 << 30  # never read
    corrupt = case.h_kv > 1 and count[b0, 1, 0] >= 2
    if corrupt:
        order[b0, 1, 0, 1] = (int(case.seqlens_k[b0]) - 1) // case.block + 1  # past the causal range
    g = cosa.osk_decode(dev.problem, dev.q, dev.k, dev.v, torch.from_numpy(order).cuda(),
                        torch.from_numpy(count).cuda(), case.tau, 3, lse=True)
    base = cosa.osk_decode(dev.problem, dev.q, dev.k, dev.v, run["order"], run["count"], case.tau, 3, lse=True)
    torch.cuda.synchronize()
    O = g["O"].float().cpu().numpy()
    O0 = base["O"].float().cpu().numpy()
    lse, lse0 = g["lse"].cpu().numpy(), base["lse"].cpu().numpy()
    t = cu[b0]
    assert np.all(O[t, 0:G] == 0.0) and np.all(lse[0:G, t] == -np.inf)
    assert np.all(g["visited"].cpu().numpy()[b0, 0:G, 0] == 0)
    touched = np.zeros(O.shape[:2], dtype=bool)
    touched[t, 0:G] = True
    if corrupt:
        assert np.all(np.isnan(O[t, G : 2 * G])) and np.all(np.isnan(lse[G : 2 * G, t]))
        touched[t, G : 2 * G] = True
    keep = ~touched
    assert np.array_equal(O[keep].view(np.uint32), O0[keep].view(np.uint32))
    assert np.array_equal(lse.T[keep].view(np.uint32), lse0.T[keep].view(np.uint32))


def test_decode_proxy_scores_tolerance(run):
    """Decode problems take the heads-as-columns score pass; its P stays within
    the max-pooled scores' tolerance of the fp64 oracle."""
    case, dev = run["case"], run["dev"]
    say(run["name"], "decode proxy scores")
    k = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, case.budget, export_scores=True)
    torch.cuda.synchronize()
    P = k["P"].cpu().numpy()
    P64 = oc.kap_case(case, precision="fp64")["P"]
    fin = np.isfinite(P64)
    assert np.array_equal(np.isfinite(P), fin)
    assert np.all(P[~fin] == -np.inf)
    assert np.abs(P[fin] - P64[fin]).max() <= 1e-2 * np.abs(P64[fin]).max()


def _shorter(problem_case, dev, drop):
    """The same batch with `drop` fewer cached tokens per non-empty sequence."""
    case = problem_case
    lk = [max(int(x) - drop, q) for x, q in zip(case.seqlens_k.tolist(), case.seqlens_q)]
    cu = case.cu_seqlens_q.tolist()
    return cosa.Problem(h_q=case.h_q, h_kv=case.h_kv, head_dim=case.head_dim, block=case.block,
                        dtype=cosa.COSA_BF16, softmax_scale=case.scale, num_pages=int(case.k_pages.shape[0]),
                        cu_seqlens_q=case.cu_seqlens_q.cuda(), seqlens_k=torch.tensor(lk, dtype=torch.int32).cuda(),
                        block_table=case.block_table.cuda(), host_cu_seqlens_q=cu, host_seqlens_k=lk)


def test_pooled_keys_reused_and_updated(run):
    """Pooled keys kept across calls give the proxy's own lists and scores bit
    for bit, and re-pooling only each sequence's last block after a token is
    appended reproduces a full re-pooling."""
    case, dev = run["case"], run["dev"]
    say(run["name"], "pooled keys")
    pooled = cosa.pool_keys(dev.problem, dev.k, case.pool)
    a = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, case.budget, export_scores=True)
    b = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, case.budget, export_scores=True, pooled_keys=pooled)
    torch.cuda.synchronize()
    for name in ("order", "hrm", "count"):
        assert torch.equal(a[name], b[name]), name
    assert torch.equal(a["P"].view(torch.int32), b["P"].view(torch.int32))
    for drop in (1, 37):
        prev = _shorter(case, dev, drop)
        buf = cosa.pool_keys(prev, dev.k, case.pool)
        if drop == 1:  # one appended token: only the last block changes
            cosa.pool_keys(dev.problem, dev.k, case.pool, out=buf, last_block_only=True)
            torch.cuda.synchronize()
            assert torch.equal(buf.view(torch.int16), pooled.view(torch.int16))
        else:  # several tokens may span a block boundary: a full pass is needed, and matches
            cosa.pool_keys(dev.problem, dev.k, case.pool, out=buf)
            torch.cuda.synchronize()
            assert torch.equal(buf.view(torch.int16), pooled.view(torch.int16))
