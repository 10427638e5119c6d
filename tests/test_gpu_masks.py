"""GPU parity of the comparison modes (binary masks, control-flow walk, exact
block mass) against the oracle, through the C ABI.

* list -> mask and mask -> ascending list: bit-exact against the oracle,
  including invalid entries, corrupt counts, non-causal mask bits, truncation
  and the no-mask (every causal block) form;
* the masked walk equals the list walk over the ascending list bit for bit
  (O, visited, skipped), and that list walk matches the oracle's ordered walk
  (O within the bf16 tolerance, skip sets outside the ambiguity band);
* exact block mass within 1e-3 relative (+1e-4 absolute) of the fp64 oracle,
  each row's masses summing to its valid row count.
Cases cover GQA 4 and 8, ragged batches, chunked offsets over shuffled
NaN-poisoned page pools, both block sizes and lists that cross 64-block mask
words.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_26_amd as cosa
import synthetic
from oracle import cases as oc, masks as om
from gpu_common import OnDevice, check_output, check_skip_sets, require_gpu, say

pytestmark = pytest.mark.gpu


def _lr(name, seed, lq, lk=None, hq=8, hkv=2, d=128, B=128, p=16, budget=0.25, **kw):
    return lambda: synthetic.lowrank_case(seed, lq, lk, h_q=hq, h_kv=hkv, head_dim=d, block=B, pool=p,
                                          budget=budget, name=name, **kw)


CASES = {
    "gqa4-ragged": _lr("gqa4-ragged", 31, [2000]),
    "sinks": _lr("sinks", 32, [3000], sink_logit=24.0),
    "chunk-paged": _lr("chunk-paged", 33, [1000], [8192], budget=0.1, spare_pages=16, shuffle_pages=True),
    "varlen-gqa8": _lr("varlen-gqa8", 34, [700, 1500, 333], [700, 1700, 1333], hq=16, hkv=2,
                       per_sequence_seeds=True, spare_pages=3, shuffle_pages=True),
    "b64-words": _lr("b64-words", 35, [300], [9000], hq=4, hkv=2, d=64, B=64, p=16, budget=0.3,
                     sink_logit=24.0, shuffle_pages=True),
    "d128-b64": _lr("d128-b64", 36, [1300], [1400], hq=4, hkv=4, d=128, B=64, p=4),
    # six KV heads: the walk's launch order takes KV groups in phases of four
    "kv6-phases": _lr("kv6-phases", 37, [900, 400], [900, 1300], hq=12, hkv=6, per_sequence_seeds=True,
                      sink_logit=24.0),
}


@pytest.fixture(scope="module", params=list(CASES))
def run(request):
    require_gpu()
    case = CASES[request.param]()
    say("case", request.param, "q", tuple(case.q.shape), "pages", tuple(case.k_pages.shape))
    dev = OnDevice(case)
    ko = oc.kap_case(case)
    return {"name": request.param, "case": case, "dev": dev, "ko": ko,
            "n": oc.n_causal_rows(case), "max_nk": oc.dims(case)["max_nk"]}


def test_mask_from_order_exact(run):
    case, dev, ko = run["case"], run["dev"], run["ko"]
    mw = cosa.mask_words_for(dev.problem)
    say(run["name"], "mask from order")
    order = torch.from_numpy(ko["order"]).cuda()
    count = torch.from_numpy(ko["count"]).cuda()
    got = cosa.mask_from_order(dev.problem, order, count).cpu().numpy().view(np.uint64)
    want = om.pack_words(om.mask_from_order(ko["order"], ko["count"], run["n"], run["max_nk"]), mw)
    np.testing.assert_array_equal(got, want)
    # corrupt lists: out-of-range and negative entries, duplicates, counts past kmax or negative
    rng = np.random.default_rng(7)
    bad_o = ko["order"].copy()
    bad_o[..., 0] = rng.integers(-3, run["max_nk"] + 5, size=bad_o.shape[:-1])
    if bad_o.shape[-1] > 1:
        bad_o[..., -1] = bad_o[..., 0]
    bad_c = ko["count"].copy()
    bad_c.flat[::3] = bad_o.shape[-1] + 4
    bad_c.flat[1::5] = -1
    say(run["name"], "mask from corrupt order")
    got = cosa.mask_from_order(dev.problem, torch.from_numpy(bad_o).cuda(),
                               torch.from_numpy(bad_c).cuda(), mask_words=mw + 1).cpu().numpy().view(np.uint64)
    want = om.pack_words(om.mask_from_order(bad_o, bad_c, run["n"], run["max_nk"]), mw + 1)
    np.testing.assert_array_equal(got, want)


def test_order_from_mask_exact(run):
    case, dev = run["case"], run["dev"]
    mw = cosa.mask_words_for(dev.problem)
    rng = np.random.default_rng(8)
    shape = run["n"].shape
    # random masks with bits set past the causal edge and in the spare words
    mask = rng.random(shape + (64 * mw,)) < 0.3
    words = om.pack_words(mask, mw)
    for kmax in (run["max_nk"], 5, 1):
        say(run["name"], "order from mask, kmax", kmax)
        g = cosa.order_from_mask(dev.problem, torch.from_numpy(words.view(np.int64)).cuda(), kmax)
        want_o, want_c = om.order_from_mask(mask, run["n"], kmax)
        np.testing.assert_array_equal(g["order"].cpu().numpy(), want_o)
        np.testing.assert_array_equal(g["count"].cpu().numpy(), want_c)
    say(run["name"], "order from no mask")
    g = cosa.order_from_mask(dev.problem, None, run["max_nk"], device="cuda")
    want_o, want_c = om.order_from_mask(None, run["n"], run["max_nk"])
    np.testing.assert_array_equal(g["order"].cpu().numpy(), want_o)
    np.testing.assert_array_equal(g["count"].cpu().numpy(), want_c)


def test_masked_walk_equals_ascending_list_walk(run):
    case, dev, ko = run["case"], run["dev"], run["ko"]
    order = torch.from_numpy(ko["order"]).cuda()
    count = torch.from_numpy(ko["count"]).cuda()
    say(run["name"], "masked walk")
    mask = cosa.mask_from_order(dev.problem, order, count)
    asc = cosa.order_from_mask(dev.problem, mask, ko["kmax"])
    gm = cosa.osk_attention_masked(dev.problem, dev.q, dev.k, dev.v, mask, case.tau, lse=True)
    gl = cosa.osk_attention(dev.problem, dev.q, dev.k, dev.v, asc["order"], asc["count"], case.tau,
                            skip_bits=True, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(gm["O"].view(torch.int16), gl["O"].view(torch.int16))
    assert torch.equal(gm["visited"], gl["visited"])
    assert torch.equal(gm["skipped"], gl["skipped"])
    assert torch.equal(gm["lse"], gl["lse"])
    # the ascending walk against the oracle's ordered walk over the same list
    a_o, a_c = asc["order"].cpu().numpy(), asc["count"].cpu().numpy()
    ref = oc.osk_case(case, a_o, a_c)
    check_output(gl["O"], ref["O"], case.dtype, run["name"] + " ascending")
    check_skip_sets(gl, ref, a_c, case.h_q // case.h_kv)
    # the same blocks as the proxy's list, in ascending order
    want_o, _ = om.order_from_mask(om.mask_from_order(ko["order"], ko["count"], run["n"], run["max_nk"]),
                                   run["n"], ko["kmax"])
    np.testing.assert_array_equal(a_o, want_o)
    if run["name"] in ("sinks", "b64-words"):
        assert int(gm["skipped"].sum()) > 0  # the skip path runs under the mask walk


def test_masked_walk_with_no_skip_equals_dense_when_full(run):
    """Every causal block selected and skipping off: the mask walk is dense attention."""
    case, dev = run["case"], run["dev"]
    say(run["name"], "full mask walk")
    mw = cosa.mask_words_for(dev.problem)
    full = torch.full((case.batch, case.h_kv, run["n"].shape[2], mw), -1, dtype=torch.int64, device="cuda")
    gm = cosa.osk_attention_masked(dev.problem, dev.q, dev.k, dev.v, full, 0.0)
    de = cosa.dense_attention(dev.problem, dev.q, dev.k, dev.v)
    torch.cuda.synchronize()
    assert torch.equal(gm["O"].view(torch.int16), de["O"].view(torch.int16))
    np.testing.assert_array_equal(gm["visited"].cpu().numpy(),
                                  np.repeat(run["n"], case.h_q // case.h_kv, axis=1))
    assert int(gm["skipped"].sum()) == 0


def test_block_mass_parity(run):
    case, dev = run["case"], run["dev"]
    rows = np.zeros((case.batch, case.h_q, run["n"].shape[2]))
    B = case.block
    for b, lq in enumerate(case.seqlens_q):
        for qb in range(-(-lq // B)):
            rows[b, :, qb] = min(B, lq - qb * B)
    # with the oracle's log-sum-exp the kernel's own arithmetic is checked
    lse_ref = torch.from_numpy(oc.dense_case(case)["lse"].astype(np.float32)).cuda()
    say(run["name"], "block mass")
    M = cosa.block_mass(dev.problem, dev.q, dev.k, lse_ref)
    torch.cuda.synchronize()
    got = M.cpu().numpy().astype(np.float64)
    want = oc.block_mass_case(case)
    assert np.isfinite(got).all()
    err = np.abs(got - want)
    assert (err <= 1e-3 * np.abs(want) + 1e-4).all(), f"max err {err.max():.3e}"
    np.testing.assert_allclose(got.sum(axis=3), rows, rtol=1e-4, atol=1e-4)
    # with the dense kernel's log-sum-exp (its sums add bf16-rounded weights)
    say(run["name"], "block mass after dense")
    de = cosa.dense_attention(dev.problem, dev.q, dev.k, dev.v, lse=True)
    Md = cosa.block_mass(dev.problem, dev.q, dev.k, de["lse"])
    torch.cuda.synchronize()
    np.testing.assert_allclose(Md.cpu().numpy().sum(axis=3), rows, rtol=1e-2, atol=1e-2)
    # recall of the proxy's selection never beats the oracle selector's
    G = case.h_q // case.h_kv
    Mg = got.reshape(case.batch, case.h_kv, G, *got.shape[2:]).sum(axis=2)
    rec = om.recall(Mg, run["ko"]["order"], run["ko"]["count"])
    best = om.oracle_recall(Mg, run["ko"]["count"])
    live = np.isfinite(rec)
    assert (rec[live] <= best[live] + 1e-6).all()


def test_union_order_exact_and_walk(run):
    case, dev, ko = run["case"], run["dev"], run["ko"]
    order = torch.from_numpy(ko["order"]).cuda()
    count = torch.from_numpy(ko["count"]).cuda()
    for uk in (run["max_nk"], 3):
        say(run["name"], "union order, width", uk)
        u = cosa.union_order(dev.problem, order, count, union_kmax=uk)
        want_o, want_c = om.union_lists(ko["order"], ko["count"], run["n"], uk)
        np.testing.assert_array_equal(u["order"].cpu().numpy(), want_o)
        np.testing.assert_array_equal(u["count"].cpu().numpy(), want_c)
    # the union walk (dense over the table, no skip) against the oracle's walk
    say(run["name"], "union walk")
    u = cosa.union_order(dev.problem, order, count)
    g = cosa.osk_attention(dev.problem, dev.q, dev.k, dev.v, u["order"], u["count"], 0.0)
    torch.cuda.synchronize()
    uo, uc = u["order"].cpu().numpy(), u["count"].cpu().numpy()
    ref = oc.osk_case(case, uo, uc, tau=0.0)
    check_output(g["O"], ref["O"], case.dtype, run["name"] + " union")
    assert int(g["skipped"].sum()) == 0
    np.testing.assert_array_equal(g["visited"].cpu().numpy(), np.repeat(uc, case.h_q // case.h_kv, axis=1))
