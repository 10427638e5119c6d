"""GPU parity of the HIP path against the CPU oracle (through the C ABI).

* KAP: order, HRM flags, counts and block scores bit-exact against the oracle
  fed the GPU's fp32 proxy scores; the proxy scores themselves within the
  bf16/fp32 tolerance of the oracle's fp64 scores.
* OSK: given the same order lists, visited sets identical, in-kernel skip
  sets identical outside a 1e-3-nat band around the threshold, O within
  2e-2 max / 2e-3 mean (bf16) or 1e-4 (fp32) of the fp64 oracle.
* Dense: O and lse against the fp64 dense oracle.
Cases span several tiles, ragged tails, chunked offsets, shuffled
NaN-poisoned page pools and packed ragged batches; GQA groups of 1, 2, 3, 4,
8 and 16; 1, 2, 4 and 6 KV heads.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_26_amd as cosa
import synthetic
from oracle import cases as oc
from gpu_common import OnDevice, check_output, check_skip_sets, require_gpu, say, TOL

pytestmark = pytest.mark.gpu


def _lr(name, seed, lq, lk=None, hq=8, hkv=2, d=128, B=128, p=16, budget=0.25, dtype="bf16", **kw):
    return lambda: synthetic.lowrank_case(seed, lq, lk, h_q=hq, h_kv=hkv, head_dim=d, block=B, pool=p,
                                          budget=budget, dtype=dtype, name=name, **kw)


CASES = {
    "cfg1": lambda: synthetic.config_case(1),
    "f32-sinks": _lr("f32-sinks", 11, [1024], hq=2, hkv=1, d=64, B=64, p=8, dtype="f32", sink_logit=24.0),
    "f32-d128": _lr("f32-d128", 12, [700], hq=4, hkv=2, d=128, B=128, p=16, dtype="f32"),
    "bf16-gqa4-ragged": _lr("bf16-gqa4-ragged", 13, [2000], hq=8, hkv=2),
    "bf16-sinks": _lr("bf16-sinks", 14, [3000], hq=8, hkv=2, sink_logit=24.0),
    "bf16-chunk-paged": _lr("bf16-chunk-paged", 15, [1000], [8192], hq=8, hkv=2, budget=0.1,
                            spare_pages=16, shuffle_pages=True),
    "bf16-varlen-gqa8": _lr("bf16-varlen-gqa8", 16, [700, 1500, 333], [700, 1700, 1333], hq=16, hkv=2,
                            per_sequence_seeds=True, spare_pages=3, shuffle_pages=True),
    "bf16-d64-b128": _lr("bf16-d64-b128", 17, [1500], hq=4, hkv=1, d=64, B=128, p=8),
    "bf16-d128-b64": _lr("bf16-d128-b64", 18, [1300], [1400], hq=4, hkv=4, d=128, B=64, p=4),
    "bf16-d64-b64-sinks": _lr("bf16-d64-b64-sinks", 19, [1100], hq=4, hkv=2, d=64, B=64, p=64,
                              sink_logit=26.0),
    # pooled keys per block (B/p) of 4, 32, 2 and 128: every block-max path of the proxy
    "bf16-b128-p32": _lr("bf16-b128-p32", 20, [900], hq=4, hkv=2, d=128, B=128, p=32),
    "bf16-b128-p4": _lr("bf16-b128-p4", 21, [800], [1000], hq=4, hkv=2, d=128, B=128, p=4),
    "bf16-b64-p32": _lr("bf16-b64-p32", 22, [700], hq=2, hkv=1, d=64, B=64, p=32),
    "bf16-b128-p1": _lr("bf16-b128-p1", 23, [600], hq=2, hkv=2, d=64, B=128, p=1),
    # odd and wide query groups: the proxy's score pass groups four (head,
    # row tile) pairs per workgroup, which straddle row tiles when G = 3
    "bf16-gqa3-b64-p16": _lr("bf16-gqa3-b64-p16", 24, [1500, 400], [1500, 900], hq=6, hkv=2, d=128, B=64, p=16,
                             per_sequence_seeds=True),
    "bf16-gqa16": _lr("bf16-gqa16", 25, [900], hq=16, hkv=1, d=128, B=128, p=16),
    # six KV groups: the attention walk's launch order takes KV groups in
    # phases of four, so the second phase holds only two
    "bf16-kv6-phases": _lr("bf16-kv6-phases", 26, [900, 300], [900, 700], hq=12, hkv=6, d=128, B=128, p=16,
                           per_sequence_seeds=True),
    # a packed batch holding a sequence with no query token (its KV cache is
    # not empty): empty lists, no output rows, nothing written for it
    "bf16-empty-seq": _lr("bf16-empty-seq", 27, [600, 0, 900], [600, 500, 1200], hq=8, hkv=2, d=128, B=128, p=16,
                          per_sequence_seeds=True, spare_pages=2, shuffle_pages=True),
}


@pytest.fixture(scope="module", params=list(CASES))
def run(request):
    require_gpu()
    case = CASES[request.param]()
    say("case", request.param, "q", tuple(case.q.shape), "pages", tuple(case.k_pages.shape))
    dev = OnDevice(case)
    ko = oc.kap_case(case)  # oracle order (fp64 proxy) drives the OSK parity
    order = torch.from_numpy(ko["order"]).cuda()
    count = torch.from_numpy(ko["count"]).cuda()
    return {"name": request.param, "case": case, "dev": dev, "ko": ko, "order": order, "count": count}


def test_osk_parity(run):
    case, dev = run["case"], run["dev"]
    say(run["name"], "osk")
    g = cosa.osk_attention(dev.problem, dev.q, dev.k, dev.v, run["order"], run["count"], case.tau,
                           skip_bits=True, lse=True)
    torch.cuda.synchronize()
    ref = oc.osk_case(case, run["ko"]["order"], run["ko"]["count"])
    check_output(g["O"], ref["O"], case.dtype, run["name"])
    namb, nskip = check_skip_sets(g, ref, run["ko"]["count"], case.h_q // case.h_kv)
    lse = g["lse"].cpu().numpy()
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - ref["lse"][fin]).max() < (1e-2 if case.dtype == "bf16" else 1e-4)
    if "sinks" in run["name"]:
        assert nskip > 0  # the case exercises both fates


def test_osk_deterministic(run):
    case, dev = run["case"], run["dev"]
    say(run["name"], "osk twice")
    a = cosa.osk_attention(dev.problem, dev.q, dev.k, dev.v, run["order"], run["count"], case.tau,
                           skip_bits=True)
    b = cosa.osk_attention(dev.problem, dev.q, dev.k, dev.v, run["order"], run["count"], case.tau,
                           skip_bits=True)
    torch.cuda.synchronize()
    assert torch.equal(a["O"].view(torch.uint8), b["O"].view(torch.uint8))
    assert torch.equal(a["skip_bits"], b["skip_bits"])


def test_dense_parity(run):
    case, dev = run["case"], run["dev"]
    say(run["name"], "dense")
    g = cosa.dense_attention(dev.problem, dev.q, dev.k, dev.v, lse=True)
    torch.cuda.synchronize()
    ref = oc.dense_case(case)
    check_output(g["O"], ref["O"], case.dtype, run["name"] + " dense")
    lse = g["lse"].cpu().numpy()
    assert np.abs(lse - ref["lse"]).max() < (1e-2 if case.dtype == "bf16" else 1e-4)


def test_full_budget_no_skip_equals_dense(run):
    """Budget 1 with skipping off lists every causal block: equals dense."""
    case, dev = run["case"], run["dev"]
    say(run["name"], "budget 1")
    full = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, 1.0)
    g = cosa.osk_attention(dev.problem, dev.q, dev.k, dev.v, full["order"], full["count"], 0.0)
    torch.cuda.synchronize()
    ref = oc.dense_case(case)
    check_output(g["O"], ref["O"], case.dtype, run["name"] + " budget1")
    assert int(g["skipped"].sum()) == 0


def test_kap_parity(run):
    case, dev = run["case"], run["dev"]
    say(run["name"], "kap export")
    k = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, case.budget, export_scores=True,
                       export_block_scores=True)
    say(run["name"], "kap workspace")
    k2 = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, case.budget)
    torch.cuda.synchronize()
    P = k["P"].cpu().numpy()
    ref = oc.kap_case(case, precision="fp32", P_given=P)
    for name in ("order", "hrm", "count"):
        got = k[name].cpu().numpy()
        np.testing.assert_array_equal(got, ref[name], err_msg=name)
        np.testing.assert_array_equal(k2[name].cpu().numpy(), got, err_msg=name + " (workspace mode)")
    s = k["s"].cpu().numpy()
    assert np.array_equal(s.view(np.uint32), ref["s"].astype(np.float32).view(np.uint32)), "block scores"
    # proxy scores upstream of the bit-exact contract: tolerance vs fp64
    P64 = oc.kap_case(case, precision="fp64")["P"]
    fin = np.isfinite(P64)
    assert np.array_equal(np.isfinite(P), fin), "visibility pattern of P"
    rel = 1e-2 if case.dtype == "bf16" else 1e-5
    assert np.abs(P[fin] - P64[fin]).max() <= rel * np.abs(P64[fin]).max()


def test_empty_and_corrupt_lists(run):
    """An empty list yields O = 0 and lse = -inf without reading any entry; an
    entry that is not a causal block of its row makes that row NaN; every other
    row is bit-identical to the run on the unmodified lists."""
    case, dev = run["case"], run["dev"]
    say(run["name"], "empty and corrupt lists")
    order = run["ko"]["order"].copy()
    count = run["ko"]["count"].copy()
    lq0 = int(case.cu_seqlens_q[1] - case.cu_seqlens_q[0])
    last_qb = (lq0 - 1) // case.block
    g_last = case.h_kv - 1
    # empty rows whose entries are garbage: must not be read
    count[0, 0, 0] = 0
    order[0, 0, 0, :] = 1 << 30
    count[0, g_last, last_qb] = 0
    order[0, g_last, last_qb, :] = -5
    # a negative count reads as an empty list (no entry read, nothing written
    # before the row's own skip bits)
    empty = [(0, 0), (g_last, last_qb)]
    if case.h_kv > 1 and last_qb >= 1:
        empty.append((g_last, 0))
    elif last_qb >= 2:
        empty.append((0, 1))
    if len(empty) == 3:
        count[0, empty[2][0], empty[2][1]] = -1000
        order[0, empty[2][0], empty[2][1], :] = 1 << 29
    # a corrupt row (needs a second query block and a list of two entries)
    corrupt = last_qb >= 1 and count[0, 0, last_qb] >= 2
    if corrupt:  # the first block past the row's causal range
        off = int(case.seqlens_k[0]) - lq0
        order[0, 0, last_qb, 1] = (off + lq0 - 1) // case.block + 1
    base = cosa.osk_attention(dev.problem, dev.q, dev.k, dev.v, run["order"], run["count"], case.tau,
                              skip_bits=True, lse=True)
    g = cosa.osk_attention(dev.problem, dev.q, dev.k, dev.v, torch.from_numpy(order).cuda(),
                           torch.from_numpy(count).cuda(), case.tau, skip_bits=True, lse=True)
    torch.cuda.synchronize()
    grp = case.h_q // case.h_kv
    B = case.block
    O = g["O"].float().cpu().numpy()
    O0 = base["O"].float().cpu().numpy()
    lse, lse0 = g["lse"].cpu().numpy(), base["lse"].cpu().numpy()
    touched = np.zeros(O.shape[:2], dtype=bool)  # [token, head]
    for (gg, qb) in empty:
        rows = slice(qb * B, min(qb * B + B, lq0))
        heads = slice(gg * grp, (gg + 1) * grp)
        assert np.all(O[rows, heads] == 0.0)
        assert np.all(lse[heads, rows] == -np.inf)
        assert np.all(g["visited"].cpu().numpy()[0, heads, qb] == 0)
        assert np.all(g["skipped"].cpu().numpy()[0, heads, qb] == 0)
        assert np.all(g["skip_bits"].cpu().numpy()[0, heads, qb] == 255)
        touched[rows, heads] = True
    if corrupt:
        rows = slice(last_qb * B, min(last_qb * B + B, lq0))
        heads = slice(0, grp)
        assert np.all(np.isnan(O[rows, heads]))
        assert np.all(np.isnan(lse[heads, rows]))
        touched[rows, heads] = True
    keep = ~touched
    assert np.array_equal(O[keep].view(np.uint32), O0[keep].view(np.uint32))
    assert np.array_equal(lse.T[keep].view(np.uint32), lse0.T[keep].view(np.uint32))
    # per-row counters and skip bits of every other row are those of the clean run
    row_keep = np.ones(g["visited"].shape, dtype=bool)  # [b, h_q, nq]
    for (gg, qb) in empty:
        row_keep[0, gg * grp:(gg + 1) * grp, qb] = False
    if corrupt:
        row_keep[0, 0:grp, last_qb] = False
    for name in ("visited", "skipped", "skip_bits"):
        a_, b_ = g[name].cpu().numpy(), base[name].cpu().numpy()
        assert np.array_equal(a_[row_keep], b_[row_keep]), name
