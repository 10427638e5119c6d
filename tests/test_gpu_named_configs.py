"""GPU parity at the named workloads' full sizes, in the launch configuration
the benchmark times (proxy in workspace mode, walk without diagnostics), with
a second diagnostic run that must agree with it bit for bit.

* 32K prefill (32 query / 8 KV heads, d 128, bf16, block 128, pool 16, 10%):
  every list row bit-exact against the oracle fed the GPU's proxy scores,
  the proxy scores within tolerance of the fp64 oracle, the full output of
  every head and query block against the oracle's ordered walk, skip sets,
  and the dense kernel on sampled query blocks.
* 4K chunk over a 64K paged cache (640-page shuffled pool, 128 NaN pages):
  the same checks, full output.
* ragged batch (8 sequences of 4K-32K, 64 / 8 heads): lists bit-exact for
  every row, output on sampled query blocks of every sequence; and at budget
  1 with skipping off the walk equals dense attention (CoSA summary §2.1: the
  accumulation does not depend on the visit order; §2.3: nothing unlisted).

Sampled query blocks are the first two, the last two and evenly spaced ones
in between (the longest lists sit at the end of a causal prefill).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_26_amd as cosa
import synthetic
from oracle import cases as oc, layout
from gpu_common import (TOL, check_dense, check_lists, check_proxy_scores, check_walk, require_gpu, run_gpu,
                        sample_qbs, say)

pytestmark = pytest.mark.gpu


def test_config2_32k_full():
    require_gpu()
    case = synthetic.config_case(2)
    say("32K prefill generated", tuple(case.q.shape))
    g = run_gpu(case)
    assert int(g["count"].sum()) == 3406 * case.h_kv  # closed form at 10%
    say("32K: lists of every row")
    assert check_lists(case, g, case.budget) == case.h_kv * 256
    check_proxy_scores(case, g)
    say("32K: full output against the oracle's walk")
    check_walk(case, g)
    say("32K: dense on sampled query blocks")
    check_dense(case, g["dev"], [sample_qbs(256, 4)])


def test_config4_chunk_over_paged_cache_full():
    require_gpu()
    case = synthetic.config_case(4)
    assert case.k_pages.shape[0] == 640 and torch.isnan(case.k_pages.float()).any()
    say("4K chunk over 64K generated", tuple(case.q.shape), "pool", tuple(case.k_pages.shape))
    g = run_gpu(case)
    assert int(g["count"].sum()) == 1604 * case.h_kv
    say("chunk: lists of every row")
    assert check_lists(case, g, case.budget) == case.h_kv * 32
    check_proxy_scores(case, g)
    say("chunk: full output against the oracle's walk")
    check_walk(case, g)
    say("chunk: dense on sampled query blocks")
    check_dense(case, g["dev"], [sample_qbs(32, 4)])


@pytest.fixture(scope="module")
def ragged():
    require_gpu()
    case = synthetic.config_case(5)
    say("ragged batch generated", case.seqlens_q, "heads", case.h_q, case.h_kv)
    return case


def test_config5_ragged_batch(ragged):
    case = ragged
    g = run_gpu(case)
    say("ragged: lists of every row")
    check_lists(case, g, case.budget)
    qbs = [sample_qbs(layout.cdiv(L, case.block), 6) for L in case.seqlens_q]
    say("ragged: output on sampled query blocks")
    check_walk(case, g, qbs)


def test_config5_full_budget_no_skip_equals_dense(ragged):
    """Budget 1 lists every causal block; with skipping off the walk is dense
    attention (checked against the fp64 dense oracle and the dense kernel)."""
    case = ragged
    g = run_gpu(case, budget=1.0, tau=0.0)
    n_all = oc.n_causal_rows(case)
    np.testing.assert_array_equal(g["count"], n_all)
    assert int(g["walk"]["skipped"].sum()) == 0
    say("ragged, budget 1: lists of sampled rows")
    qbs = [sample_qbs(layout.cdiv(L, case.block), 6) for L in case.seqlens_q]
    check_lists(case, g, 1.0, rows=qbs)
    say("ragged, budget 1: walk against dense")
    Od = check_dense(case, g["dev"], qbs)
    cu = case.cu_seqlens_q.tolist()
    B = case.block
    idx = np.concatenate([cu[b] + np.concatenate([np.arange(qb * B, min(qb * B + B, L)) for qb in qbs[b]])
                          for b, L in enumerate(case.seqlens_q)])
    ref = oc.dense_case(case, rows_per_seq=[np.concatenate([np.arange(qb * B, min(qb * B + B, L))
                                                            for qb in qbs[b]])
                                            for b, L in enumerate(case.seqlens_q)])["O"]
    mx, mean = TOL[case.dtype]
    err = np.abs(g["O"][idx] - ref[idx])
    assert err.max() <= mx and err.mean() <= mean, (err.max(), err.mean())
    # the walk over every block and the dense kernel differ only by rounding
    # (different visit order): both within the bf16 tolerance of each other
    d = np.abs(g["O"] - Od)
    assert d.max() <= mx and d.mean() <= mean, (d.max(), d.mean())
