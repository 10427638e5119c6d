"""The allocation-free decode step, cosa_osk_decode_noalloc, through the C ABI
against cosa_osk_decode with a caller's workspace: the same kernels over the
same inputs, so output, log-sum-exp and per-row counters must agree bit for
bit. Two calls in a row, the second on a smaller problem (fewer sequences,
heads and segments), so the second runs over the first's leftover scratch
contents; then the first problem again; a problem whose partial results
exceed the fixed scratch is rejected before any launch."""
import numpy as np
import pytest
import torch

import block_sparse_attention_26_amd as cosa
import synthetic
from gpu_common import OnDevice, require_gpu, say

pytestmark = pytest.mark.gpu


def _case(seed, lk, h_q, h_kv, sink=None):
    return synthetic.lowrank_case(seed, [1] * len(lk), lk, h_q=h_q, h_kv=h_kv, head_dim=128, block=128, pool=16,
                                  budget=0.2, per_sequence_seeds=True, spare_pages=2, shuffle_pages=True,
                                  sink_logit=sink, name=f"decode-{seed}")


def _noalloc(dev, order, count, tau, n_splits):
    """cosa_osk_decode_noalloc on NaN/garbage-filled outputs (raw C entry point)."""
    pr = dev.problem
    d = pr.dims()
    o = torch.full(tuple(dev.q.shape), float("nan"), dtype=dev.q.dtype, device=dev.q.device)
    vis = torch.full((pr.c.batch, pr.c.h_q, d.max_nq), -7, dtype=torch.int32, device=dev.q.device)
    skp = torch.full_like(vis, -7)
    lse = torch.full((pr.c.h_q, d.total_q), float("nan"), dtype=torch.float32, device=dev.q.device)
    c = pr.for_tensors(dev.q, o)
    cosa.cosa_osk_decode_noalloc(c, dev.q.data_ptr(), dev.k.data_ptr(), dev.v.data_ptr(), order.data_ptr(),
                                 count.data_ptr(), int(order.shape[3]), pr.group, tau, n_splits, o.data_ptr(),
                                 vis.data_ptr(), skp.data_ptr(), lse.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    return {"O": o, "visited": vis, "skipped": skp, "lse": lse}


def _check_pair(dev, case, n_splits):
    pr = dev.problem
    ko = cosa.kap_order(pr, dev.q, dev.k, case.pool, case.budget)
    ref = cosa.osk_decode(pr, dev.q, dev.k, dev.v, ko["order"], ko["count"], case.tau, n_splits, lse=True)
    got = _noalloc(dev, ko["order"], ko["count"], case.tau, n_splits)
    torch.cuda.synchronize()
    assert torch.equal(got["O"].view(torch.int16), ref["O"].view(torch.int16)), "O"
    assert torch.equal(got["lse"].view(torch.int32), ref["lse"].view(torch.int32)), "lse"
    for name in ("visited", "skipped"):
        assert torch.equal(got[name], ref[name]), name
    assert int(ref["visited"].sum()) > 0
    return int(ref["skipped"].sum())


def test_noalloc_decode_matches_workspace_decode():
    require_gpu()
    big = _case(71, [9000, 3000, 12000, 130, 5000, 7000], 16, 2, sink=24.0)
    small = _case(72, [2500, 777], 8, 2)
    dbig, dsmall = OnDevice(big), OnDevice(small)
    say("no-alloc decode", "large problem, 8 segments")
    skipped = _check_pair(dbig, big, 8)
    assert skipped > 0  # aligned sinks: some blocks skipped in-kernel
    say("no-alloc decode", "smaller problem, 3 segments, over the previous call's scratch")
    _check_pair(dsmall, small, 3)
    say("no-alloc decode", "large problem again, 5 segments")
    _check_pair(dbig, big, 5)


def test_noalloc_decode_rejects_oversized_problem():
    require_gpu()
    case = _case(73, [600] * 8, 8, 2)
    dev = OnDevice(case)
    pr = dev.problem
    ko = cosa.kap_order(pr, dev.q, dev.k, case.pool, case.budget)
    # 8 sequences x 8 heads x 1024 segments x (128 + 2) floats > 32 MiB
    assert cosa.cosa_osk_decode_workspace_size(pr.c, 1024) > 32 << 20
    assert cosa.cosa_osk_decode_workspace_size(pr.c, 512) <= 32 << 20
    with pytest.raises(cosa.CosaError, match="scratch") as ei:
        _noalloc(dev, ko["order"], ko["count"], case.tau, 1024)
    assert ei.value.status == -2
    # the largest segment count that fits still matches the workspace entry point
    _check_pair(dev, case, 512)
