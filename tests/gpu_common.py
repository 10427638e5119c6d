"""Helpers shared by the GPU tests: move a synthetic case to the device, run
the library through its C ABI, and compare with the oracle."""
import math
import sys

import numpy as np
import torch

import block_sparse_attention_26_amd as cosa

# bf16 inputs: max-abs 2e-2 and mean-abs 2e-3 against the fp64 oracle; fp32 inputs: 1e-4.
TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-4)}
# skip decisions whose fp64 margin is within this many nats of the threshold
# may legitimately differ between fp32 GPU arithmetic and the fp64 oracle
AMBIGUOUS_NATS = 1e-3


def say(*args):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[gpu]", *args, file=sys.stderr, flush=True)


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cosa.load()


class OnDevice:
    def __init__(self, case):
        self.case = case
        self.q = case.q.cuda()
        self.k = case.k_pages.cuda()
        self.v = case.v_pages.cuda()
        self.problem = cosa.Problem.from_case(case)


def check_output(O_gpu, O_ref, dtype, what=""):
    """Element-wise comparison of the GPU output with the oracle's."""
    o = O_gpu.float().cpu().numpy().astype(np.float64)
    err = np.abs(o - O_ref)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    mx, mean = TOL[dtype]
    assert err.max() <= mx, f"{what}: max abs err {err.max():.3e} > {mx}"
    assert err.mean() <= mean, f"{what}: mean abs err {err.mean():.3e} > {mean}"
    return float(err.max()), float(err.mean())


def check_skip_sets(gpu, ref, count, G):
    """visited identical; skip bits identical outside the ambiguity band."""
    vis = gpu["visited"].cpu().numpy()
    nb, hq, nq = vis.shape
    want_vis = np.repeat(count, G, axis=1)  # [b, h_kv, nq] -> [b, h_q, nq]
    np.testing.assert_array_equal(vis, want_vis)
    np.testing.assert_array_equal(vis, ref["visited"])
    bits = gpu["skip_bits"].cpu().numpy()
    rb = ref["skip_bits"]
    amb = np.abs(ref["margin"]) < AMBIGUOUS_NATS
    diff = (bits != rb) & ~amb
    assert not diff.any(), f"{int(diff.sum())} skip decisions differ outside the ambiguity band"
    sk = gpu["skipped"].cpu().numpy()
    np.testing.assert_array_equal(sk, (bits == 1).sum(axis=3))
    return int(amb.sum()), int((bits == 1).sum())
