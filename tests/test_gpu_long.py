"""GPU parity at long contexts, up to the proxy's limit of 4096 KV blocks per
sequence (B = 64, 262144 cached tokens), through the C ABI.

The proxy's sort network holds 256*E keys, E in {1, 2, 4, 8, 16} by the
number of causal blocks; these chunked cases reach E = 2, 4, 8 and 16 (the
other tests stay at or below 1024 blocks). Checked: proxy lists, HRM flags,
counts and block scores bit-exact against the oracle fed the GPU's fp32
scores, each score within its a-priori rounding bound of the fp64 oracle, the
ordered walk against the oracle, and the same for a decode step over the
longest cache.

The proxy rounds pooled queries and keys to bf16 and sums their products in
fp32. Per entry, |P - P64| is then at most scale * [(2u + u^2) * sum_d |qbar_d|
|kbar_d| + e_acc] for the window that attains the max (u = 2^-8, the bf16 unit
roundoff), where e_acc covers the fp32 pooling and the d-term fp32 sum
(both at most d * 2^-24 of the mean absolute operands). At 4096 blocks the
maximum over all entries reaches 1.5% of max |P|, so a tolerance relative to
max |P| is not a bound; the per-entry one is, and it stays near 0.5% of |P|.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_26_amd as cosa
import synthetic
from oracle import cases as oc, decode as odec, kap as okap
from gpu_common import OnDevice, check_output, check_skip_sets, require_gpu, say

pytestmark = pytest.mark.gpu

# cached tokens -> causal blocks of the last query block at B = 64:
# 20000 -> 313 (E = 2), 60000 -> 938 (4), 100000 -> 1563 (8), 262144 -> 4096 (16)
LENGTHS = [20000, 60000, 100000, 262144]


def _case(lk, lq=200, seed=70):
    return synthetic.lowrank_case(seed, [lq], [lk], h_q=4, h_kv=2, head_dim=64, block=64, pool=16, budget=0.1,
                                  sink_logit=24.0, name=f"long-{lk}")


def _rounding_bound(case):
    """Per-entry bound on |P_gpu - P_fp64| from bf16 rounding of the pooled
    operands and fp32 summation, [batch, h_q, max_nr, max_nk] (0 where unused)."""
    dm = oc.dims(case)
    B, p, G = case.block, case.pool, case.h_q // case.h_kv
    per = B // p
    u = 2.0 ** -8
    acc = case.head_dim * 2.0 ** -23  # fp32 pooling plus the d-term fp32 sum
    out = np.zeros((case.batch, case.h_q, dm["max_nr"], dm["max_nk"]))
    for b in range(case.batch):
        if case.seqlens_q[b] == 0:
            continue
        q, k, _ = oc.sequence_inputs(case, b)
        qm, km = np.abs(okap.pool_tokens(q, case.pool)), np.abs(okap.pool_tokens(k, case.pool))
        qa, ka = okap.pool_tokens(np.abs(q), p), okap.pool_tokens(np.abs(k), p)
        nr, nk = qm.shape[0], -(-int(case.seqlens_k[b]) // B)
        for h in range(case.h_q):
            e = (2 * u + u * u) * (qm[:, h] @ km[:, h // G].T) + acc * (qa[:, h] @ ka[:, h // G].T)
            pad = np.zeros((nr, nk * per))
            pad[:, : e.shape[1]] = e
            out[b, h, :nr, :nk] = case.scale * pad.reshape(nr, nk, per).max(axis=2)
    return out


@pytest.mark.parametrize("lk", LENGTHS)
def test_long_context_proxy_and_walk(lk):
    require_gpu()
    case = _case(lk)
    say("long context", lk, "pages", tuple(case.k_pages.shape))
    dev = OnDevice(case)
    k = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, case.budget, export_scores=True,
                       export_block_scores=True)
    torch.cuda.synchronize()
    P = k["P"].cpu().numpy()
    ref = oc.kap_case(case, precision="fp32", P_given=P)
    for name in ("order", "hrm", "count"):
        np.testing.assert_array_equal(k[name].cpu().numpy(), ref[name], err_msg=name)
    s = k["s"].cpu().numpy()
    assert np.array_equal(s.view(np.uint32), ref["s"].astype(np.float32).view(np.uint32)), "block scores"
    P64 = oc.kap_case(case, precision="fp64")["P"]
    fin = np.isfinite(P64)
    assert np.array_equal(np.isfinite(P), fin)
    err = np.abs(P[fin] - P64[fin])
    bound = _rounding_bound(case)[fin]
    assert np.all(err <= bound), f"score error {err.max():.3e}, worst error/bound {(err / bound).max():.3f}"
    say("long context", lk, "walk")
    g = cosa.osk_attention(dev.problem, dev.q, dev.k, dev.v, k["order"], k["count"], case.tau, skip_bits=True)
    torch.cuda.synchronize()
    oref = oc.osk_case(case, ref["order"], ref["count"])
    check_output(g["O"], oref["O"], case.dtype, f"long {lk}")
    check_skip_sets(g, oref, ref["count"], case.h_q // case.h_kv)


def test_long_context_decode():
    require_gpu()
    case = synthetic.lowrank_case(71, [1, 1], [262144, 100000], h_q=4, h_kv=2, head_dim=64, block=64, pool=16,
                                  budget=0.1, sink_logit=24.0, per_sequence_seeds=True, name="long-decode")
    say("long decode", tuple(case.k_pages.shape))
    dev = OnDevice(case)
    k = cosa.kap_order(dev.problem, dev.q, dev.k, case.pool, case.budget, export_scores=True)
    g = cosa.osk_decode(dev.problem, dev.q, dev.k, dev.v, k["order"], k["count"], case.tau, 4)
    torch.cuda.synchronize()
    ref = oc.kap_case(case, precision="fp32", P_given=k["P"].cpu().numpy())
    for name in ("order", "hrm", "count"):
        np.testing.assert_array_equal(k[name].cpu().numpy(), ref[name], err_msg=name)
    dref = odec.decode_case(case, ref["order"], ref["count"], 4)
    check_output(g["O"], dref["O"], case.dtype, "long decode")
    np.testing.assert_array_equal(g["visited"].cpu().numpy()[:, :, 0], dref["visited"])
