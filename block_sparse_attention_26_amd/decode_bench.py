"""Decode-step measurement on one GPU: one new token per sequence against a
long KV cache, through the library's C ABI.

For a batch of sequences (default 8 x 131072 cached tokens, 32 query / 8 KV
heads, head_dim 128, bf16, block 128, pool 16, budget 10%, tau e^-16) it times
the proxy two ways - cosa_kap_order re-pooling the whole cache, and the
decode-loop form that keeps pooled keys (cosa_kap_pool_keys on each
sequence's last block, then cosa_kap_order_pooled) - the split decode walk
(cosa_osk_decode) for several segment counts, and the same walk over every
causal block with skipping off (dense decode). The walk is bandwidth-bound: its roofline is the K and V
bytes of the walked pages over the 8 TB/s HBM peak.

    python -m block_sparse_attention_26_amd.decode_bench [--batch 8] [--context 131072]
        [--budget 0.1] [--splits 1,2,4,8,16] [--sink-logit X] [--reps 10]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HBM_PEAK_GBS = 8000.0


def _log(*a):
    print("[decode]", *a, file=sys.stderr, flush=True)


def _timed(fn, reps, stream):
    """Mean device time per call over `reps` back-to-back calls between one
    pair of events (the host enqueues the next call while the device runs the
    previous one, so per-call host work does not count as device time)."""
    import torch
    out = fn()  # warm
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        out = fn()
    b.record(stream)
    torch.cuda.synchronize()
    return out, a.elapsed_time(b) / reps


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--context", type=int, default=131072)
    ap.add_argument("--budget", type=float, default=0.1)
    ap.add_argument("--tau", type=float, default=math.exp(-16.0))
    ap.add_argument("--splits", default="1,2,4,8,16")
    ap.add_argument("--sink-logit", type=float, default=None)
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args(argv)

    import torch

    sys.path.insert(0, ROOT)
    import block_sparse_attention_26_amd as cosa
    import synthetic

    if not torch.cuda.is_available():
        raise SystemExit("the decode measurement runs on a GPU")
    kw = {} if args.sink_logit is None else {"sink_logit": args.sink_logit}
    case = synthetic.lowrank_case(4000, [1] * args.batch, [args.context] * args.batch, budget=args.budget,
                                  tau=args.tau, per_sequence_seeds=True, name="decode", **kw)
    _log(f"batch {args.batch} x {args.context} cached tokens generated")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    q, k, v = case.q.to(dev), case.k_pages.to(dev), case.v_pages.to(dev)
    pr = cosa.Problem.from_case(case, device=dev)
    d = pr.dims(case.pool, case.budget)
    tile_bytes = case.block * case.head_dim * 2  # one K or V slab of a page and KV head
    ka, kap_ms = _timed(lambda: cosa.kap_order(pr, q, k, case.pool, case.budget), args.reps, stream)
    pooled = cosa.pool_keys(pr, k, case.pool)  # the decode loop's standing pooled keys

    def proxy_step():
        cosa.pool_keys(pr, k, case.pool, out=pooled, last_block_only=True)
        return cosa.kap_order(pr, q, k, case.pool, case.budget, pooled_keys=pooled)

    kp, kap_pooled_ms = _timed(proxy_step, args.reps, stream)
    for name in ("order", "hrm", "count"):
        assert torch.equal(kp[name], ka[name]), name  # same lists either way
    full = cosa.order_from_mask(pr, None, d.max_nk, device=dev)
    dn, dense_ms = _timed(lambda: cosa.osk_decode(pr, q, k, v, full["order"], full["count"], 0.0, 16),
                          args.reps, stream)
    O_ref = dn["O"].float()
    listed = int(ka["count"].sum())
    causal = int(full["count"].sum())
    meta = {"workload": f"decode step, {args.batch} sequences x {args.context} cached tokens, 32q/8kv heads, "
                        f"d128, bf16, block 128, pool 16",
            "batch": args.batch, "context": args.context, "budget": case.budget, "skip_threshold": case.tau,
            "listed_blocks": listed, "causal_blocks": causal}
    rows = [{"mode": "dense-decode", "walk_ms": dense_ms, "splits": 16,
             "hbm_gbs": causal * 2 * tile_bytes / (dense_ms * 1e-3) / 1e9}]
    rows[0]["hbm_frac"] = rows[0]["hbm_gbs"] / HBM_PEAK_GBS
    _log(f"proxy {kap_ms:.3f} ms re-pooling the cache, {kap_pooled_ms:.3f} ms with kept pooled keys; "
         f"dense decode {dense_ms:.3f} ms ({rows[0]['hbm_gbs']:.0f} GB/s)")
    for S in [int(x) for x in args.splits.split(",")]:
        res, ms = _timed(lambda: cosa.osk_decode(pr, q, k, v, ka["order"], ka["count"], case.tau, S),
                         args.reps, stream)
        visited = int(res["visited"].sum())
        skipped = int(res["skipped"].sum())
        err = res["O"].float() - O_ref
        row = {"mode": "cosa-decode", "splits": S, "walk_ms": ms, "proxy_ms": kap_ms,
               "proxy_pooled_ms": kap_pooled_ms, "step_ms": kap_pooled_ms + ms,
               "hbm_gbs": listed * 2 * tile_bytes / (ms * 1e-3) / 1e9,
               "visited": visited, "skipped": skipped,
               "rel_l2_vs_dense": float(err.norm() / O_ref.norm())}
        row["hbm_frac"] = row["hbm_gbs"] / HBM_PEAK_GBS
        rows.append(row)
        _log(f"splits {S:3d}: walk {ms:.4f} ms, {row['hbm_gbs']:.0f} GB/s ({100 * row['hbm_frac']:.1f}% of HBM), "
             f"skipped {skipped}/{visited}, rel L2 vs dense {row['rel_l2_vs_dense']:.3e}")
    for r in rows:
        r["config"] = meta
        print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
