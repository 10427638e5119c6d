"""Benchmark of the CoSA prefill path on one MI355X.

One step = the whole hot path over one layer: the Kernel-Aware Proxy
(pool, proxy scores, rank/sort; cosa_kap_order) followed by the
Ordered-Skipping Kernel (cosa_osk_attention), inputs resident in HBM.
Default workload: a 131072-token causal prefill, 32 query / 8 KV heads,
head_dim 128, bf16, block 128, pool 16, budget 10%, skip threshold e^-16,
seeded synthetic inputs (rank-16 factors + noise, RoPE, sinks, 32 needle
blocks per KV head).

Prints one JSON line: effective TFLOP/s (dense-causal FLOPs / step time),
ms per layer, the dense baseline and speedup, the OSK's roofline (executed
tile FLOPs per launch / measured launch time vs the bf16 MFMA peak), and the
CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload cfg3]
                    [--budget B] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
METRIC = "ms/layer + effective TFLOP/s, 128K causal prefill at 10% budget; speedup vs dense"

WORKLOADS = {
    # name: (config number, default budget, description)
    "cfg1": (1, 0.25, "1K causal prefill, 1q/1kv head, d64, fp32, block 64, pool 8, 4 planted keys"),
    "cfg3": (3, 0.10, "128K causal prefill, 32q/8kv heads, d128, bf16, block 128, pool 16, 32 needle blocks/KV head"),
    "cfg2": (2, 0.10, "32K causal prefill, 32q/8kv heads, d128, bf16, block 128, pool 16"),
    "cfg4": (4, 0.10, "4K chunk over a 64K paged cache (shuffled pages), 32q/8kv, d128, bf16"),
    "cfg5": (5, 0.10, "ragged batch of 8 (4K-32K), 64q/8kv heads, d128, bf16"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="cfg3", choices=sorted(WORKLOADS))
    ap.add_argument("--budget", type=float, default=None)
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--sink-logit", type=float, default=None,
                    help="aligned-sink inputs (not the named workload)")
    ap.add_argument("--dense-steps", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (HBM counter calibration)")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="only time large bf16 matrix products (torch.matmul, the vendor GEMM): the "
                         "MFMA rate the box sustains, against which the walk's fraction of peak is read")
    ap.add_argument("--no-gemm", action="store_true",
                    help="skip the vendor-GEMM rate measured beside the walk (one 16384^3 product size)")
    return ap.parse_args()


def blas_info():
    """Vendor, version and thread count of the BLAS numpy calls into."""
    try:
        import numpy  # noqa: F401  (loads the BLAS that threadpoolctl then finds)
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return {"vendor": i.get("internal_api"), "version": i.get("version"),
                        "threads": i.get("num_threads"), "library": os.path.basename(i.get("filepath", ""))}
    except Exception:
        pass
    return {"vendor": "unknown", "version": None, "threads": os.cpu_count() or 1, "library": ""}


def gemm_ceiling(sizes=((8192, 8192, 8192), (16384, 16384, 16384)), reps=20, emit=True):
    """bf16 C = A.B with torch.matmul (hipBLASLt on ROCm) at large square sizes:
    TFLOP/s from HIP events around each of `reps` products after a warm-up."""
    import torch
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    out = []
    for (m, n, k) in sizes:
        g = torch.Generator(device="cpu").manual_seed(5)
        a = torch.randn((m, k), generator=g).to(dev, torch.bfloat16)
        b = torch.randn((k, n), generator=g).to(dev, torch.bfloat16)
        c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ms = []
        for _ in range(reps):
            e0.record(stream)
            torch.matmul(a, b, out=c)
            e1.record(stream)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        ms.sort()
        med = ms[len(ms) // 2]
        fl = 2.0 * m * n * k
        out.append({"m": m, "n": n, "k": k, "median_ms": med, "min_ms": ms[0],
                    "tflops_median": fl / (med * 1e-3) / 1e12, "tflops_best": fl / (ms[0] * 1e-3) / 1e12})
        print(f"[gemm] {m}x{n}x{k} bf16: median {med:.3f} ms = {out[-1]['tflops_median']:.0f} TFLOP/s "
              f"(best {out[-1]['tflops_best']:.0f})", file=sys.stderr, flush=True)
        del a, b, c
    if emit:
        print(json.dumps({"gemm_ceiling": out, "peak_bf16_tflops": MFMA_BF16_PEAK_TFLOPS}), flush=True)
    return out


OSK_SOURCE = os.path.join(ROOT, "block_sparse_attention_26_amd", "csrc", "osk_bf16.hip")
HBM_PROFILE = os.path.join(ROOT, "profiles", "hbm_counters_128k_b10.md")


def profiled_traffic():
    """HBM bytes per OSK launch from the committed counter summary, or None
    when the summary was taken on a different kernel source."""
    import hashlib
    import re

    try:
        src = hashlib.sha256(open(OSK_SOURCE, "rb").read()).hexdigest()
        text = open(HBM_PROFILE).read()
    except OSError:
        return None
    m_src = re.search(r"osk_bf16\.hip sha256: ([0-9a-f]{64})", text)
    m_val = re.search(r"osk HBM bytes per launch: ([0-9.eE+]+)", text)
    if not (m_src and m_val) or m_src.group(1) != src:
        return None
    return float(m_val.group(1))


def cpu_baseline(case, kap_count, seconds_target=20.0):
    """Time the oracle on KV group 0 of the first sequence: its whole proxy,
    then its ordered walk over evenly spaced query blocks until about
    `seconds_target` seconds of CPU work, and extrapolate to the whole layer
    (the proxy by its pooled score-matrix size summed over the sequences, the
    walk by listed blocks)."""
    import numpy as np
    from oracle import kap as okap, osk as oosk, layout

    blas = blas_info()
    cores = int(blas["threads"] or 1)
    G = case.h_q // case.h_kv
    B, p = case.block, case.pool
    T = case.seqlens_q[0]
    Lk = int(case.seqlens_k[0])
    qg = case.q[: T, :G].float().numpy()  # sequence 0 (packed first)
    kg = case.kv_contiguous(0, "k")[:, 0:1].float().numpy()
    vg = case.kv_contiguous(0, "v")[:, 0:1].float().numpy()
    kmax = layout.kmax(B, [T], [Lk], case.budget)
    t0 = time.perf_counter()
    ko = okap.kap_sequence(qg, kg, case.scale, B, p, case.budget, kmax, "fp64")
    t_kap = time.perf_counter() - t0
    nq = layout.cdiv(T, B)
    t_osk, done_blocks, done_q = 0.0, 0, []
    stride = max(1, nq // 128)  # up to 128 evenly spaced query blocks
    for qb in list(range(nq - 1, -1, -stride)):
        if t_osk > seconds_target / 2:
            break
        t0 = time.perf_counter()
        oosk.osk_sequence(qg, kg, vg, ko["order"], ko["count"], case.scale, case.tau, G, B, query_blocks=[qb])
        t_osk += time.perf_counter() - t0
        done_blocks += int(ko["count"][0, qb])
        done_q.append(qb)
    # every list of the layer (all KV groups); each is walked by G query heads,
    # as the sampled lists of group 0 were
    total_blocks = int(kap_count.sum())
    kap_scale = sum(lq * int(lk) for lq, lk in zip(case.seqlens_q, case.seqlens_k.tolist())) / (T * Lk)
    layer_s = t_kap * case.h_kv * kap_scale + t_osk * total_blocks / max(1, done_blocks)
    return {
        "layer_seconds": layer_s,
        "cores": int(cores),
        "blas": blas,
        "sample": (f"oracle (numpy fp64) proxy of KV group 0 over all {T} tokens of sequence 0 ({t_kap:.1f} s, "
                   f"x{case.h_kv} groups x{kap_scale:.2f} for the batch) "
                   f"+ ordered walk of KV group 0 ({G} query heads) over {len(done_q)} query blocks "
                   f"({done_blocks} listed blocks, {t_osk:.1f} s), extrapolated by listed-block count "
                   f"to all {total_blocks} lists of the layer"),
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.gemm_ceiling:
        gemm_ceiling()
        return

    import block_sparse_attention_26_amd as cosa
    import synthetic
    cfg_n, default_budget, desc = WORKLOADS[args.workload]
    budget = default_budget if args.budget is None else args.budget
    kw = {}
    if args.sink_logit is not None:
        kw["sink_logit"] = args.sink_logit
    t0 = time.perf_counter()
    case = synthetic.config_case(cfg_n, budget=budget, **kw)
    if args.tau is not None:
        case.tau = args.tau
    gen_s = time.perf_counter() - t0
    print(f"[bench] {args.workload}: inputs generated in {gen_s:.1f} s", file=sys.stderr, flush=True)

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    q, k, v = case.q.to(dev), case.k_pages.to(dev), case.v_pages.to(dev)
    pr = cosa.Problem.from_case(case, device=dev)
    d = pr.dims(case.pool, case.budget)
    kmax = d.kmax
    order = torch.empty((case.batch, case.h_kv, d.max_nq, kmax), dtype=torch.int32, device=dev)
    hrm = torch.empty(order.shape, dtype=torch.uint8, device=dev)
    count = torch.empty(order.shape[:3], dtype=torch.int32, device=dev)
    ws_bytes = cosa.cosa_kap_workspace_size(pr.c, case.pool, True)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    vis = torch.empty((case.batch, case.h_q, d.max_nq), dtype=torch.int32, device=dev)
    skp = torch.empty_like(vis)
    G = case.h_q // case.h_kv

    def kap():
        cosa.cosa_kap_order(pr.c, q.data_ptr(), k.data_ptr(), case.pool, case.budget, order.data_ptr(),
                            hrm.data_ptr(), count.data_ptr(), kmax, None, None, ws.data_ptr(), ws_bytes, sptr)

    def osk():
        cosa.cosa_osk_attention(pr.c, q.data_ptr(), k.data_ptr(), v.data_ptr(), order.data_ptr(),
                                count.data_ptr(), kmax, G, case.tau, o.data_ptr(), vis.data_ptr(),
                                skp.data_ptr(), None, None, sptr)

    for _ in range(args.warmup):
        kap()
        osk()
    torch.cuda.synchronize()
    visited = int(vis.sum())
    skipped = int(skp.sum())
    computed = visited - skipped
    listed = int(count.sum())
    print(f"[bench] warmup done: {listed} listed blocks, {visited} visited (x heads), {skipped} skipped",
          file=sys.stderr, flush=True)

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        kap()
        ev[i][1].record(stream)
        osk()
        ev[i][2].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / K
    kap_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    osk_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    step_ms = sorted(e[0].elapsed_time(e[2]) for e in ev)
    osk_sorted = sorted(e[1].elapsed_time(e[2]) for e in ev)
    med = lambda xs: xs[len(xs) // 2] if len(xs) % 2 else 0.5 * (xs[len(xs) // 2 - 1] + xs[len(xs) // 2])
    print(f"[bench] timed {K} steps: {ms_step:.3f} ms/step (kap {kap_ms:.3f}, osk {osk_ms:.3f})",
          file=sys.stderr, flush=True)

    dense_ms = None
    if not args.no_dense:
        od = torch.empty_like(q)
        KD = args.dense_steps or max(1, min(K, 5))
        cosa.cosa_dense_attention(pr.c, q.data_ptr(), k.data_ptr(), v.data_ptr(), od.data_ptr(), None, sptr)
        torch.cuda.synchronize()
        a_ev = torch.cuda.Event(enable_timing=True)
        b_ev = torch.cuda.Event(enable_timing=True)
        a_ev.record(stream)
        for _ in range(KD):
            cosa.cosa_dense_attention(pr.c, q.data_ptr(), k.data_ptr(), v.data_ptr(), od.data_ptr(), None, sptr)
        b_ev.record(stream)
        torch.cuda.synchronize()
        dense_ms = a_ev.elapsed_time(b_ev) / KD
        print(f"[bench] dense {dense_ms:.3f} ms", file=sys.stderr, flush=True)

    if args.calibrate_copy:
        # a plain copy of known size: reads and writes exactly 1 GiB each
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    B, D = case.block, case.head_dim
    dense_flops = cosa.dense_causal_flops(case.seqlens_q, case.seqlens_k.tolist(), case.h_q, D)
    eff_tflops = dense_flops / (ms_step * 1e-3) / 1e12
    # executed MFMA tile work of one OSK launch: every visited (head, query
    # block, KV block) pays a B x B x d QK^T tile, every computed one also P.V
    tile = 2.0 * B * B * D
    osk_flops = (visited + computed) * tile
    osk_tflops = osk_flops / (osk_ms * 1e-3) / 1e12
    peak = MFMA_BF16_PEAK_TFLOPS if case.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS

    gemm = None
    if not args.no_gemm and case.dtype == "bf16":
        g = gemm_ceiling(sizes=((16384, 16384, 16384),), reps=10, emit=False)[0]
        gemm = g["tflops_median"]
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        cb = cpu_baseline(case, count.cpu().numpy())
        print(f"[bench] cpu baseline: {time.perf_counter() - t0:.1f} s of oracle work", file=sys.stderr,
              flush=True)
        cpu = {
            "value": dense_flops / cb["layer_seconds"] / 1e12,
            "unit": "TFLOP/s (effective, dense-causal-equivalent)",
            "cores": cb["cores"],
            "blas": cb["blas"],
            "kind": "oracle",
            "sample": cb["sample"],
            "layer_seconds_extrapolated": cb["layer_seconds"],
        }

    line = {
        "metric": METRIC,
        "value": eff_tflops,
        "unit": "TFLOP/s (effective, dense-causal-equivalent)",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {
            "workload": desc if args.sink_logit is None else desc + f", aligned sinks {args.sink_logit} nats",
            "seq_len": int(case.seqlens_q[0]) if case.batch == 1 else case.seqlens_q,
            "kv_len": int(case.seqlens_k[0]) if case.batch == 1 else case.seqlens_k.tolist(),
            "batch": case.batch,
            "h_q": case.h_q, "h_kv": case.h_kv, "head_dim": D, "block": B, "pool": case.pool,
            "budget": case.budget, "skip_threshold": case.tau,
        },
        "ms_per_layer": ms_step,
        "ms_per_layer_median": med(step_ms),
        "ms_per_layer_min": step_ms[0],
        "kap_ms": kap_ms,
        "osk_ms": osk_ms,
        "osk_ms_median": med(osk_sorted),
        "osk_ms_min": osk_sorted[0],
        "dense_ms": dense_ms,
        "speedup_vs_dense": (dense_ms / ms_step) if dense_ms else None,
        "dense_tflops": (dense_flops / (dense_ms * 1e-3) / 1e12) if dense_ms else None,
        "listed_blocks": listed,
        "visited_head_blocks": visited,
        "skipped_head_blocks": skipped,
        "roofline": {
            "kernel": ("osk_bf16_kernel<128,128> (ordered-skip walk)" if case.dtype == "bf16"
                       else f"osk_kernel<fp32,{D},{B}> (ordered-skip walk)"),
            "bound": "mfma",
            "achieved": osk_tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": osk_tflops / peak,
            "traffic": profiled_traffic() if args.workload == "cfg3" and abs(case.budget - 0.1) < 1e-12 else None,
            "algorithmic_flops_per_launch": osk_flops,
            # the vendor GEMM (torch.matmul, 16384^3 bf16) timed in the same
            # process: what the box sustains on plain matrix work
            "measured_gemm_tflops": gemm,
            "frac_of_measured_gemm": (osk_tflops / gemm) if gemm else None,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
