"""Host-side checks of bench.py (no GPU): the one-GPU contract and the CPU
baseline leg (the oracle timed on a bounded sample), including a packed batch
whose first sequence is timed and scaled to the batch."""
import os
import subprocess
import sys

import numpy as np

import bench
import synthetic
from oracle import cases as oc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_bench(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=e, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run_bench(["--gpus", "2"])
    assert r.returncode == 2 and "one GPU" in r.stderr
    r = _run_bench([], env={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_sample_single_and_packed():
    for case in (synthetic.config_case(2, scale_down=32), synthetic.config_case(5, scale_down=32)):
        count = oc.kap_case(case)["count"]
        cb = bench.cpu_baseline(case, count, seconds_target=1.0)
        assert cb["layer_seconds"] > 0 and np.isfinite(cb["layer_seconds"])
        assert cb["cores"] >= 1
        assert cb["blas"]["vendor"] not in (None, "")
        assert f"all {int(count.sum())} lists" in cb["sample"]
        assert f"{case.seqlens_q[0]} tokens of sequence 0" in cb["sample"]
