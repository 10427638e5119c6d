"""The committed profile summaries describe the kernels in the tree.

Every summary under profiles/ names the kernel sources it was taken on by
their sha256 ("<file> sha256: <hex>"). A kernel edited after its profile was
taken makes that summary (and the bench's HBM traffic figure, read from it)
describe other code; this test names the stale summary and source.
"""
import hashlib
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "block_sparse_attention_26_amd", "csrc")


def _recorded():
    out = []
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith(".md"):
            continue
        text = open(os.path.join(PROFILES, name)).read()
        for src, digest in re.findall(r"^([\w.]+\.(?:hip|cpp|h)) sha256: ([0-9a-f]{64})\s*$", text, re.M):
            out.append((name, src, digest))
    return out


def test_profiles_name_their_sources():
    rec = _recorded()
    assert rec, "no profile summary records the sha256 of its kernel sources"
    # the walk's and the proxy's summaries name both kernel sources
    files = {(p, s) for p, s, _ in rec}
    for prof in ("kernel_trace_128k_b10.md", "hbm_counters_128k_b10.md", "sq_counters_128k_b10.md"):
        assert (prof, "osk_bf16.hip") in files and (prof, "kap.hip") in files, prof


@pytest.mark.parametrize("prof,src,digest", _recorded(), ids=lambda x: x if isinstance(x, str) and len(x) < 40 else "")
def test_profile_matches_source(prof, src, digest):
    path = os.path.join(CSRC, src)
    assert os.path.exists(path), f"{prof} names {src}, which is not in the tree"
    now = hashlib.sha256(open(path, "rb").read()).hexdigest()
    assert now == digest, f"{prof} was taken on another version of {src}: re-take it after changing the kernel"
