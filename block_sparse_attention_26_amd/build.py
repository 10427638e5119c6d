"""Build libcosa.so (HIP kernels + C-ABI host layer) for gfx950 with hipcc.

    python -m block_sparse_attention_26_amd.build [--jobs N]

Each translation unit is compiled separately (in parallel) into
``block_sparse_attention_26_amd/_build/`` and linked into
``block_sparse_attention_26_amd/libcosa.so``. Always rebuilds.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcosa.so")
SOURCES = ["cosa_api.cpp", "osk.hip", "osk_bf16.hip", "kap.hip", "mask.hip", "mass.hip", "decode.hip", "cobs.hip"]

ARCH = "gfx950"
FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # packed fp32 VALU ops are kept out of every code object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall",
    "-Wno-unused-function",
    # MFMA results in arch VGPRs: the softmax works on them directly instead of
    # copying accumulators out of AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


# per-source additions to the flags
EXTRA = {}


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand) and shutil.which(cand) is None:
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libcosa")
    return cand


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        # keep real warnings visible; the host pass always notes the unknown
        # packed-fp32 feature, which is expected
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if any(l.strip() for l in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(jobs: int = 3, verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    # export only the C ABI (cosa_*): internal launchers stay local
    exports = os.path.join(OUT, "exports.map")
    with open(exports, "w") as f:
        f.write("{ global: cosa_*; local: *; };\n")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", f"-Wl,--version-script={exports}", "-o", tmp,
           *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=3)
    args = ap.parse_args()
    build(args.jobs, verbose=True)


if __name__ == "__main__":
    main()
