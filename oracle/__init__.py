"""CPU oracle for the CoSA prefill path (test infrastructure only).

This package is the slow, plain reference that the HIP library is checked
against. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import it; the product path never calls into it and it
never calls into the product path (it shares no code with the HIP sources).

Sources. The method is CoSA as summarised on the gist.science pages
"CoSA: Accelerating Long-Context Inference via Proxy-Kernel Co-Designed Sparse
Attention" (English technical summary, with Dutch and Italian versions):

* §2.1 Core Design Principles: online-softmax accumulation does not depend on
  the order key blocks are visited in; the proxy emits a computation-order
  mask instead of a binary one.
* §2.2 Stage 1, Kernel-Aware Proxy: downsample Q and K, approximate scores,
  MaxPool over keys, MaxNorm, "Have Rowmax" (HRM) flags, flag-grouped sort
  under a budget.
* §2.3 Stage 2, Ordered-Skipping Kernel: unselected blocks are never visited
  (page remapping), retained blocks may be skipped in-kernel by comparing the
  local and running row maxima, the rest is computed.
* §1 Problem Statement: the skip veto is per tile (one outlier row blocks the
  skip for the whole tile, the "bucket effect"), and the running max is a
  lower bound of the global max.

Where the pages leave a step open, the oracle takes one stated reading (listed
in each module's docstring and collected in the design notes).

Modules:
    exp32  - the proxy's fp32 exponential (our own specification).
    dense  - dense causal softmax attention in fp64 (textbook definition).
    kap    - the Kernel-Aware Proxy: pooling, proxy scores, MaxNorm, HRM,
             flag-grouped sort and budget truncation.
    osk    - ordered online-softmax accumulation with the in-kernel skip rule.
    masks  - binary block masks <-> ascending lists, block-union tables,
             exact block attention mass and the recall of a selection
             (comparison modes).
    decode - the decode-stage walk: one query token, the list cut into
             segments walked separately and merged by log-sum-exp.
    cobs   - second-order block scores (mean + half variance of the scores
             over a block's keys) as an alternative proxy ranking.
    layout - causal block arithmetic and page gathering used by the above.
    cases  - convenience wrappers that run the oracle on a whole packed batch.
"""
from . import exp32, dense, kap, osk, masks, decode, cobs, layout, cases  # noqa: F401
