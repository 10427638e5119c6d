"""exp32: the fp32 exponential the proxy's MaxNorm step uses (oracle side).

The CoSA pages (§2.2, Block Ranking) turn max-pooled scores into "relative
ranking contributions" but give no numerics. To make the proxy's ranking
bit-reproducible between this oracle and the GPU, the exponential is fixed by a
specification of our own (not taken from any vendor library):

    exp32(x) = 0                      if not (x >= -87)   (also NaN and -inf)
    t = x (*) L,  L = fp32(log2 e)
    n = round-half-even(t);  f = t (-) n          (exact, |f| <= 1/2)
    p = c7;  p = (f (*) p) (+) c_k  for k = 6, ..., 0
    exp32(x) = p * 2**n

with c_k = fp32(ln(2)**k / k!) (the Taylor series of 2**f), and (*), (+), (-)
single IEEE-754 binary32 operations rounded to nearest even, never fused.
For x >= -87 the result is a normal float. NumPy float32 ufuncs round every
operation separately, which is exactly this specification.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = np.float32(math.log2(math.e))
COEFFS = tuple(np.float32(math.log(2.0) ** k / math.factorial(k)) for k in range(8))
LOWER = np.float32(-87.0)


def exp32(x) -> np.ndarray:
    """Elementwise exp32 of a float32 array (returns float32)."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        ok = x >= LOWER
        xs = np.where(ok, x, np.float32(0.0)).astype(np.float32)
        t = (xs * LOG2E).astype(np.float32)
        n = np.rint(t).astype(np.float32)
        f = (t - n).astype(np.float32)
        p = np.full_like(f, COEFFS[7])
        for k in range(6, -1, -1):
            p = (f * p).astype(np.float32)
            p = (p + COEFFS[k]).astype(np.float32)
        r = np.ldexp(p, n.astype(np.int32)).astype(np.float32)
    return np.where(ok, r, np.float32(0.0)).astype(np.float32)
