"""The rounding margins that the 16-bit square-root kernels rely on, checked
with exact rational arithmetic over every positive finite 16-bit input.

For x a positive finite binary16 / bfloat16 value, let d be the distance
from sqrt(x) to the nearest rounding boundary (midpoint) of the 16-bit
format, in units of the binary32 ulp of sqrt(x).  A binary32 root within e
ulps of sqrt(x) narrows to the correctly rounded 16-bit root whenever
e < d.  binary16: d > 1/2, so the correctly rounded binary32 root (e <= 1/2)
narrows correctly -- the binary16 kernel selects it from the hardware root
and its neighbours.  bfloat16: d >= 32, so the hardware root (within one
ulp) narrows correctly with no refinement.
"""
from fractions import Fraction
import math

import numpy as np


def _margins(fmt):
    """Minimum over every positive finite pattern of d (see above)."""
    best = None
    for b in range(1, 1 << 15):
        if fmt == "f16":
            if (b & 0x7C00) == 0x7C00:
                continue
            v, p, emin = float(np.uint16(b).view(np.float16)), 11, -14
        else:
            if (b & 0x7F80) == 0x7F80:
                continue
            v, p, emin = float(np.array([b << 16], np.uint32).view(np.float32)[0]), 8, -126
        q = Fraction(v)
        r = math.sqrt(v)
        e = math.floor(math.log2(r))
        half = Fraction(2) ** (max(e, emin) - p)           # midpoints: odd multiples
        k = int(Fraction(r) / half)
        d = min(abs(q - (kk * half) ** 2) / (Fraction(r) + kk * half)
                for kk in range(k - 3, k + 4) if kk % 2)
        # sqrt(q) - m = (q - m^2) / (sqrt(q) + m); r approximates sqrt(q) to
        # ~1e-16 relative, far below the margins measured here
        m = d / Fraction(2) ** (e - 23)
        best = m if best is None or m < best else best
    return float(best)


def test_binary16_roots_are_more_than_half_a_binary32_ulp_from_a_midpoint():
    assert 0.5 < _margins("f16") < 0.6


def test_bfloat16_roots_are_at_least_32_binary32_ulps_from_a_midpoint():
    assert _margins("bf16") >= 32.0
