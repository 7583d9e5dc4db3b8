"""Round-to-nearest-even of float64 values into narrower binary formats.

TEST INFRASTRUCTURE ONLY (part of the CPU oracle): used by the storage-faithful
evaluation of the Newton-Schulz iteration, which rounds at the points where a
half-precision implementation stores a matrix. The DeepSpeed-Muon article
(section on the Newton-Schulz kernels) runs the standard quintic in bf16 and the
Gram variant in fp16; neither it nor the other pages fix a rounding mode, so
IEEE round-to-nearest-even is taken, applied once, directly from float64.
"""
from __future__ import annotations

import numpy as np

# (precision p including the implicit bit, minimum normal exponent, maximum exponent)
FORMATS = {
    "bf16": (8, -126, 127),
    "f16": (11, -14, 15),
    "f32": (24, -126, 127),
}


def round_to(x, fmt: str) -> np.ndarray:
    """Nearest value of format `fmt` (ties to even), returned as float64.

    Finite values whose rounded magnitude exceeds the format's largest finite
    value become signed infinity; NaN and infinities pass through; signs of
    zeros are kept.
    """
    p, emin, emax = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)                       # xf = f * 2**e with 0.5 <= |f| < 1
    lead = np.maximum(e - 1, emin)            # exponent of the leading bit (clamped: subnormals)
    quantum = np.ldexp(1.0, lead - (p - 1))   # spacing of the format at that exponent
    r = np.round(xf / quantum) * quantum      # exact scaling; numpy rounds half to even
    max_finite = (2.0 - 2.0 ** (1 - p)) * 2.0 ** emax
    r = np.where(np.abs(r) > max_finite, np.copysign(np.inf, xf), r)
    return np.where(finite, r, x)


def storer(fmt):
    """A function that stores a matrix in `fmt` (None: keep float64)."""
    if fmt is None or fmt == "f64":
        return lambda z: z
    return lambda z: round_to(z, fmt)
