"""Rounding of float64 values to a narrower IEEE-style binary format.

TEST INFRASTRUCTURE ONLY (see the package docstring).

round_to_format(a, fmt) returns the float64 value of the nearest number of
format fmt ("f32", "f16" or "bf16"), ties to even, with gradual underflow
(subnormals spaced 2^(emin - mantissa bits)) and overflow to infinity.  It is
the rounding a device applies when it stores a value in that format; the
oracle uses it only where the layer keeps a value in its storage dtype (see
``layer_forward(store=...)``).
"""

import numpy as np

_FORMATS = {  # mantissa bits, smallest normal exponent, largest exponent
    "f32": (23, -126, 127),
    "f16": (10, -14, 15),
    "bf16": (7, -126, 127),
}


def round_to_format(a, fmt):
    mbits, emin, emax = _FORMATS[fmt]
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)                       # a = m 2^e with 1/2 <= |m| < 1
    lead = np.maximum(e - 1, emin)           # exponent of the leading bit (clamped: subnormals)
    q = np.ldexp(1.0, lead - mbits)          # spacing of the format around a
    r = np.round(a / q) * q                  # a / q is exact; np.round ties to even
    largest = np.ldexp(2.0 - np.ldexp(1.0, -mbits), emax)
    r = np.where(np.abs(r) > largest, np.copysign(np.inf, a), r)
    return np.where(np.isfinite(a), r, a)
