"""bf16 rounding and ulp, float64 in and out.

bf16 keeps 8 significant bits (a 7-bit stored mantissa); the AstrAI paper's
"BF16 dead zone" paragraph puts its ulp at 1.0 at 2^-7.  Rounding is IEEE 754
round-to-nearest, ties to even (the paper cites IEEE 754 for the format).
Normal range only: results below 2^-126 in magnitude or above the bf16 maximum
do not occur in these workloads and are not modelled.
"""

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value of each float64 ``x`` (ties to even), as float64."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)               # x = m * 2**e with 0.5 <= |m| < 1
    # m * 2**8 has 8 integer bits; rint rounds half to even.
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def ulp_bf16(y) -> np.ndarray:
    """Spacing of bf16 numbers at |y|: 2**(floor(log2|y|) - 7); 2**-133 at 0."""
    y = np.abs(np.asarray(y, dtype=np.float64))
    _, e = np.frexp(y)               # y = m * 2**e, floor(log2 y) = e - 1
    u = np.ldexp(1.0, e - 1 - 7)
    return np.where(y == 0, np.ldexp(1.0, -133), u)
