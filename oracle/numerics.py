"""Storage semantics shared by every oracle stage (test infrastructure only).

bf16 has an 8-bit significand (7 stored bits plus the implicit one) and the
float32 exponent range. Widening bf16 to float64 is exact; rounding a float64
to bf16 keeps 8 significant bits, ties to even.
"""

from __future__ import annotations

import numpy as np


def widen(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of a stored tensor.

    ``uint16`` arrays hold bf16 bit patterns: the bf16 value is the float32
    whose top 16 bits are the pattern and whose low 16 bits are zero.
    Anything else is taken as a float array.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even).

    Written from the format's definition: write x = f * 2**e with
    0.5 <= |f| < 1 (``frexp``), keep 8 significant bits of f by rounding
    f * 2**8 to the nearest integer with ties to even (``rint``), and scale
    back. Zeros stay zero. Values below the bf16 normal range do not occur in
    the seeded workloads' data and are not treated specially.
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    q = np.rint(f * 256.0)
    return np.ldexp(q / 256.0, e)
