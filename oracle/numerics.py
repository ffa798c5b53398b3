"""Storage-precision rounding used by the oracle.

The method stores some intermediate tensors (index keys, chunk/group
summaries, coarse pyramid levels) in the workload element type.  Where a
later selection decision is taken on those stored values, the oracle rounds
its exact fp64 value once, round-to-nearest-even, to the same element type.
"""
import numpy as np


def round_bf16(x):
    """Round fp64 values to the nearest bfloat16 (ties to even), as fp64.

    bfloat16 keeps 8 significant bits; frexp gives x = m * 2**e with
    0.5 <= |m| < 1, so m * 2**8 carries exactly those bits and np.rint rounds
    the rest half-to-even.  Overflow and subnormals are out of range for the
    magnitudes used here and are not special-cased.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def round_fp32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_store(x, dtype):
    """Round to the stored element type: "bf16" or "fp32"."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return round_fp32(x)
    raise ValueError(dtype)


def bf16_ulp(x):
    """Spacing of bfloat16 values at |x| (for 1-ulp tolerances)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.maximum(x, 1e-30))
    return np.ldexp(1.0, e - 8)
