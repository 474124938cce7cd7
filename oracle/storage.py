"""Exact decoding of stored K/V/Q values to float64, and rounding of float64
results to a storage dtype for reporting.  Test infrastructure only.

float32 and float16 values are exactly representable in float64.  bfloat16 is
held as uint16 bit patterns: the value is the float32 whose upper 16 bits are
those bits and whose lower 16 bits are zero (IEEE-754 binary32 truncated to
an 8-bit significand), again exact in float64.
"""

import numpy as np


def to_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype in ("f32", "f16"):
        return np.asarray(x).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> storage dtype, round to nearest, ties to even.

    float64 -> float32 -> bfloat16 double rounding can differ from a direct
    rounding only on exact float32 ties, which reporting does not care about.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        f = x.astype(np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        out = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        out[np.isnan(f)] = 0x7FC0
        return out
    raise ValueError(f"unknown dtype {dtype!r}")
