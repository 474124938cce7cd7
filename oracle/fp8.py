"""FP8 KV-cache codes: their values, and the quantiser that turns stored
16-bit K/V values into codes under one scale per tensor.  Test
infrastructure only.

Source: [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践",
section "工程边界与架构取舍": quantising the KV cache from FP16 to FP8 halves
its memory, and FP8 (rather than INT4) is the conservative choice for KV.
The page fixes neither the 8-bit format nor the scale; readings taken here:

* Format: OCP 8-bit floating point E4M3 ("e4m3fn"): 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits.  Exponent field 0 holds subnormals
  (m/8) * 2^-6; the pattern with all exponent and mantissa bits set is NaN;
  there are no infinities; the largest finite magnitude is 448.
* Scale: one float32 scale for the key pool and one for the value pool; a
  stored code c stands for value(c) * scale.
* Quantiser: y = float32(x) / float32(scale), an IEEE float32 division
  (rounded to nearest); y then goes to the nearest E4M3 value, ties to the
  code whose last bit is 0; magnitudes above 448 (infinity included)
  saturate to 448; NaN stays NaN; the sign of zero is kept.
"""

import numpy as np

FP8_MAX = 448.0


def _code_values() -> np.ndarray:
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * (m / 8.0) * 2.0**-6
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


# value of every code 0..255 (float64, exact)
E4M3_VALUES = _code_values()
_POS = E4M3_VALUES[:0x7F]  # codes 0x00..0x7E: the non-negative finite values, ascending


def fp8_value(codes) -> np.ndarray:
    """Codes (uint8) -> their values, float64, scale not applied."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def fp8_encode(y) -> np.ndarray:
    """Round values to E4M3 codes (nearest, ties to even code, saturating)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    # The two representable neighbours of each magnitude: lo <= a <= hi.
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    lo = np.where(_POS[hi] == a, hi, lo)  # exactly representable
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(a >= FP8_MAX, 0x7E, pick)  # saturate (448 itself is code 0x7E)
    code = pick.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << 7)
    code = np.where(np.isnan(y), np.uint8(0x7F) | (np.signbit(y).astype(np.uint8) << 7), code)
    return code.astype(np.uint8)


def fp8_quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """float16 (or float32) K/V values -> codes under ``scale``."""
    y = np.asarray(x).astype(np.float32) / np.float32(scale)
    return fp8_encode(y.astype(np.float32))


def fp8_dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """Codes -> float64 values the cache stands for (value * float32 scale)."""
    return fp8_value(codes) * np.float64(np.float32(scale))


def reshape_and_cache_fp8(key_cache, value_cache, key, value, slots, k_scale, v_scale) -> None:
    """The scatter into an FP8 pool: quantise each new token's K and V with
    the pool's scales, then write the codes to their slots (same slot rules as
    the 16-bit scatter)."""
    from .paging import reshape_and_cache

    reshape_and_cache(key_cache, value_cache, fp8_quantize(key, k_scale), fp8_quantize(value, v_scale), slots)
