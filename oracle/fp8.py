"""OCP FP8 E4M3FN codec, written from the format's definition (test infrastructure).

The pages serve the model with FP8 weights in E4M3 format (intelliparadigm,
GLM4-MoE production optimisation, section 3.1 test configuration; Optimizing
GLM4-MoE for production, "Benchmark configuration": GLM-4.7 FP8). The OCP
E4M3FN layout used here:

    bit 7 sign | bits 6..3 exponent, bias 7 | bits 2..0 mantissa
    exponent 0      -> subnormal: m * 2^-9
    exponent 1..15  -> (1 + m/8) * 2^(exp-7); exponent 15 with m = 7 is NaN
    no infinities; largest finite magnitude 448.

Encoding is "nearest representable value, ties to the even code, saturate at
+-448", done by a lookup over the sorted table of all finite magnitudes.
"""
import numpy as np

E4M3_MAX = 448.0


def _decode_code(c: int) -> float:
    s = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_DECODE = np.array([_decode_code(c) for c in range(256)], dtype=np.float64)
# finite non-negative magnitudes, ascending, indexed by code 0..126
_MAGS = _DECODE[:127].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values."""
    return _DECODE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float values -> uint8 codes: round to nearest, ties to even code, saturate at 448.

    The sign bit is kept as the input's (a negative value that rounds to zero
    gives 0x80). NaN gives 0x7F.
    """
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_MAGS, a, side="left")       # first magnitude >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _MAGS[hi], hi, code)         # exact hits
    code = code.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)
