"""Number formats and rounding used by the oracle (plain NumPy, written for reading).

Test infrastructure only: see the package docstring for who may import it.

* fp16 scales are stored with round-to-nearest-even and saturate to the largest
  finite fp16 (a reading: the pages only say scales are fp16, "Runtime-Certified
  Bounded-Error Quantized Attention", Methodology section 1; the explicit
  saturation keeps the format total).
* E4M3 is the OCP "E4M3FN" byte (bias 7, no infinities, 0x7F/0xFF are NaN,
  largest finite 448) used as the per-16 block scale of NVFP4 in "Search Your
  Block Floating Point Scales!", Problem statement.  The value table is built by
  enumerating all 256 bit patterns.
* E2M1 is the 4-bit FP4 element of the same format: magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}; the largest magnitude 6 is the one the page maps
  the block absmax onto (Methodology, ScaleSearch mechanism).
"""

import numpy as np

F16_MAX = 65504.0


def f32(x):
    """Round to IEEE binary32 (round-to-nearest-even), elementwise."""
    return np.asarray(x, dtype=np.float32)


def f16_sat(x):
    """fp32 -> fp16 with round-to-nearest-even, saturating to +-65504.

    NumPy's float32->float16 cast is IEEE round-to-nearest-even; values that
    round past the largest finite fp16 are clamped to it instead of becoming inf.
    Returns a float16 array.
    """
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16)
    h = np.where(np.isinf(h), np.copysign(np.float16(F16_MAX), h), h).astype(np.float16)
    return h


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32 values (exact widening)."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def f16_bits_to_f32(bits):
    """fp16 bit patterns (uint16) -> float32 values (exact widening)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def widen_input(bits, dtype):
    """Input vectors (as uint16 bit patterns) -> exact float32 values.

    The write side widens the new K/V head vector to fp32 in registers before
    the sign flip ("When Quantization Is Free", Methodology section 2, load and
    sign step).  Both fp16 and bf16 widen exactly.
    """
    if dtype == "f16":
        return f16_bits_to_f32(bits)
    if dtype == "bf16":
        return bf16_bits_to_f32(bits)
    raise ValueError(dtype)


# ---------------------------------------------------------------- E4M3 (OCP FN)
def e4m3_table():
    """Value of each of the 256 E4M3FN bit patterns (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3_table()
_E4M3_POS = _E4M3[:0x7F]  # codes 0x00..0x7E: non-negative finite, increasing


def e4m3_encode_nonneg(v):
    """Non-negative float -> E4M3 code, round-to-nearest-even, saturating to 448.

    Ties between two neighbouring codes go to the code whose last mantissa bit
    is 0.  Anything at or above 448 encodes as 448 (0x7E).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode_nonneg expects non-negative finite values")
    idx = np.searchsorted(_E4M3_POS, v, side="left")  # first value >= v
    idx = np.clip(idx, 0, len(_E4M3_POS) - 1)
    lo = np.clip(idx - 1, 0, len(_E4M3_POS) - 1)
    dv_hi = _E4M3_POS[idx] - v
    dv_lo = v - _E4M3_POS[lo]
    pick_lo = (dv_lo < dv_hi) | ((dv_lo == dv_hi) & ((lo & 1) == 0))
    code = np.where(v >= _E4M3_POS[idx], idx, np.where(pick_lo, lo, idx))
    code = np.where(v >= _E4M3_POS[-1], len(_E4M3_POS) - 1, code)
    return code.astype(np.uint8)


def e4m3_value(code):
    return _E4M3[np.asarray(code, dtype=np.int64)]


# ---------------------------------------------------------------- E2M1 (FP4)
def e2m1_table():
    """Value of each of the 16 E2M1 bit patterns (sign bit 3, exponent bits 1-2,
    mantissa bit 0, exponent bias 1, exponent field 0 is subnormal)."""
    vals = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        m = code & 0x1
        vals[code] = sign * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return vals


_E2M1 = e2m1_table()
E2M1_MAG = _E2M1[:8]  # 0, 0.5, 1, 1.5, 2, 3, 4, 6


def e2m1_quantize(y, s):
    """Nearest E2M1 code to y / s (exact quotient), ties to the even code.

    y: float32 array; s: positive scale values broadcastable to y.  Magnitudes
    above 6 saturate to 6.  The sign bit is the IEEE sign bit of y (so -0.0 and
    small negatives that round to zero keep the sign bit).  Comparisons are made
    between |y| and (midpoint x s), both exact in fp64 (midpoints have at most
    3 significant bits, s at most 4, y at most 24).
    """
    y = np.asarray(y, dtype=np.float32)
    ay = np.abs(y).astype(np.float64)
    s = np.asarray(s, dtype=np.float64)
    mids = (E2M1_MAG[:-1] + E2M1_MAG[1:]) / 2.0  # 0.25 .. 5.0
    idx = np.zeros(y.shape, dtype=np.int64)
    for j, mid in enumerate(mids):
        t = mid * s
        idx += ay > t
        if j % 2 == 1:  # tie between j (odd) and j+1 (even): take j+1
            idx += ay == t
    sign = np.signbit(y).astype(np.int64)
    return (sign << 3 | idx).astype(np.uint8)


def e2m1_value(code):
    return _E2M1[np.asarray(code, dtype=np.int64)]


def rne_quotient(y, s):
    """Round-half-to-even of the exact real quotient y / s.

    y is fp32, s an fp16 or fp32 value (<= 24 significant bits): the fp64
    quotient cannot land on a half-integer unless the exact quotient is one, so
    np.rint of the fp64 quotient is the exact RNE (ties to even) result.
    """
    return np.rint(np.asarray(y, dtype=np.float64) / np.asarray(s, dtype=np.float64))
