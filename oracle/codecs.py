"""Number-format codecs for the oracle, written from the format definitions.

Test infrastructure only (see ``oracle/__init__.py``).

Formats (OCP 8-bit Floating Point Specification; OCP Microscaling (MX) Formats v1.0):

* e4m3fn ("FP8-e4m3" of the EpiLoRA abstract, which names FP8 weights): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal with
  step 2^-9; there is no infinity; the all-ones pattern S.1111.111 is NaN, so the
  largest finite magnitude is 1.75 * 2^8 = 448.
* e2m1 (the MXFP4 element, the "4-bit format" of the EpiLoRA abstract): 1 sign bit,
  2 exponent bits with bias 1, 1 mantissa bit; magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
* e8m0 (the MX shared scale): an unsigned biased exponent, value 2^(c-127); c = 255
  is NaN.
* bf16: the upper 16 bits of an IEEE binary32.

All decoders return float64 numpy arrays; they are exact (every code is a dyadic
rational well inside binary64).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_SUBNORMAL = 2.0 ** -9
E4M3_MIN_NORMAL = 2.0 ** -6
E2M1_MAX = 6.0


def decode_e4m3fn(codes) -> np.ndarray:
    """Decode e4m3fn codes (uint8) to float64; NaN codes decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** -9
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def decode_e2m1(nibbles) -> np.ndarray:
    """Decode e2m1 nibbles (values 0..15 in any integer array) to float64."""
    n = np.asarray(nibbles).astype(np.int64) & 0xF
    sign = np.where((n >> 3) & 1, -1.0, 1.0)
    e = (n >> 1) & 0x3
    m = n & 0x1
    sub = m * 0.5
    nrm = (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    return sign * np.where(e == 0, sub, nrm)


def decode_e8m0(codes) -> np.ndarray:
    """Decode e8m0 scale codes to float64 powers of two; 255 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def bf16_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def encode_e4m3fn_rne(values) -> np.ndarray:
    """Encode float64 values with |v| <= 448 to e4m3fn codes, round to nearest even.

    Magnitudes below the smallest normal 2^-6 lie on the subnormal grid of step
    2^-9 (grid index 8 is the smallest normal, whose code is also 8).  In binade
    2^e (e >= -6) the grid step is 2^(e-3); a significand that rounds up to 2^(e+1)
    moves to the next binade.  The sign bit is kept, also for results that round
    to zero.  All divisions are by powers of two, hence exact, and ``np.rint``
    rounds halves to even.  Inputs beyond +-448 or NaN raise ValueError (the MX rule
    clamps before encoding).
    """
    v = np.asarray(values, dtype=np.float64)
    if np.isnan(v).any() or (np.abs(v) > E4M3_MAX).any():
        raise ValueError("e4m3fn encode: values outside [-448, 448]")
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    a = np.abs(v)
    sub = a < E4M3_MIN_NORMAL
    k_sub = np.rint(a / E4M3_MIN_SUBNORMAL).astype(np.int64)
    _, e = np.frexp(np.where(sub, 1.0, a))
    exp = e.astype(np.int64) - 1
    r = np.rint(np.ldexp(np.where(sub, 1.0, a), -(exp - 3).astype(np.int32))).astype(np.int64)
    carry = r == 16
    exp = np.where(carry, exp + 1, exp)
    r = np.where(carry, 8, r)
    k_nrm = ((exp + 7) << 3) | (r - 8)
    return (sign | np.where(sub, k_sub, k_nrm)).astype(np.uint8)


def e4m3fn_finite_values() -> np.ndarray:
    """All 127 non-negative finite e4m3fn magnitudes in code order (0x00..0x7E)."""
    return decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
