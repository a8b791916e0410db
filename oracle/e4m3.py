"""E4M3 element format: table-driven decoder and encoder (oracle).

TEST INFRASTRUCTURE ONLY -- not part of the product path.

What the pages fix about the format
  * 1 sign, 4 exponent and 3 mantissa bits, used for weights and
    activations ("[vLLM] FP8", introduction and the format table in the
    paper summary; "FP8 and FP4: Throughput Needs Scaling", E4M3 vs E5M2).
  * No infinity is encoded, which buys range ("[vLLM] FP8", paper summary).
  * The largest magnitude is 448 ("[vLLM] FP8" format table;
    "fp8-serving-slower-than-bf16", hardware-generation section gives the
    range as [-448, 448]).

Reading taken where the pages stop (all forced or the plainest reading):
  * Exponent bias 7.  448 = 1.75 * 2**8 needs the top exponent field (15)
    to hold finite numbers, i.e. 15 - bias = 8.  With the top field
    reserved the maximum would be 1.875 * 2**7 = 240 instead.
  * Hence only the pattern S.1111.111 is NaN (codes 0x7F and 0xFF).
  * Exponent field 0 holds subnormals m * 2**-9 (the usual IEEE-style
    gradual underflow, which the same closed form gives).
  * Encoding: round to nearest, ties to the even code (even mantissa),
    saturating: magnitudes above 448, and infinities, map to 448.  NaN maps
    to the NaN code with the input's sign.  The sign bit is kept for zero
    and for values that round to zero (-0 -> 0x80).
"""

import numpy as np

BIAS = 7
MAX_FINITE = 448.0
NAN_CODES = (0x7F, 0xFF)


def decode_one(code):
    """Value of one 8-bit code, from the bit fields (float, NaN for 0x7F/0xFF)."""
    code = int(code)
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** (1 - BIAS - 3)          # m * 2**-9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - BIAS)


def decode_table():
    """All 256 code values as float64 (index = code)."""
    return np.array([decode_one(c) for c in range(256)], dtype=np.float64)


_TABLE = decode_table()
# Non-negative finite values, indexed by code 0x00..0x7E.  Their order is the
# code order (exponent field above mantissa field), which the tests pin.
_POS = _TABLE[:0x7F].copy()


def decode(codes):
    """Decode an array of uint8 codes to float64 (NaN for the NaN codes)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(x):
    """Encode an array of floats (float32 or float64) to uint8 E4M3 codes.

    Nearest of the 127 non-negative finite values, ties to the even code,
    saturating at 448, sign bit or-ed in from the input (so -0 -> 0x80).
    The comparison is done in float64, where every code value and every
    midpoint between neighbouring codes is exact.
    """
    x = np.asarray(x)
    xf = x.astype(np.float64)
    sign = np.signbit(xf)
    nan = np.isnan(xf)
    a = np.minimum(np.abs(np.where(nan, 0.0, xf)), MAX_FINITE)

    # hi = first table index with value >= a; lo = hi - 1 (clipped).
    hi = np.searchsorted(_POS, a, side="left")
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code).astype(np.uint8)
    code = code | (sign.astype(np.uint8) << 7)
    return code.astype(np.uint8)


def closed_form_max(exp_bits, man_bits, ieee_reserved_top):
    """Largest finite value of a sign/exponent/mantissa format.

    With ``ieee_reserved_top`` the top exponent field is reserved for
    Inf/NaN (E5M2, FP16 style); without it only the all-ones mantissa at
    the top exponent is NaN (the E4M3 reading above).  Used to pin the
    reading of the pages' format table against its three printed maxima.
    """
    bias = 2 ** (exp_bits - 1) - 1
    top = 2 ** exp_bits - 1
    if ieee_reserved_top:
        e_max = top - 1 - bias
        frac = 2.0 - 2.0 ** (-man_bits)
    else:
        e_max = top - bias
        frac = 2.0 - 2.0 ** (1 - man_bits)
    return frac * 2.0 ** e_max
