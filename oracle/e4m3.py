"""OCP 8-bit floating point E4M3 ("FN" variant), from its bit-level definition.

Format (OCP 8-bit Floating Point Specification, E4M3): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits. Exponent field 0 encodes subnormals
m * 2^-9 (m = 1..7); exponent fields 1..15 encode (1 + m/8) * 2^(e - 7), except
that exponent 15 with mantissa 7 (S.1111.111) is NaN. There are no infinities;
the largest finite magnitude is 1.75 * 2^8 = 448.

Encoding rounds to nearest with ties to the even code (mantissa LSB 0) and
saturates finite values beyond +-448 to +-448 (the saturating conversion used
to quantise attention inputs with a per-tensor scale amax / 448).

The pages only say that FlashAttention-3 adds FP8 support ("11.11 Flash
Attention", section "Flash Attention 3"); the choice of OCP E4M3 with a
per-tensor scale is a reading of that (the pages name no format).
"""

import numpy as np

E4M3_MAX = 448.0
_NAN_CODE = 0x7F


def _decode_one(code):
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
# non-negative finite codes 0x00..0x7E in increasing value order
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = _TABLE[:0x7F]


def e4m3_decode(codes):
    """Map uint8 codes to float64 values (NaN code -> nan)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _TABLE[codes]


def e4m3_encode(x):
    """Round float64 values to E4M3 codes (RNE, saturating at +-448, nan -> 0x7F)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # index of the largest representable value <= a
    lo = np.searchsorted(_POS_VALUES, a, side="right") - 1
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & ((_POS_CODES[lo] & 1) == 1))
    mag = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.int64)
    neg = np.signbit(x) & (mag != 0)
    code = np.where(neg, mag | 0x80, mag)
    code = np.where(np.isnan(x), _NAN_CODE, code)
    return code.astype(np.uint8)
