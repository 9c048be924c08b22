"""OCP 8-bit floating point E4M3FN codec (test infrastructure only).

The pages name FP8 only (the FlashAttention page, section on FlashAttention-3:
low-precision GEMM with block quantisation).  The reading taken here is the OCP
E4M3FN format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, NaN only at S.1111.111, largest finite magnitude 448.  Encoding is
round-to-nearest-even onto that grid; callers clamp to [-448, 448] first.

Everything here is derived from the bit layout, not from any library.
"""
import numpy as np

FP8_MAX = 448.0
NAN_CODE = 0x7F


def decode_table() -> np.ndarray:
    """Value of each of the 256 codes as float64 (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)     # subnormal
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_TABLE = decode_table()
# non-negative finite codes 0x00..0x7E, values strictly increasing with the code
_POS_VALS = _TABLE[:0x7F]


def encode_rne(y) -> np.ndarray:
    """Round each value (already within [-448, 448], not NaN) to the nearest
    E4M3 code; ties go to the code with an even mantissa (last bit 0).
    The sign bit is the sign of the input, so -0.0 and negative values that
    round to zero give 0x80."""
    y = np.asarray(y, dtype=np.float64)
    assert not np.isnan(y).any(), "encode_rne takes no NaN"
    a = np.abs(y)
    assert (a <= FP8_MAX).all(), "clamp to +-448 before encoding"
    hi = np.searchsorted(_POS_VALS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    exact = d_hi == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(exact | pick_hi, hi, lo).astype(np.uint8)
    code = code | np.where(np.signbit(y), 0x80, 0x00).astype(np.uint8)
    return code


def decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]
