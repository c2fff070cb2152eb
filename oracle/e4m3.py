"""OCP float8 E4M3 ("e4m3fn") codec, written from the format definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The record format in the flydsl_sparse_mla page's module docstring keeps
the 512 latent values as one E4M3 byte each (next to four float32 tile
scales and the 64 bf16 rope values), and the fused_mla_key_concat_kv_cache
page writes them through ``torch.float8_e4m3fn``.  The ``fp8_word`` helper
on the mono/attention/mla page says the writer's quantization saturates.

Format (OCP 8-bit floating point, E4M3 variant): 1 sign bit, 4 exponent
bits (bias 7), 3 mantissa bits; exponent field 0 encodes subnormals
m * 2^-9; the only NaN encodings are S.1111.111 (0x7F / 0xFF); there are
no infinities; the largest finite magnitude is 1.75 * 2^8 = 448.

Reading used for the encoder (the pages give no code for it): clamp to
[-448, 448], then round to nearest, ties to even, keeping the sign of zero.
"""

import numpy as np

E4M3_MAX = 448.0


def decode_table():
    """The value of every byte 0..255 as float64 (NaN for 0x7F / 0xFF)."""
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            table[code] = np.nan
        elif exp_field == 0:
            table[code] = sign * mant * 2.0**-9
        else:
            table[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return table


_TABLE = decode_table()


def e4m3_decode(codes):
    """Byte array -> float64 values (exact)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x):
    """Saturating round-to-nearest-even float -> E4M3 byte.

    ``x`` is any float array (float32 values are converted to float64
    exactly).  Returns uint8 codes.  NaN maps to a NaN code (0x7F or 0xFF).
    """
    x = np.asarray(x, dtype=np.float64)
    negative = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)  # saturate; |x| only from here on

    # Subnormal range |x| < 2^-6: the code is the integer m with value
    # m * 2^-9; rounding |x| * 2^9 to the nearest even integer is exact in
    # float64 (scaling by a power of two) and may give m = 8, which is the
    # smallest normal 0x08 = 2^-6, so the two ranges join without a seam.
    sub_code = np.rint(a * 2.0**9)

    # Normal range: a = 2^e * (1 + f), keep 3 fraction bits with RNE.  A
    # carry out of the fraction (mantissa 8) bumps the exponent, which the
    # integer sum below does by itself.
    frac, exp2 = np.frexp(a)  # a = frac * 2^exp2, frac in [0.5, 1)
    e = exp2.astype(np.int64) - 1  # unbiased exponent of a
    mant = np.rint((2.0 * frac - 1.0) * 8.0)  # 0..8, exact
    nrm_code = ((e + 7) << 3) + mant.astype(np.int64)

    codes = np.where(a < 2.0**-6, sub_code.astype(np.int64), nrm_code)
    codes = np.where(np.isnan(a), 0x7F, codes)
    codes = codes | np.where(negative, 0x80, 0)
    return codes.astype(np.uint8)
