"""FP8 E4M3 and BF16 rounding, written from the bit-field definitions (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

E4M3 is the format of every FP8 tensor in V3 ("DeepSeek-V3" summary page,
section 6 "FP8 mixed-precision training", ingredient (c) "E4M3 everywhere"):
one sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0
encodes subnormals m/8 * 2^-6; the all-ones pattern S.1111.111 is NaN and
there is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448
(the table in the FP8 section of "DeepSeek-V3: the recipe, and the interconnect
that shaped it": max finite 448, min normal 1.562e-2, 8 steps per octave).

Readings (the pages leave these open; the book's chapter 16 "Exponent and
mantissa" says the conventions depend on the variant):
  * rounding is round-to-nearest, ties to the even mantissa;
  * magnitudes above 448 saturate to 448 (the scaled quantiser never exceeds
    448 by more than rounding, so this only fixes a convention);
  * subnormals are kept (no flush to zero) and the sign of a zero is kept.
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_MANT_BITS = 3
E4M3_BIAS = 7


def round_to_grid(x, mant_bits, emin):
    """Round float64 values to the nearest binary float with ``mant_bits``
    fraction bits and minimum normal exponent ``emin`` (ties to even).

    No overflow handling: the caller saturates.  A value is written
    |x| = f * 2^p with f in [0.5, 1); its leading bit has weight 2^(p-1), and
    below 2^emin the spacing stays that of the subnormal range.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, p = np.frexp(ax)
    e = np.maximum(p - 1, emin)
    spacing = np.ldexp(1.0, e - mant_bits)
    r = np.rint(ax / spacing) * spacing  # np.rint: half to even; ax/spacing is exact
    return np.copysign(r, x)


CHUNK = 1 << 20


def _chunked(fn, x, out_dtype):
    """Apply an elementwise function over a flattened array in cache-sized
    pieces (numpy is much slower on large multi-dimensional temporaries)."""
    x = np.asarray(x)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, out_dtype)
    for i in range(0, flat.size, CHUNK):
        out[i:i + CHUNK] = fn(flat[i:i + CHUNK])
    return out.reshape(x.shape)


def e4m3_decode(codes):
    """Decode uint8 E4M3 codes to float64 (NaN for S.1111.111): a lookup in the
    256-entry table that the bit-field decoder below produces."""
    return _DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def _e4m3_decode(codes):
    c = codes.astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = np.ldexp(m / 8.0, 1 - E4M3_BIAS)
    nrm = np.ldexp(1.0 + m / 8.0, e - E4M3_BIAS)
    v = np.where(e == 0, sub, nrm)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return sign * v


_DECODE_TABLE = _e4m3_decode(np.arange(256, dtype=np.uint8))


def e4m3_round(x):
    """Round float64/float32 values to E4M3 values (RNE, saturating at 448)."""
    r = round_to_grid(x, E4M3_MANT_BITS, 1 - E4M3_BIAS)
    return np.clip(r, -E4M3_MAX, E4M3_MAX)


def e4m3_encode(x):
    """Encode values as E4M3 codes: RNE to the grid, saturate, then pack the
    sign, exponent and mantissa fields.  -0 and values rounding to zero from
    below keep the sign bit (code 0x80)."""
    return _chunked(_e4m3_encode, x, np.uint8)


def _e4m3_encode(x):
    x = np.asarray(x, dtype=np.float64)
    v = e4m3_round(x)
    av = np.abs(v)
    sign = np.signbit(v).astype(np.int64) << 7
    normal = av >= E4M3_MIN_NORMAL
    _, p = np.frexp(np.where(normal, av, 1.0))
    e_unb = p - 1
    e_field = np.where(normal, e_unb + E4M3_BIAS, 0)
    mant = np.where(normal,
                    (np.ldexp(av, -np.where(normal, e_unb, 0)) - 1.0) * 8.0,
                    av / np.ldexp(1.0, 1 - E4M3_BIAS - E4M3_MANT_BITS))
    m_field = np.rint(mant).astype(np.int64)
    return (sign | (e_field << 3) | m_field).astype(np.uint8)


def f32(x):
    """Round to IEEE float32 (round to nearest even), returned as float32."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_round(x):
    """Round float64 values to bfloat16 values (8 significant bits, same
    exponent range as float32), ties to even; returned as float32."""
    return round_to_grid(x, 7, -126).astype(np.float32)


def bf16_bits_to_f32(bits):
    """Widen uint16 bfloat16 bit patterns to float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f32_to_bf16_bits(x):
    """Bit pattern of float32 values that are already bfloat16 values."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    return (b >> 16).astype(np.uint16)
