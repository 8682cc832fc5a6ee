"""Fine-grained FP8 quantisation with online scales (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

Activations get one scale per 1x128 tile (one token, 128 channels) and weights
one scale per 128x128 block ("DeepSeek-V3" summary page, section 6, ingredient
(a) "Fine-grained quantization"; the book's chapter 16 "V3's grouping").  The
scale comes from the current tile's max-abs value, not from history (ingredient
(d) "Online scaling"; chapter 16 "Online scales").

Per tile, with x the FP32 value of each BF16 input (exact widening):
  amax  = max |x|
  scale = fl32(amax / 448)       -- the stored scale is the dequantisation
                                    multiplier (chapter 16 "Scaling a group":
                                    the released weights are dequantised by
                                    multiplying with the stored factor)
  q     = E4M3(fl32(x / scale))  -- a correctly rounded FP32 division, then RNE
Reading: an all-zero tile gets scale 1.0 and all-zero codes (the pages are
silent on it).

Power-of-two scale rule (``rule="pow2"``).  The pages' training recipe keeps
power-of-two scaling factors for some tensors ("DeepSeek-V3" summary page,
section 6; the book's chapter 17 on the backward pass), and hardware with
block-scaled matrix instructions takes one 8-bit exponent (E8M0, bias 127) per
block.  Reading: the scale is the smallest power of two not below
fl32(amax / 448), so no scaled value exceeds 448 except by the FP32 rounding
of that quotient (then the cast saturates, as in the FP32 rule); it is at
least 2^-127, the smallest E8M0 value; an all-zero tile gets 1.  The codes are
E4M3(fl32(x / scale)) as before (the division by a power of two is exact
unless the quotient is subnormal).
"""

import numpy as np

from .fp8 import E4M3_MAX, e4m3_encode, e4m3_decode

BLOCK = 128


def _scale_from_amax(amax):
    amax = np.asarray(amax, dtype=np.float32)
    s = amax / np.float32(E4M3_MAX)          # float32 / float32: IEEE RNE division
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


E8M0_MIN = np.float32(2.0 ** -127)


def _pow2_scale_from_amax(amax):
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    m, e = np.frexp(s.astype(np.float64))             # s = m * 2^e, 0.5 <= m < 1
    p = np.where(m == 0.5, s.astype(np.float64), np.ldexp(1.0, e))
    p = np.maximum(p, np.float64(E8M0_MIN))
    return np.where(amax == 0, 1.0, p).astype(np.float32)


def scale_from_amax(amax, rule="fp32"):
    """The tile scale of either rule (see the module docstring)."""
    if rule == "fp32":
        return _scale_from_amax(amax)
    if rule == "pow2":
        return _pow2_scale_from_amax(amax)
    raise ValueError(rule)


def quant_1x128(x, rule="fp32"):
    """x: float32 array [rows, cols] (BF16 values), cols % 128 == 0.
    Returns (codes uint8 [rows, cols], scale float32 [rows, cols/128])."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    assert cols % BLOCK == 0
    t = x.reshape(rows, cols // BLOCK, BLOCK)
    amax = np.max(np.abs(t), axis=2)
    scale = scale_from_amax(amax, rule)
    y = (t / scale[:, :, None]).astype(np.float32)   # float32 division, per element
    q = e4m3_encode(y).reshape(rows, cols)
    return q, scale


def quant_128x128(w, rule="fp32"):
    """w: float32 array [N, K] (BF16 values), N and K multiples of 128.
    Returns (codes uint8 [N, K], scale float32 [N/128, K/128])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert n % BLOCK == 0 and k % BLOCK == 0
    t = w.reshape(n // BLOCK, BLOCK, k // BLOCK, BLOCK)
    amax = np.max(np.abs(t), axis=(1, 3))
    scale = scale_from_amax(amax, rule)
    y = (t / scale[:, None, :, None]).astype(np.float32)
    q = e4m3_encode(y).reshape(n, k)
    return q, scale


def dequant_1x128(q, scale):
    """Float64 values of 1x128-tiled codes: code value times its tile scale."""
    q = np.asarray(q)
    rows, cols = q.shape
    v = e4m3_decode(q).reshape(rows, cols // BLOCK, BLOCK)
    return (v * np.asarray(scale, np.float64)[:, :, None]).reshape(rows, cols)


def dequant_128x128(q, scale):
    """Float64 values of 128x128-blocked codes."""
    q = np.asarray(q)
    n, k = q.shape
    v = e4m3_decode(q).reshape(n // BLOCK, BLOCK, k // BLOCK, BLOCK)
    return (v * np.asarray(scale, np.float64)[:, None, :, None]).reshape(n, k)
