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
"""

import numpy as np

from .fp8 import E4M3_MAX, e4m3_encode, e4m3_decode

BLOCK = 128


def _scale_from_amax(amax):
    amax = np.asarray(amax, dtype=np.float32)
    s = amax / np.float32(E4M3_MAX)          # float32 / float32: IEEE RNE division
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quant_1x128(x):
    """x: float32 array [rows, cols] (BF16 values), cols % 128 == 0.
    Returns (codes uint8 [rows, cols], scale float32 [rows, cols/128])."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    assert cols % BLOCK == 0
    t = x.reshape(rows, cols // BLOCK, BLOCK)
    amax = np.max(np.abs(t), axis=2)
    scale = _scale_from_amax(amax)
    y = (t / scale[:, :, None]).astype(np.float32)   # float32 division, per element
    q = e4m3_encode(y).reshape(rows, cols)
    return q, scale


def quant_128x128(w):
    """w: float32 array [N, K] (BF16 values), N and K multiples of 128.
    Returns (codes uint8 [N, K], scale float32 [N/128, K/128])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert n % BLOCK == 0 and k % BLOCK == 0
    t = w.reshape(n // BLOCK, BLOCK, k // BLOCK, BLOCK)
    amax = np.max(np.abs(t), axis=(1, 3))
    scale = _scale_from_amax(amax)
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
