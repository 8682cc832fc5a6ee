"""Blocked FP8 GEMM with per-128-K-block scales (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

The scales lie along the inner dimension K, so every 128-wide K block's partial
sum needs its own dequantisation factor before it joins the total (the book's
chapter 16 "Scales along the GEMM inner dimension"); the partial sums are
promoted to FP32 every 128 K-elements with the group scales applied at
promotion ("DeepSeek-V3" summary page, section 6, ingredient (b)
"Higher-precision accumulation"; chapter 16 "Periodic high-precision
promotion").

The oracle computes the exact value of that blocked sum:
    y[m, n] = sum_kb  sa[m, kb] * sw[n // 128, kb] * P[m, n, kb],
    P[m, n, kb] = sum_{i in block kb} qa[m, i] * qw[n, i].
Every E4M3 value is an integer multiple of 2^-9 of magnitude <= 448, so each
product is a multiple of 2^-18 below 2^18 in magnitude and a 128-term sum needs
fewer than 43 bits: P is exact in float64 in any summation order.  The outer
sum is float64; callers round it to FP32 where the method holds FP32.
"""

import numpy as np

from .fp8 import e4m3_decode

BLOCK = 128


def blocked_gemm(qa, sa, qw, sw):
    """qa uint8 [M, K], sa float32 [M, K/128], qw uint8 [N, K], sw float32 [N/128, K/128].
    Returns float64 [M, N]."""
    qa = np.asarray(qa)
    qw = np.asarray(qw)
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2 and K % BLOCK == 0 and N % BLOCK == 0
    kb_n = K // BLOCK
    a = e4m3_decode(qa)
    w = e4m3_decode(qw)
    sa = np.asarray(sa, np.float64)
    sw_rows = np.repeat(np.asarray(sw, np.float64), BLOCK, axis=0)    # [N, K/128]
    y = np.zeros((M, N))
    for kb in range(kb_n):
        blk = slice(kb * BLOCK, (kb + 1) * BLOCK)
        p = a[:, blk] @ w[:, blk].T                      # exact partial sums
        y += (sa[:, kb:kb + 1] * sw_rows[None, :, kb]) * p
    return y
