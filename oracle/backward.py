"""Backward pass of the MoE layer's experts and combine (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

What the pages fix ("DeepSeek-V3" summary page, section 6 "FP8 mixed-precision
training"; the book's chapter 17 "One linear layer creates three GEMMs",
"SwiGLU recomputation", "Attention-related saved activations", "Backward
grouping and gradient sensitivity"; chapter 16 "Why transposition is not
trivial"):
  * every linear layer runs three FP8 GEMMs: Fprop, Dgrad (activation
    gradient) and Wgrad (weight gradient), with FP32 accumulation and BF16 or
    FP32 outputs;
  * the MoE's SwiGLU inputs are cached in FP8 by the forward, and the SwiGLU
    output is recomputed from them in the backward;
  * activation gradients keep tile-wise (1x128) grouping; where a backward
    GEMM needs the other orientation, tiles are regrouped from 1x128 to 128x1
    by dequantising and requantising, with power-of-two scales.

Readings where the pages leave a step open:
  1. Every quantisation in the backward uses the power-of-two rule of
     ``oracle.quant`` (so all backward GEMM operands have E8M0-exact scales).
  2. Dgrad operands: dY and [dG, dU] in 1x128 tiles along their columns (the
     GEMM's inner dimension); the weights are the forward's 128x128 blocks,
     transposed (a block scale serves both orientations).
  3. Wgrad operands are 128x1 tiles along the rows (tokens) of one expert: dY
     and H for W2, [dG, dU] and X for W13.  An expert's rows are padded with
     zero rows to a multiple of 128 (zeros change no amax and no sum).  X is
     the forward's FP8 cache (1x128) dequantised in FP32 and requantised.
  4. Rounding points: dY = BF16(fl32(w * dOut)) for routed rows, dOut for the
     shared expert's rows; the gate gradient dw = fl32(sum_c dOut * Y) in
     float64; dH and the expert input gradient are FP32 then BF16 (like Y);
     the token gradient dX = BF16(float64 sum of the token's rows); SwiGLU
     backward in float64 from the FP8 cache, rounded to FP32; weight gradients
     fl32 of the float64 blocked sum.
  5. SwiGLU derivatives: with s = sigmoid(g), h = g*s*u,
     dG = dH * u * s * (1 + g*(1 - s)), dU = dH * g * s.

``quantize=False`` replaces every backward quantisation by the identity
(float64 values flow through), which the pins compare with automatic
differentiation.
"""

import numpy as np

from .fp8 import f32, bf16_round, e4m3_decode
from .quant import quant_1x128, dequant_1x128, BLOCK

RULE = "pow2"


def quant_128x1(x, rule=RULE):
    """128x1 tiles along the rows of x [R, C] (rows padded with zeros to a
    multiple of 128).  Returns (codes uint8 [Rp, C], scales float32
    [Rp/128, C]) with Rp = ceil(R/128)*128: the 1x128 quantisation of x^T,
    transposed back."""
    x = np.asarray(x, np.float32)
    R, C = x.shape
    Rp = -(-R // BLOCK) * BLOCK
    xp = np.zeros((Rp, C), np.float32)
    xp[:R] = x
    q, s = quant_1x128(np.ascontiguousarray(xp.T), rule)
    return np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)


def dequant_128x1(q, s):
    return dequant_1x128(np.ascontiguousarray(np.asarray(q).T), np.ascontiguousarray(np.asarray(s).T)).T


def gemm_rows_scaled(qa, sa, qb, sb):
    """sum over 128-wide K blocks of sa[m, kb] * sb[n, kb] * (exact block dot
    product): both operands with one scale per row and K block.
    qa [M, K], sa [M, K/128], qb [N, K], sb [N, K/128] -> float64 [M, N]."""
    a = e4m3_decode(np.asarray(qa))
    b = e4m3_decode(np.asarray(qb))
    sa = np.asarray(sa, np.float64)
    sb = np.asarray(sb, np.float64)
    M, K = a.shape
    y = np.zeros((M, b.shape[0]))
    for kb in range(K // BLOCK):
        blk = slice(kb * BLOCK, (kb + 1) * BLOCK)
        y += (sa[:, kb:kb + 1] * sb[None, :, kb]) * (a[:, blk] @ b[:, blk].T)
    return y


def _q1x128(x, quantize):
    """(values the GEMM sees, codes, scales) of a 1x128 quantisation."""
    if not quantize:
        return np.asarray(x, np.float64), None, None
    q, s = quant_1x128(np.asarray(x, np.float32), RULE)
    return dequant_1x128(q, s), q, s


def _q128x1(x, quantize):
    if not quantize:
        return np.asarray(x, np.float64), None, None
    q, s = quant_128x1(np.asarray(x, np.float32), RULE)
    return dequant_128x1(q, s)[:x.shape[0]], q, s


def _round(x, quantize, kind):
    """Storage rounding of an intermediate (identity when not quantising)."""
    if not quantize:
        return np.asarray(x, np.float64)
    return bf16_round(f32(x)).astype(np.float64) if kind == "bf16" else f32(x).astype(np.float64)


def swiglu_backward(g, u, dh):
    """(h, dG, dU) in float64 from g, u, dh."""
    g = np.asarray(g, np.float64); u = np.asarray(u, np.float64); dh = np.asarray(dh, np.float64)
    s = 1.0 / (1.0 + np.exp(-g))
    return g * s * u, dh * u * s * (1.0 + g * (1.0 - s)), dh * g * s


def combine_backward(dout, y, w, pos, T, k, quantize=True):
    """Gradients of out[t] = sum_j w[t,j] * y[pos[t,j]] + y[T*k + t].
    Returns (dY rows [T*k + T, d], dw [T, k])."""
    dout = np.asarray(dout, np.float64)
    y = np.asarray(y, np.float64)
    pos = np.asarray(pos, np.int64)
    w = np.asarray(w, np.float64)
    d = dout.shape[1]
    dy = np.zeros((T * k + T, d))
    dy[pos.reshape(-1)] = (w[:, :, None] * dout[:, None, :]).reshape(T * k, d)
    dy[T * k:] = dout
    dw = np.einsum("td,tkd->tk", dout, y[pos])
    if quantize:
        dy[:T * k] = bf16_round(f32(dy[:T * k]))
        dw = f32(dw)
    return dy, dw


def expert_backward(x, gu_cache, dy, w13, w2, quantize=True):
    """Backward of one SwiGLU expert over its rows.

    x         the rows' FP8 input as (codes, scales) of the forward's 1x128
              quantisation, or float values when ``quantize`` is False
    gu_cache  the forward's FP8 cache of [G, U] as (codes, scales), or float
              [rows, 2f] values
    dy        gradient of the expert output [rows, d]
    w13, w2   (codes, 128x128 scales) of W13 [2f, d] and W2 [d, f], or floats
    Returns dict: dx [rows, d] (gradient of the expert input), dw13 [2f, d],
    dw2 [d, f], and the intermediates dh, h, dg, du."""
    if quantize:
        xv = f32(dequant_1x128(*x)).astype(np.float64)
        gu = f32(dequant_1x128(*gu_cache)).astype(np.float64)
        from .quant import dequant_128x128
        W13 = dequant_128x128(*w13)
        W2 = dequant_128x128(*w2)
    else:
        xv, gu = np.asarray(x, np.float64), np.asarray(gu_cache, np.float64)
        W13, W2 = np.asarray(w13, np.float64), np.asarray(w2, np.float64)
    f = W2.shape[1]
    dy = np.asarray(dy, np.float64)
    # Dgrad of the second GEMM: dH = dY W2
    dyq, _, _ = _q1x128(dy, quantize)
    dh = _round(dyq @ W2, quantize, "bf16")
    # SwiGLU recomputed from the cache
    g, u = gu[:, :f], gu[:, f:]
    h, dg, du = swiglu_backward(g, u, dh)
    h, dg, du = (_round(v, quantize, "f32") for v in (h, dg, du))
    dgu = np.concatenate([dg, du], axis=1)
    # Dgrad of the first GEMM: dX = [dG, dU] W13
    dguq, _, _ = _q1x128(dgu, quantize)
    dx = _round(dguq @ W13, quantize, "bf16")
    # Wgrad: dW2 = dY^T H, dW13 = [dG, dU]^T X, operands in 128x1 tiles
    dyt, _, _ = _q128x1(dy, quantize)
    ht, _, _ = _q128x1(h, quantize)
    dgut, _, _ = _q128x1(dgu, quantize)
    xt, _, _ = _q128x1(xv, quantize)
    dw2 = dyt.T @ ht
    dw13 = dgut.T @ xt
    if quantize:
        dw2, dw13 = f32(dw2), f32(dw13)
    return {"dx": dx, "dw13": dw13, "dw2": dw2, "dh": dh, "h": h, "dg": dg, "du": du}


def token_grad(dx_rows, pos, T, k, quantize=True):
    """dX[t] = sum_j dx_rows[pos[t, j]] + dx_rows[T*k + t] (float64 sum)."""
    dx_rows = np.asarray(dx_rows, np.float64)
    pos = np.asarray(pos, np.int64)
    out = dx_rows[pos].sum(axis=1) + dx_rows[T * k:T * k + T]
    return bf16_round(out) if quantize else out
