"""SwiGLU experts, shared expert, combine and the whole MoE layer (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

The layer ("DeepSeek-V3" summary page section 1, DeepSeekMoE paragraph; the
book's chapter 7): N_s = 1 shared expert always runs, and of N_r routed experts
the top K_r get a nonzero gate.  Each expert is a SwiGLU FFN with input/output
width d and two intermediate branches of width f (chapter 7 "What one expert
computes"; the equation is missing from the extracted text, so the reading is
the standard SwiGLU  FFN(x) = W2 (SiLU(W1 x) * (W3 x)), SiLU(z) = z / (1 + e^-z),
no biases).  The summary page's section 6 keeps every principal GEMM of a
linear layer in FP8, so the SwiGLU output is quantised in 1x128 tiles before
the down projection, as the SwiGLU inputs are cached in FP8 (chapter 17
"SwiGLU recomputation").  Expert outputs and the combine stay BF16 (summary
page section 6 "Storage and communication"; chapter 17 "FP8 dispatch, BF16
combine").  The combine adds the gated routed outputs and the shared expert's
output; the residual connection is kept apart from the expert sum and added by
the caller (chapter 7, "Selecting and combining experts").

Rounding points emulated (readings): the GEMM outputs G and U are rounded to
FP32; h = fl32(SiLU(g) * u); each expert output is fl32 then BF16; the combine
sums in float64 and rounds once to BF16.

``rule`` selects the scale rule of every quantisation on the path ("fp32",
the pages' amax/448, or "pow2", the power-of-two rule of ``oracle.quant``); the
GEMMs use whatever scales the operands carry.

Weight layout: w13[e] is [2f, d] with rows [0, f) = W1 (gate branch) and rows
[f, 2f) = W3 (up branch); w2[e] is [d, f]; expert index E is the shared expert.
"""

import numpy as np

from .fp8 import f32, bf16_round
from .quant import quant_1x128, quant_128x128
from .gemm import blocked_gemm
from .route import route as route_tokens
from .permute import permute, gather_rows


def silu(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(g, u):
    """h = fl32(SiLU(g) * u), evaluated in float64 from FP32 g and u."""
    return f32(silu(g) * np.asarray(u, np.float64))


def quantize_expert(w13, w2, rule="fp32"):
    """Offline 128x128 quantisation of one expert's BF16 weights."""
    w13q, w13s = quant_128x128(w13, rule)
    w2q, w2s = quant_128x128(w2, rule)
    return w13q, w13s, w2q, w2s


def expert_ffn(xq, xs, w13q, w13s, w2q, w2s, rule="fp32"):
    """One expert on its FP8 rows.  Returns (y BF16 values as float32 [rows, d],
    dict of intermediates: g, u, h (FP32), hq, hs (its 1x128 quantisation))."""
    f = w13q.shape[0] // 2
    gu = f32(blocked_gemm(xq, xs, w13q, w13s))
    g, u = gu[:, :f], gu[:, f:]
    h = swiglu(g, u)
    hq, hs = quant_1x128(h, rule)
    y = bf16_round(f32(blocked_gemm(hq, hs, w2q, w2s)))
    return y, {"g": g, "u": u, "h": h, "hq": hq, "hs": hs}


def combine(y_routed, w, y_shared, residual=None):
    """out[t] = BF16( sum_j w[t, j] * y_routed[t, j] + y_shared[t] (+ residual[t]) ),
    float64 sum, one rounding.  y_routed [T, k, d], w [T, k], y_shared [T, d],
    residual [T, d] or None (the book's chapter 15 lists the residual path
    among what combine adds; the layer itself passes none)."""
    acc = np.einsum("tk,tkd->td", np.asarray(w, np.float64), np.asarray(y_routed, np.float64))
    acc += np.asarray(y_shared, np.float64)
    if residual is not None:
        acc += np.asarray(residual, np.float64)
    return bf16_round(acc)


def moe_layer(x, wg, bias, experts, n_groups, topk_groups, k, route_scale, rule="fp32"):
    """Whole-batch layer.  ``experts(e)`` returns the quantised weights
    (w13q, w13s, w2q, w2s) of expert e, e = 0..E (E = shared).
    Returns a dict with every intermediate of the path."""
    x = np.asarray(x, np.float32)
    T, d = x.shape
    E = np.asarray(wg).shape[0]
    r = route_tokens(x, wg, bias, n_groups, topk_groups, k, route_scale)
    xq, xs = quant_1x128(x, rule)
    offsets, pos, row_token = permute(r["idx"], E)
    xq_perm = gather_rows(xq, row_token, T)
    xs_perm = gather_rows(xs, row_token, T)
    rows = T * k + T
    f = None
    y = np.zeros((rows, d), np.float32)
    hq = hs = g = u = h = None
    for e in range(E + 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        w13q, w13s, w2q, w2s = experts(e)
        if f is None:
            f = w13q.shape[0] // 2
            hq = np.zeros((rows, f), np.uint8)
            hs = np.zeros((rows, f // 128), np.float32)
            g, u, h = (np.zeros((rows, f), np.float32) for _ in range(3))
        ye, inter = expert_ffn(xq_perm[lo:hi], xs_perm[lo:hi], w13q, w13s, w2q, w2s, rule)
        y[lo:hi] = ye
        hq[lo:hi] = inter["hq"]
        hs[lo:hi] = inter["hs"]
        g[lo:hi], u[lo:hi], h[lo:hi] = inter["g"], inter["u"], inter["h"]
    y_routed = y[np.asarray(pos, np.int64)]                   # [T, k, d]
    out = combine(y_routed, r["w"], y[T * k:T * k + T])
    return {"route": r, "xq": xq, "xs": xs, "offsets": offsets, "pos": pos,
            "row_token": row_token, "xq_perm": xq_perm, "xs_perm": xs_perm,
            "g": g, "u": u, "h": h, "hq": hq, "hs": hs, "y": y, "out": out}


def moe_layer_tokens(x_rows, wg, bias, experts, n_groups, topk_groups, k, route_scale, rule="fp32"):
    """Layer output for a set of tokens evaluated on their own.  Every step after
    routing acts on one token at a time (1x128 tiles lie within a row, experts act
    row-wise, the combine is per token) and routing is per token, so this equals
    the corresponding rows of the whole-batch layer.  Returns (out [n, d],
    route dict, intermediates: y_routed [n, k, d], y_shared [n, d], and the
    expert_ffn intermediates per (token, slot) and per token for the shared
    expert)."""
    x_rows = np.asarray(x_rows, np.float32)
    n, d = x_rows.shape
    E = np.asarray(wg).shape[0]
    r = route_tokens(x_rows, wg, bias, n_groups, topk_groups, k, route_scale)
    xq, xs = quant_1x128(x_rows, rule)
    y_routed = np.zeros((n, k, d), np.float32)
    y_shared = np.zeros((n, d), np.float32)
    need = {}
    inter_routed, inter_shared = {}, {}
    for t in range(n):
        for j in range(k):
            need.setdefault(int(r["idx"][t, j]), []).append((t, j))
    for e in sorted(need):
        w13q, w13s, w2q, w2s = experts(e)
        ts = [t for t, _ in need[e]]
        ye, inter = expert_ffn(xq[ts], xs[ts], w13q, w13s, w2q, w2s, rule)
        for i, ((t, j), row) in enumerate(zip(need[e], ye)):
            y_routed[t, j] = row
            inter_routed[(t, j)] = {key: val[i:i + 1] for key, val in inter.items()}
    w13q, w13s, w2q, w2s = experts(E)
    y_shared[:], inter = expert_ffn(xq, xs, w13q, w13s, w2q, w2s, rule)
    for t in range(n):
        inter_shared[t] = {key: val[t:t + 1] for key, val in inter.items()}
    extra = {"xq": xq, "xs": xs, "y_routed": y_routed, "y_shared": y_shared,
             "inter_routed": inter_routed, "inter_shared": inter_shared}
    return combine(y_routed, r["w"], y_shared), r, extra
