"""Forward pass of one DeepSeek-V3 MoE layer on an MI355X (gfx950).

The compute lives in libmoe.so (hand-written HIP kernels behind a C ABI, see
``include/moe.h``).  This module is the thin Python binding: each function
has the name of a C entry point, takes torch tensors that already live on the
GPU, and passes their pointers plus the current HIP stream.  PyTorch provides
device memory and streams only.  ``MoELayer`` strings the six calls together
with preallocated buffers.
"""

import ctypes

import torch

from . import _lib
from ._lib import MoEError, RouteParams  # noqa: F401

__all__ = ["moe_route", "moe_route_workspace_bytes", "fp8_quant_1x128", "fp8_quant_128x128", "moe_permute_workspace_bytes",
           "moe_permute", "moe_permute_noalloc", "grouped_gemm_fp8_swiglu", "grouped_gemm_fp8_up", "grouped_gemm_fp8_down",
           "moe_combine", "moe_bias_update", "fp8_quant_1x128_pow2", "fp8_quant_128x128_pow2",
           "grouped_gemm_fp8_up_e8m0", "grouped_gemm_fp8_down_e8m0", "grouped_gemm_fp8_up_train",
           "moe_transpose_fp8_blocks", "moe_combine_backward", "moe_wgrad_columns", "moe_regroup_128x1",
           "moe_swiglu_backward", "grouped_gemm_fp8_wgrad", "MoEWeights", "MoELayer",
           "MoEError", "RouteParams"]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, dtype, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def moe_route_workspace_bytes(T, E):
    return int(_lib.load().moe_route_workspace_bytes(T, E))


def moe_route(x, wg, bias, n_groups, topk_groups, topk, route_scale, idx, w, stream=None, workspace=None):
    """Router: idx [T, k] int32 (ascending expert ids), w [T, k] float32.
    With ``workspace`` (a uint8 device tensor of moe_route_workspace_bytes(T, E)
    bytes) it runs moe_route_ws: the same results, the logits spread over more
    workgroups for small batches."""
    _dev(x, torch.bfloat16, "x"); _dev(wg, torch.bfloat16, "wg"); _dev(bias, torch.float32, "bias")
    _dev(idx, torch.int32, "idx"); _dev(w, torch.float32, "w")
    T, d = x.shape
    p = RouteParams(wg.shape[0], n_groups, topk_groups, topk, route_scale)
    lib = _lib.load()
    if workspace is None:
        _lib.check("moe_route", lib.moe_route(_ptr(x), _ptr(wg), _ptr(bias), T, d, p, _ptr(idx), _ptr(w),
                                              _stream(stream)))
    else:
        _dev(workspace, torch.uint8, "workspace")
        _lib.check("moe_route_ws", lib.moe_route_ws(_ptr(x), _ptr(wg), _ptr(bias), T, d, p, _ptr(idx),
                                                    _ptr(w), _ptr(workspace), workspace.numel(),
                                                    _stream(stream)))


def _quant_1x128(name, x, q, scale, stream):
    _dev(x, torch.bfloat16, "x"); _dev(q, torch.uint8, "q"); _dev(scale, torch.float32, "scale")
    rows, cols = x.shape
    fn = getattr(_lib.load(), name)
    _lib.check(name, fn(_ptr(x), rows, cols, _ptr(q), _ptr(scale), _stream(stream)))


def _quant_128x128(name, w, q, scale, stream):
    _dev(w, torch.bfloat16, "w"); _dev(q, torch.uint8, "q"); _dev(scale, torch.float32, "scale")
    K = w.shape[-1]
    N = w.numel() // K
    fn = getattr(_lib.load(), name)
    _lib.check(name, fn(_ptr(w), N, K, _ptr(q), _ptr(scale), _stream(stream)))


def fp8_quant_1x128(x, q, scale, stream=None):
    """x [rows, cols] BF16 -> q [rows, cols] uint8 E4M3, scale [rows, cols/128] float32."""
    _quant_1x128("fp8_quant_1x128", x, q, scale, stream)


def fp8_quant_1x128_pow2(x, q, scale, stream=None):
    """fp8_quant_1x128 with power-of-two scales."""
    _quant_1x128("fp8_quant_1x128_pow2", x, q, scale, stream)


def fp8_quant_128x128(w, q, scale, stream=None):
    """w [..., N, K] BF16 (leading dims folded into N) -> q uint8, scale [..., N/128, K/128]."""
    _quant_128x128("fp8_quant_128x128", w, q, scale, stream)


def fp8_quant_128x128_pow2(w, q, scale, stream=None):
    """fp8_quant_128x128 with power-of-two scales."""
    _quant_128x128("fp8_quant_128x128_pow2", w, q, scale, stream)


def moe_permute_workspace_bytes(T, k, E):
    return int(_lib.load().moe_permute_workspace_bytes(T, k, E))


def moe_permute(idx, n_experts, offsets, pos, row_token, workspace, xq=None, xs=None,
                xq_perm=None, xs_perm=None, stream=None):
    """Group assignments by expert: offsets [E+2], pos [T, k], row_token [T*k + T];
    optionally copies the FP8 rows into xq_perm / xs_perm."""
    for t, dt, n in ((idx, torch.int32, "idx"), (offsets, torch.int32, "offsets"),
                     (pos, torch.int32, "pos"), (row_token, torch.int32, "row_token"),
                     (workspace, torch.uint8, "workspace"), (xq, torch.uint8, "xq"),
                     (xs, torch.float32, "xs"), (xq_perm, torch.uint8, "xq_perm"),
                     (xs_perm, torch.float32, "xs_perm")):
        _dev(t, dt, n)
    T, k = idx.shape
    d = xq.shape[1] if xq is not None else 0
    lib = _lib.load()
    _lib.check("moe_permute", lib.moe_permute(
        _ptr(idx), T, k, n_experts, _ptr(xq), _ptr(xs), d, _ptr(offsets), _ptr(pos),
        _ptr(row_token), _ptr(xq_perm), _ptr(xs_perm), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream(stream)))


def moe_permute_noalloc(idx, n_experts, offsets, pos, row_token, xq=None, xs=None, xq_perm=None,
                        xs_perm=None, stream=None):
    """moe_permute without a workspace: the histograms live in the library's
    static device array (for callers that cannot allocate; calls that overlap
    on one GPU race)."""
    for t, dt, n in ((idx, torch.int32, "idx"), (offsets, torch.int32, "offsets"),
                     (pos, torch.int32, "pos"), (row_token, torch.int32, "row_token"),
                     (xq, torch.uint8, "xq"), (xs, torch.float32, "xs"),
                     (xq_perm, torch.uint8, "xq_perm"), (xs_perm, torch.float32, "xs_perm")):
        _dev(t, dt, n)
    T, k = idx.shape
    d = xq.shape[1] if xq is not None else 0
    lib = _lib.load()
    _lib.check("moe_permute_noalloc", lib.moe_permute_noalloc(
        _ptr(idx), T, k, n_experts, _ptr(xq), _ptr(xs), d, _ptr(offsets), _ptr(pos),
        _ptr(row_token), _ptr(xq_perm), _ptr(xs_perm), _stream(stream)))


def grouped_gemm_fp8_swiglu(aq, as_, row_src, offsets, w13, w13_s, w2, w2_s, h, hs, y, stream=None):
    """Both expert GEMMs: h/hs [rows, f] E4M3 + scales, y [rows, d] BF16."""
    for t, dt, n in ((aq, torch.uint8, "aq"), (as_, torch.float32, "as"),
                     (row_src, torch.int32, "row_src"), (offsets, torch.int32, "offsets"),
                     (w13, torch.uint8, "w13"), (w13_s, torch.float32, "w13_s"),
                     (w2, torch.uint8, "w2"), (w2_s, torch.float32, "w2_s"),
                     (h, torch.uint8, "h"), (hs, torch.float32, "hs"), (y, torch.bfloat16, "y")):
        _dev(t, dt, n)
    n_groups, two_f, d = w13.shape
    rows = h.shape[0]
    lib = _lib.load()
    _lib.check("grouped_gemm_fp8_swiglu", lib.grouped_gemm_fp8_swiglu(
        _ptr(aq), _ptr(as_), aq.shape[0], _ptr(row_src), _ptr(offsets), n_groups, rows, d,
        two_f // 2, _ptr(w13), _ptr(w13_s), _ptr(w2), _ptr(w2_s), _ptr(h), _ptr(hs), _ptr(y),
        _stream(stream)))


def _gemm_up(name, aq, as_, row_src, offsets, w13, w13_s, h, hs, stream):
    for t, dt, n in ((aq, torch.uint8, "aq"), (as_, torch.float32, "as"),
                     (row_src, torch.int32, "row_src"), (offsets, torch.int32, "offsets"),
                     (w13, torch.uint8, "w13"), (w13_s, torch.float32, "w13_s"),
                     (h, torch.uint8, "h"), (hs, torch.float32, "hs")):
        _dev(t, dt, n)
    n_groups, two_f, d = w13.shape
    fn = getattr(_lib.load(), name)
    _lib.check(name, fn(
        _ptr(aq), _ptr(as_), aq.shape[0], _ptr(row_src), _ptr(offsets), n_groups, h.shape[0], d,
        two_f // 2, _ptr(w13), _ptr(w13_s), _ptr(h), _ptr(hs), _stream(stream)))


def grouped_gemm_fp8_up(aq, as_, row_src, offsets, w13, w13_s, h, hs, stream=None):
    """First expert GEMM with the SwiGLU epilogue: h/hs [rows, f]."""
    _gemm_up("grouped_gemm_fp8_up", aq, as_, row_src, offsets, w13, w13_s, h, hs, stream)


def grouped_gemm_fp8_up_e8m0(aq, as_, row_src, offsets, w13, w13_s, h, hs, stream=None):
    """grouped_gemm_fp8_up for power-of-two scales (hardware block-scaled MFMA)."""
    _gemm_up("grouped_gemm_fp8_up_e8m0", aq, as_, row_src, offsets, w13, w13_s, h, hs, stream)


def _gemm_down(name, h, hs, offsets, w2, w2_s, y, stream):
    for t, dt, n in ((h, torch.uint8, "h"), (hs, torch.float32, "hs"),
                     (offsets, torch.int32, "offsets"), (w2, torch.uint8, "w2"),
                     (w2_s, torch.float32, "w2_s"), (y, torch.bfloat16, "y")):
        _dev(t, dt, n)
    n_groups, d, f = w2.shape
    fn = getattr(_lib.load(), name)
    _lib.check(name, fn(
        _ptr(h), _ptr(hs), _ptr(offsets), n_groups, h.shape[0], d, f, _ptr(w2), _ptr(w2_s),
        _ptr(y), _stream(stream)))


def grouped_gemm_fp8_down(h, hs, offsets, w2, w2_s, y, stream=None):
    """Second expert GEMM: y [rows, d] BF16."""
    _gemm_down("grouped_gemm_fp8_down", h, hs, offsets, w2, w2_s, y, stream)


def grouped_gemm_fp8_down_e8m0(h, hs, offsets, w2, w2_s, y, stream=None):
    """grouped_gemm_fp8_down for power-of-two scales (hardware block-scaled MFMA)."""
    _gemm_down("grouped_gemm_fp8_down_e8m0", h, hs, offsets, w2, w2_s, y, stream)


def moe_combine(y, pos, w, shared_row0, out, stream=None, residual=None):
    """out [T, d] = BF16(sum_j w[t, j] * y[pos[t, j]] + y[shared_row0 + t]
    (+ residual[t] when given, a [T, d] BF16 tensor))."""
    _dev(y, torch.bfloat16, "y"); _dev(pos, torch.int32, "pos"); _dev(w, torch.float32, "w")
    _dev(out, torch.bfloat16, "out"); _dev(residual, torch.bfloat16, "residual")
    T, k = pos.shape
    if residual is not None and tuple(residual.shape) != tuple(out.shape):
        raise ValueError("residual must have the shape of out")
    lib = _lib.load()
    _lib.check("moe_combine", lib.moe_combine(_ptr(y), _ptr(pos), _ptr(w), T, k, y.shape[1],
                                              shared_row0, _ptr(residual), _ptr(out), _stream(stream)))


def moe_bias_update(offsets, bias, gamma, stream=None):
    """Bias controller step: bias[e] -= gamma * sign(load[e] - mean load) for the
    bias.numel() routed experts, loads from moe_permute's offsets."""
    _dev(offsets, torch.int32, "offsets"); _dev(bias, torch.float32, "bias")
    E = bias.numel()
    if offsets.numel() < E + 1:
        raise ValueError(f"offsets has {offsets.numel()} entries, {E + 1} needed")
    lib = _lib.load()
    _lib.check("moe_bias_update", lib.moe_bias_update(_ptr(offsets), E, float(gamma), _ptr(bias),
                                                      _stream(stream)))


def grouped_gemm_fp8_up_train(aq, as_, row_src, offsets, w13, w13_s, h, hs, gu, gus, stream=None):
    """grouped_gemm_fp8_up that also writes the FP8 cache of [G, U] (gu [rows, 2f],
    gus [rows, 2f/128]) for the backward's SwiGLU recomputation."""
    for t, dt, n in ((aq, torch.uint8, "aq"), (as_, torch.float32, "as"),
                     (row_src, torch.int32, "row_src"), (offsets, torch.int32, "offsets"),
                     (w13, torch.uint8, "w13"), (w13_s, torch.float32, "w13_s"),
                     (h, torch.uint8, "h"), (hs, torch.float32, "hs"), (gu, torch.uint8, "gu"),
                     (gus, torch.float32, "gus")):
        _dev(t, dt, n)
    n_groups, two_f, d = w13.shape
    lib = _lib.load()
    _lib.check("grouped_gemm_fp8_up_train", lib.grouped_gemm_fp8_up_train(
        _ptr(aq), _ptr(as_), aq.shape[0], _ptr(row_src), _ptr(offsets), n_groups, h.shape[0], d,
        two_f // 2, _ptr(w13), _ptr(w13_s), _ptr(h), _ptr(hs), _ptr(gu), _ptr(gus), _stream(stream)))


def moe_transpose_fp8_blocks(w, ws, wt, wts, stream=None):
    """[G, N, K] E4M3 + [G, N/128, K/128] scales -> [G, K, N] + [G, K/128, N/128]."""
    for t, dt, n in ((w, torch.uint8, "w"), (ws, torch.float32, "ws"), (wt, torch.uint8, "wt"),
                     (wts, torch.float32, "wts")):
        _dev(t, dt, n)
    G, N, K = w.shape
    lib = _lib.load()
    _lib.check("moe_transpose_fp8_blocks", lib.moe_transpose_fp8_blocks(
        _ptr(w), _ptr(ws), G, N, K, _ptr(wt), _ptr(wts), _stream(stream)))


def moe_combine_backward(dout, y, pos, w, shared_row0, dy, dw, stream=None, dyq=None, dys=None):
    """dy [rows, d] BF16 and dw [T, k] FP32 from dout [T, d] and the forward's y;
    with dyq [rows, d] uint8 and dys [rows, d/128] FP32 also the 1x128
    power-of-two FP8 copy of the dY rows (moe_combine_backward_q)."""
    for t, dt, n in ((dout, torch.bfloat16, "dout"), (y, torch.bfloat16, "y"), (pos, torch.int32, "pos"),
                     (w, torch.float32, "w"), (dy, torch.bfloat16, "dy"), (dw, torch.float32, "dw")):
        _dev(t, dt, n)
    T, k = pos.shape
    lib = _lib.load()
    if dyq is None and dys is None:
        _lib.check("moe_combine_backward", lib.moe_combine_backward(
            _ptr(dout), _ptr(y), _ptr(pos), _ptr(w), T, k, dout.shape[1], shared_row0, _ptr(dy),
            _ptr(dw), _stream(stream)))
        return
    _dev(dyq, torch.uint8, "dyq")
    _dev(dys, torch.float32, "dys")
    _lib.check("moe_combine_backward_q", lib.moe_combine_backward_q(
        _ptr(dout), _ptr(y), _ptr(pos), _ptr(w), T, k, dout.shape[1], shared_row0, _ptr(dy),
        _ptr(dw), _ptr(dyq), _ptr(dys), _stream(stream)))


def moe_wgrad_columns(total_rows, n_groups):
    return int(_lib.load().moe_wgrad_columns(total_rows, n_groups))


def moe_regroup_128x1(offsets, n_groups, total_rows, out, out_s, xq=None, xs=None, x_bf16=None,
                      row_src=None, stream=None):
    """K-major 128x1 power-of-two copy out [C, Kp], out_s [Kp/128, C] of either
    a 1x128 FP8 tensor (xq, xs, gathered through row_src) or a BF16 one."""
    for t, dt, n in ((offsets, torch.int32, "offsets"), (out, torch.uint8, "out"),
                     (out_s, torch.float32, "out_s"), (xq, torch.uint8, "xq"), (xs, torch.float32, "xs"),
                     (x_bf16, torch.bfloat16, "x_bf16"), (row_src, torch.int32, "row_src")):
        _dev(t, dt, n)
    C = out.shape[0]
    lib = _lib.load()
    _lib.check("moe_regroup_128x1", lib.moe_regroup_128x1(
        _ptr(xq), _ptr(xs), _ptr(x_bf16), _ptr(row_src), _ptr(offsets), n_groups, total_rows, C,
        _ptr(out), _ptr(out_s), _stream(stream)))


def moe_swiglu_backward(gu, gus, dh, offsets, n_groups, dgu, dgus, dgu_t, dgu_ts, h_t, h_ts, stream=None):
    """SwiGLU backward from the FP8 [G, U] cache: the Dgrad operand (dgu, dgus)
    and the K-major Wgrad operands of [dG, dU] and h."""
    for t, dt, n in ((gu, torch.uint8, "gu"), (gus, torch.float32, "gus"), (dh, torch.bfloat16, "dh"),
                     (offsets, torch.int32, "offsets"), (dgu, torch.uint8, "dgu"),
                     (dgus, torch.float32, "dgus"), (dgu_t, torch.uint8, "dgu_t"),
                     (dgu_ts, torch.float32, "dgu_ts"), (h_t, torch.uint8, "h_t"), (h_ts, torch.float32, "h_ts")):
        _dev(t, dt, n)
    rows, f = dh.shape
    lib = _lib.load()
    _lib.check("moe_swiglu_backward", lib.moe_swiglu_backward(
        _ptr(gu), _ptr(gus), _ptr(dh), _ptr(offsets), n_groups, rows, f, _ptr(dgu), _ptr(dgus),
        _ptr(dgu_t), _ptr(dgu_ts), _ptr(h_t), _ptr(h_ts), _stream(stream)))


def grouped_gemm_fp8_wgrad(a_t, a_ts, b_t, b_ts, offsets, n_groups, total_rows, dw, stream=None):
    """dw [n_groups, M, N] FP32 from the K-major operands a_t [M, Kp], b_t [N, Kp]."""
    for t, dt, n in ((a_t, torch.uint8, "a_t"), (a_ts, torch.float32, "a_ts"), (b_t, torch.uint8, "b_t"),
                     (b_ts, torch.float32, "b_ts"), (offsets, torch.int32, "offsets"),
                     (dw, torch.float32, "dw")):
        _dev(t, dt, n)
    lib = _lib.load()
    _lib.check("grouped_gemm_fp8_wgrad", lib.grouped_gemm_fp8_wgrad(
        _ptr(a_t), _ptr(a_ts), _ptr(b_t), _ptr(b_ts), _ptr(offsets), n_groups, total_rows,
        a_t.shape[0], b_t.shape[0], _ptr(dw), _stream(stream)))


class MoEWeights:
    """FP8 expert weights of one layer: w13 [E+1, 2f, d], w2 [E+1, d, f] E4M3
    with 128x128 block scales; index E is the shared expert."""

    def __init__(self, w13q, w13s, w2q, w2s):
        self.w13q, self.w13s, self.w2q, self.w2s = w13q, w13s, w2q, w2s
        self.n_groups, two_f, self.d = w13q.shape
        self.f = two_f // 2

    @classmethod
    def empty(cls, n_groups, d, f, device="cuda"):
        return cls(torch.empty(n_groups, 2 * f, d, dtype=torch.uint8, device=device),
                   torch.empty(n_groups, 2 * f // 128, d // 128, dtype=torch.float32, device=device),
                   torch.empty(n_groups, d, f, dtype=torch.uint8, device=device),
                   torch.empty(n_groups, d // 128, f // 128, dtype=torch.float32, device=device))

    def quantize_expert(self, e, w13_bf16, w2_bf16, stream=None, pow2=False):
        """Offline 128x128 quantisation of expert e's BF16 weights into place
        (power-of-two scales when ``pow2``)."""
        q = fp8_quant_128x128_pow2 if pow2 else fp8_quant_128x128
        q(w13_bf16, self.w13q[e], self.w13s[e], stream)
        q(w2_bf16, self.w2q[e], self.w2s[e], stream)

    def transposed(self, stream=None):
        """The weights as Dgrad multiplies them: W13^T [G, d, 2f] and W2^T
        [G, f, d] with transposed block scales (moe_transpose_fp8_blocks)."""
        G, d, f = self.n_groups, self.d, self.f
        dev = dict(device=self.w13q.device)
        t = MoEWeights.__new__(MoEWeights)
        t.w13q = torch.empty(G, d, 2 * f, dtype=torch.uint8, **dev)
        t.w13s = torch.empty(G, d // 128, 2 * f // 128, dtype=torch.float32, **dev)
        t.w2q = torch.empty(G, f, d, dtype=torch.uint8, **dev)
        t.w2s = torch.empty(G, f // 128, d // 128, dtype=torch.float32, **dev)
        moe_transpose_fp8_blocks(self.w13q, self.w13s, t.w13q, t.w13s, stream)
        moe_transpose_fp8_blocks(self.w2q, self.w2s, t.w2q, t.w2s, stream)
        t.n_groups, t.d, t.f = G, d, f
        return t


# From this many tokens the layer quantises X on a side stream beside the
# router (measured: 0.05 ms less per step at 16384 tokens; at 64 tokens the
# fork and join cost more than the overlap gains).
OVERLAP_QUANT_T = 2048


class MoELayer:
    """Buffers and call sequence of the layer for up to ``T`` tokens:
    moe_route -> fp8_quant_1x128 -> moe_permute -> grouped_gemm_fp8_swiglu -> moe_combine.

    With ``dispatch=False`` (default) the permute produces only the metadata and
    the first GEMM reads each token's FP8 row through row_token; with
    ``dispatch=True`` the rows are first copied into grouped order.

    ``scales="pow2"`` runs the power-of-two scale variant: X and H get
    power-of-two scales and the GEMMs use the hardware block-scaled MFMA (the
    weights must then be quantised with ``pow2=True``).

    From OVERLAP_QUANT_T tokens on, the activation quantisation runs on a
    side stream of the layer's own (default priority), forked from and joined
    back into the caller's stream within ``forward``, so the calls stay
    ordered on that stream as seen by the caller (and capturable in a graph)."""

    def __init__(self, T, d, E, n_groups, topk_groups, topk, f, route_scale=2.5, device="cuda",
                 dispatch=False, scales="fp32"):
        if scales not in ("fp32", "pow2"):
            raise ValueError(f"scales={scales!r} must be 'fp32' or 'pow2'")
        self.pow2 = scales == "pow2"
        self.T, self.d, self.E, self.k, self.f = T, d, E, topk, f
        self.n_groups, self.topk_groups, self.route_scale = n_groups, topk_groups, route_scale
        self.dispatch = dispatch
        self._side = None        # stream of the overlapped activation quantisation
        rows = T * topk + T
        dev = dict(device=device)
        self.idx = torch.empty(T, topk, dtype=torch.int32, **dev)
        self.w = torch.empty(T, topk, dtype=torch.float32, **dev)
        self.xq = torch.empty(T, d, dtype=torch.uint8, **dev)
        self.xs = torch.empty(T, d // 128, dtype=torch.float32, **dev)
        self.offsets = torch.empty(E + 2, dtype=torch.int32, **dev)
        self.pos = torch.empty(T, topk, dtype=torch.int32, **dev)
        self.row_token = torch.empty(rows, dtype=torch.int32, **dev)
        self.ws = torch.empty(max(16, moe_permute_workspace_bytes(T, topk, E)), dtype=torch.uint8, **dev)
        self.route_ws = torch.empty(max(16, moe_route_workspace_bytes(T, E)), dtype=torch.uint8, **dev)
        self.xq_perm = torch.empty(rows, d, dtype=torch.uint8, **dev) if dispatch else None
        self.xs_perm = torch.empty(rows, d // 128, dtype=torch.float32, **dev) if dispatch else None
        self.h = torch.empty(rows, f, dtype=torch.uint8, **dev)
        self.hs = torch.empty(rows, f // 128, dtype=torch.float32, **dev)
        self.y = torch.empty(rows, d, dtype=torch.bfloat16, **dev)
        self.out = torch.empty(T, d, dtype=torch.bfloat16, **dev)

    def forward(self, x, wg, bias, weights, stream=None, mark=None, train=False):
        """Run the layer on x [T, d].  ``mark(name)``, if given, is called after
        each stage is enqueued (the bench records HIP events there).  With
        ``train`` the first expert GEMM also caches [G, U] in FP8 for
        ``backward`` (FP32-scale method only)."""
        mark = mark or (lambda name: None)
        quant = fp8_quant_1x128_pow2 if self.pow2 else fp8_quant_1x128
        if self.T >= OVERLAP_QUANT_T:
            # the activation quantisation does not depend on the routing: on a
            # side stream it runs beside the router (whose workgroups leave
            # room on every CU), joined before the expert GEMMs.  The side
            # stream first waits for everything before this call on the
            # caller's stream (x, and the previous step's reads of xq/xs).
            main = torch.cuda.current_stream() if stream is None else stream
            if self._side is None:
                self._side = torch.cuda.Stream(device=x.device)
            self._side.wait_stream(main)
            quant(x, self.xq, self.xs, self._side)
            moe_route(x, wg, bias, self.n_groups, self.topk_groups, self.k, self.route_scale,
                      self.idx, self.w, main, workspace=self.route_ws)
            mark("route")
            main.wait_stream(self._side)
            mark("quant")
        else:
            moe_route(x, wg, bias, self.n_groups, self.topk_groups, self.k, self.route_scale,
                      self.idx, self.w, stream, workspace=self.route_ws)
            mark("route")
            quant(x, self.xq, self.xs, stream)
            mark("quant")
        if self.dispatch:
            moe_permute(self.idx, self.E, self.offsets, self.pos, self.row_token, self.ws,
                        self.xq, self.xs, self.xq_perm, self.xs_perm, stream)
            aq, as_, src = self.xq_perm, self.xs_perm, None
        else:
            moe_permute(self.idx, self.E, self.offsets, self.pos, self.row_token, self.ws,
                        stream=stream)
            aq, as_, src = self.xq, self.xs, self.row_token
        mark("permute")
        up = grouped_gemm_fp8_up_e8m0 if self.pow2 else grouped_gemm_fp8_up
        down = grouped_gemm_fp8_down_e8m0 if self.pow2 else grouped_gemm_fp8_down
        if train:
            if self.pow2:
                raise ValueError("the training forward runs the FP32-scale method")
            self._train_buffers()
            grouped_gemm_fp8_up_train(aq, as_, src, self.offsets, weights.w13q, weights.w13s, self.h,
                                      self.hs, self.gu, self.gus, stream)
        else:
            up(aq, as_, src, self.offsets, weights.w13q, weights.w13s, self.h, self.hs, stream)
        mark("gemm_up")
        down(self.h, self.hs, self.offsets, weights.w2q, weights.w2s, self.y, stream)
        mark("gemm_down")
        moe_combine(self.y, self.pos, self.w, self.T * self.k, self.out, stream)
        mark("combine")
        return self.out

    def _train_buffers(self):
        if getattr(self, "gu", None) is not None:
            return
        T, k, d, f, E = self.T, self.k, self.d, self.f, self.E
        rows, G = T * k + T, E + 1
        dev = dict(device=self.h.device)
        kp = moe_wgrad_columns(rows, G)
        self.gu = torch.empty(rows, 2 * f, dtype=torch.uint8, **dev)
        self.gus = torch.empty(rows, 2 * f // 128, dtype=torch.float32, **dev)
        self.dy = torch.empty(rows, d, dtype=torch.bfloat16, **dev)
        self.dw = torch.empty(T, k, dtype=torch.float32, **dev)
        self.dyq = torch.empty(rows, d, dtype=torch.uint8, **dev)
        self.dys = torch.empty(rows, d // 128, dtype=torch.float32, **dev)
        self.dh = torch.empty(rows, f, dtype=torch.bfloat16, **dev)
        self.dgu = torch.empty(rows, 2 * f, dtype=torch.uint8, **dev)
        self.dgus = torch.empty(rows, 2 * f // 128, dtype=torch.float32, **dev)
        self.dgu_t = torch.empty(2 * f, kp, dtype=torch.uint8, **dev)
        self.dgu_ts = torch.empty(kp // 128, 2 * f, dtype=torch.float32, **dev)
        self.h_t = torch.empty(f, kp, dtype=torch.uint8, **dev)
        self.h_ts = torch.empty(kp // 128, f, dtype=torch.float32, **dev)
        self.dy_t = torch.empty(d, kp, dtype=torch.uint8, **dev)
        self.dy_ts = torch.empty(kp // 128, d, dtype=torch.float32, **dev)
        self.x_t = torch.empty(d, kp, dtype=torch.uint8, **dev)
        self.x_ts = torch.empty(kp // 128, d, dtype=torch.float32, **dev)
        self.dx_rows = torch.empty(rows, d, dtype=torch.bfloat16, **dev)
        self.dx = torch.empty(T, d, dtype=torch.bfloat16, **dev)
        self.ones = torch.ones(T, k, dtype=torch.float32, **dev)
        self.dw13 = torch.empty(G, 2 * f, d, dtype=torch.float32, **dev)
        self.dw2 = torch.empty(G, d, f, dtype=torch.float32, **dev)

    def backward(self, dout, weights_t, stream=None, mark=None):
        """Backward of the last ``forward(..., train=True)`` for the output
        gradient dout [T, d] BF16, with ``weights_t = weights.transposed()``.
        Returns (dX [T, d] BF16, dW13 [E+1, 2f, d] FP32, dW2 [E+1, d, f] FP32,
        gate gradients [T, k] FP32).  Every backward quantisation uses
        power-of-two scales; Dgrad runs on grouped_gemm_fp8_down with the
        transposed weights, Wgrad on the K-major 128x1 operands."""
        mark = mark or (lambda name: None)
        T, k, d, f, E = self.T, self.k, self.d, self.f, self.E
        rows, G = T * k + T, E + 1
        moe_combine_backward(dout, self.y, self.pos, self.w, T * k, self.dy, self.dw, stream,
                             dyq=self.dyq, dys=self.dys)
        mark("combine_bwd")
        grouped_gemm_fp8_down(self.dyq, self.dys, self.offsets, weights_t.w2q, weights_t.w2s, self.dh, stream)
        mark("dgrad_w2")
        moe_swiglu_backward(self.gu, self.gus, self.dh, self.offsets, G, self.dgu, self.dgus,
                            self.dgu_t, self.dgu_ts, self.h_t, self.h_ts, stream)
        mark("swiglu_bwd")
        grouped_gemm_fp8_down(self.dgu, self.dgus, self.offsets, weights_t.w13q, weights_t.w13s,
                              self.dx_rows, stream)
        moe_combine(self.dx_rows, self.pos, self.ones, T * k, self.dx, stream)
        mark("dgrad_w13")
        moe_regroup_128x1(self.offsets, G, rows, self.dy_t, self.dy_ts, x_bf16=self.dy, stream=stream)
        moe_regroup_128x1(self.offsets, G, rows, self.x_t, self.x_ts, xq=self.xq, xs=self.xs,
                          row_src=self.row_token, stream=stream)
        mark("regroup")
        grouped_gemm_fp8_wgrad(self.dy_t, self.dy_ts, self.h_t, self.h_ts, self.offsets, G, rows,
                               self.dw2, stream)
        mark("wgrad_w2")
        grouped_gemm_fp8_wgrad(self.dgu_t, self.dgu_ts, self.x_t, self.x_ts, self.offsets, G, rows,
                               self.dw13, stream)
        mark("wgrad_w13")
        return self.dx, self.dw13, self.dw2, self.dw

    def update_bias(self, bias, gamma, stream=None):
        """After forward(): one step of the balancing controller on ``bias``
        [E] from this batch's expert loads (training-time only)."""
        moe_bias_update(self.offsets, bias, gamma, stream)
