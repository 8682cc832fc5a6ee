"""Pins of the backward oracle (oracle/backward.py) against automatic
differentiation in float64 (torch on the CPU) and against the properties the
pages state for the regrouping."""

import numpy as np
import torch

from oracle import backward as ob, fp8, quant


def _t(a):
    return torch.tensor(np.asarray(a, np.float64), requires_grad=True)


def test_swiglu_backward_matches_autograd():
    rng = np.random.default_rng(1)
    g, u, dh = rng.normal(0, 3, (3, 64, 96))
    tg, tu = _t(g), _t(u)
    h = torch.nn.functional.silu(tg) * tu
    h.backward(torch.tensor(dh))
    rh, rdg, rdu = ob.swiglu_backward(g, u, dh)
    assert np.allclose(rh, h.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(rdg, tg.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(rdu, tu.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_combine_backward_matches_autograd():
    rng = np.random.default_rng(2)
    T, k, d, E = 9, 3, 16, 5
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    from oracle import permute as op
    _, pos, _ = op.permute(idx, E)
    y = rng.standard_normal((T * k + T, d))
    w = rng.uniform(0.1, 1.0, (T, k))
    dout = rng.standard_normal((T, d))
    ty, tw = _t(y), _t(w)
    out = (tw[:, :, None] * ty[torch.tensor(pos, dtype=torch.long)]).sum(1) + ty[T * k:]
    out.backward(torch.tensor(dout))
    dy, dw = ob.combine_backward(dout, y, w, pos, T, k, quantize=False)
    assert np.allclose(dy, ty.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dw, tw.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_expert_backward_matches_autograd():
    """Without quantisation the expert's backward is the exact gradient of
    y = (SiLU(x W1^T) * (x W3^T)) W2^T: a transposed operand, a swapped branch
    or a wrong index in any of the five products changes one of the four."""
    rng = np.random.default_rng(3)
    rows, d, f = 40, 24, 16
    x = rng.standard_normal((rows, d))
    w13 = rng.standard_normal((2 * f, d)) / 5
    w2 = rng.standard_normal((d, f)) / 4
    dy = rng.standard_normal((rows, d))
    tx, tw13, tw2 = _t(x), _t(w13), _t(w2)
    gu = tx @ tw13.T
    y = (torch.nn.functional.silu(gu[:, :f]) * gu[:, f:]) @ tw2.T
    y.backward(torch.tensor(dy))
    r = ob.expert_backward(x, gu.detach().numpy(), dy, w13, w2, quantize=False)
    assert np.allclose(r["dw2"], tw2.grad.numpy(), rtol=1e-10, atol=1e-10)
    assert np.allclose(r["dw13"], tw13.grad.numpy(), rtol=1e-10, atol=1e-10)
    # dX through both branches of the SwiGLU
    assert np.allclose(r["dx"], tx.grad.numpy(), rtol=1e-10, atol=1e-10)


def test_token_grad_matches_autograd():
    rng = np.random.default_rng(4)
    T, k, d, E = 7, 2, 8, 4
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    from oracle import permute as op
    _, pos, row_token = op.permute(idx, E)
    x = _t(rng.standard_normal((T, d)))
    rows = torch.cat([x[torch.tensor(row_token, dtype=torch.long)], x])    # the dispatch
    g = rng.standard_normal((T * k + T, d))
    rows.backward(torch.tensor(g))
    assert np.allclose(ob.token_grad(g, pos, T, k, quantize=False), x.grad.numpy(), rtol=1e-12)


def test_quant_128x1_is_the_transposed_1x128_quantisation():
    rng = np.random.default_rng(5)
    x = fp8.bf16_round(rng.standard_normal((300, 256)) * np.exp(rng.normal(0, 2, (1, 256)))).astype(np.float32)
    q, s = ob.quant_128x1(x)
    assert q.shape == (384, 256) and s.shape == (3, 256)
    assert np.all(q[300:] == 0)                               # padding rows
    # each 128-row block of a column is one tile: scale = pow2 rule of its amax
    xp = np.zeros((384, 256), np.float32); xp[:300] = x
    amax = np.abs(xp.reshape(3, 128, 256)).max(1)
    assert np.array_equal(s, quant.scale_from_amax(amax, "pow2"))
    assert np.array_equal(q[:300], fp8.e4m3_encode((xp.reshape(3, 128, 256) / s[:, None, :]).astype(np.float32)).reshape(384, 256)[:300])


def test_regrouping_power_of_two_tiles_is_exact_above_the_subnormals():
    """The pages use power-of-two scales so that regrouping 1x128 tiles into
    128x1 tiles adds no quantisation error: every value of a power-of-two
    scaled E4M3 tile is representable again after the rescaling, except where
    it falls into the E4M3 subnormal range of its new tile."""
    rng = np.random.default_rng(6)
    x = fp8.bf16_round(rng.standard_normal((256, 512)) * np.exp(rng.normal(0, 1, (256, 1)))).astype(np.float32)
    q1, s1 = quant.quant_1x128(x, "pow2")
    v1 = quant.dequant_1x128(q1, s1).astype(np.float32)            # exact in FP32
    q2, s2 = ob.quant_128x1(v1)
    v2 = ob.dequant_128x1(q2, s2)[:256]
    changed = v2 != v1
    scaled = np.abs(v1) / np.repeat(s2, 128, axis=0)[:256]
    assert not np.any(changed & (scaled >= 2.0 ** -6))            # normal range: exact
    assert changed.mean() < 0.1
    # with amax/448 scales the same regrouping rounds most values again
    q3, s3 = quant.quant_1x128(x, "fp32")
    v3 = quant.dequant_1x128(q3, s3).astype(np.float32)
    q4, s4 = quant.quant_1x128(np.ascontiguousarray(v3.T), "fp32")
    assert (quant.dequant_1x128(q4, s4).T != v3).mean() > 0.3


def test_quantised_backward_is_close_to_exact():
    """With every backward quantisation on, the gradients stay within FP8
    distance of the exact ones (relative L2 of a few percent)."""
    rng = np.random.default_rng(7)
    rows, d, f = 200, 256, 128
    x = fp8.bf16_round(rng.standard_normal((rows, d))).astype(np.float32)
    w13 = fp8.bf16_round(rng.standard_normal((2 * f, d)) / 16).astype(np.float32)
    w2 = fp8.bf16_round(rng.standard_normal((d, f)) / 11).astype(np.float32)
    xq = quant.quant_1x128(x)
    w13q, w2q = quant.quant_128x128(w13), quant.quant_128x128(w2)
    gu = ob.f32(quant.dequant_1x128(*xq) @ quant.dequant_128x128(*w13q).T)
    guq = quant.quant_1x128(gu)
    dy = fp8.bf16_round(rng.standard_normal((rows, d))).astype(np.float32)
    rq = ob.expert_backward(xq, guq, dy, w13q, w2q, quantize=True)
    rx = ob.expert_backward(quant.dequant_1x128(*xq), quant.dequant_1x128(*guq), dy,
                            quant.dequant_128x128(*w13q), quant.dequant_128x128(*w2q), quantize=False)
    for key in ("dx", "dw13", "dw2", "dh"):
        err = np.linalg.norm(rq[key] - rx[key]) / np.linalg.norm(rx[key])
        assert err < 0.08, (key, err)
        assert err > 1e-4, key                                   # quantisation did happen
