"""Pins of the oracle's permute, blocked GEMM, SwiGLU and whole layer (CPU only)."""

import math

import numpy as np
import pytest
import torch

from oracle import fp8, quant, gemm, layer, permute as P, route as R
from routing_fp8_grouped_amd import configs, inputs


def brute_permute(idx, E):
    rows = []
    T, k = idx.shape
    for e in range(E):
        for t in range(T):
            if e in list(idx[t]):
                rows.append((e, t))
    return rows


def random_idx(rng, T, E, k):
    return np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(1, 4, 2), (37, 16, 4), (200, 32, 8), (0, 8, 2)])
def test_permute_brute_force(T, E, k):
    rng = np.random.default_rng(T + E + k)
    idx = random_idx(rng, T, E, k) if T else np.zeros((0, k), np.int32)
    offsets, pos, row_token = P.permute(idx, E)
    rows = brute_permute(idx, E)
    assert [t for _, t in rows] == list(row_token)
    for e in range(E):
        assert offsets[e + 1] - offsets[e] == sum(1 for ee, _ in rows if ee == e)
        assert all(rows[r][0] == e for r in range(offsets[e], offsets[e + 1]))
    assert offsets[E] == T * k and offsets[E + 1] == T * k + T
    # bijection onto [0, T*k) and consistency of pos with row_token
    assert sorted(pos.reshape(-1).tolist()) == list(range(T * k))
    for t in range(T):
        for j in range(k):
            assert row_token[pos[t, j]] == t
            assert offsets[idx[t, j]] <= pos[t, j] < offsets[idx[t, j] + 1]



def test_combine_residual():
    """The residual path is added once, unscaled, inside the single rounding:
    with no routed or shared contribution the output is the (BF16) residual
    itself; residual and shared rows play symmetric roles; a zero residual
    changes nothing; and a residual that cancels the shared row leaves the
    routed sum alone."""
    rng = np.random.default_rng(4)
    T, k, d = 9, 4, 256
    bf = lambda a: fp8.bf16_round(np.asarray(a, np.float32)).astype(np.float64)
    yr, ys, res = bf(rng.standard_normal((T, k, d))), bf(rng.standard_normal((T, d))), bf(rng.standard_normal((T, d)))
    w = rng.random((T, k)).astype(np.float32)
    zero_y, zero_w, zero_s = np.zeros((T, k, d)), np.zeros((T, k), np.float32), np.zeros((T, d))
    assert np.array_equal(layer.combine(zero_y, zero_w, zero_s, res), res)
    assert np.array_equal(layer.combine(yr, w, ys, res), layer.combine(yr, w, res, ys))
    assert np.array_equal(layer.combine(yr, w, ys, np.zeros((T, d))), layer.combine(yr, w, ys))
    assert np.array_equal(layer.combine(yr, w, ys, -ys), layer.combine(yr, w, zero_s))
    # one rounding of the exact sum, not a rounding per addend
    exact = np.einsum("tk,tkd->td", w.astype(np.float64), yr) + ys + res
    assert np.array_equal(layer.combine(yr, w, ys, res), fp8.bf16_round(exact))

@pytest.mark.parametrize("k", [4, 8])
def test_permute_combine_round_trip(k):
    """combine(permute(X), w = 1/k) == X bitwise (power-of-two weights)."""
    rng = np.random.default_rng(k)
    T, E, d = 64, 32, 256
    x = fp8.bf16_round(rng.standard_normal((T, d)))
    idx = random_idx(rng, T, E, k)
    offsets, pos, row_token = P.permute(idx, E)
    y = P.gather_rows(x, row_token, T)
    out = layer.combine(y[pos.astype(np.int64)], np.full((T, k), 1.0 / k, np.float32), np.zeros((T, d)))
    assert np.array_equal(out, x)
    # the shared rows are the identity
    assert np.array_equal(y[T * k:], x)


def test_blocked_gemm_equals_dense_dequantised():
    """Sum over K blocks of scaled exact partial sums == dense float64 GEMM of
    the dequantised operands (a textbook identity); N != K catches a transposed
    scale grid."""
    rng = np.random.default_rng(1)
    M, N, K = 7, 384, 640
    a = fp8.bf16_round(rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, K))))
    w = fp8.bf16_round(rng.standard_normal((N, K)) * 0.05 * np.exp(rng.standard_normal((N, 1))))
    qa, sa = quant.quant_1x128(a)
    qw, sw = quant.quant_128x128(w)
    y = gemm.blocked_gemm(qa, sa, qw, sw)
    dense = quant.dequant_1x128(qa, sa) @ quant.dequant_128x128(qw, sw).T
    assert np.allclose(y, dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())


def test_blocked_gemm_single_block_is_scaled_dot():
    rng = np.random.default_rng(2)
    qa = rng.choice(np.arange(0, 0x7E, dtype=np.uint8), (3, 128))
    qw = rng.choice(np.arange(0x80, 0xFE, dtype=np.uint8), (128, 128))
    sa = np.array([[0.5], [2.0], [0.125]], np.float32)
    sw = np.array([[4.0]], np.float32)
    y = gemm.blocked_gemm(qa, sa, qw, sw)
    for m in range(3):
        for n in (0, 17, 127):
            ref = sum(fp8.e4m3_decode(qa[m, i]) * fp8.e4m3_decode(qw[n, i]) for i in range(128))
            assert y[m, n] == sa[m, 0] * 4.0 * ref


def test_swiglu_closed_form():
    """SiLU(ln 3) = 0.75 ln 3 and SiLU(-ln 3) = -0.25 ln 3 (sigmoid(ln 3) = 3/4);
    SiLU is applied to the first (gate) argument only."""
    l3 = math.log(3.0)
    h = layer.swiglu(np.array([l3, -l3, 0.0, 2.0]), np.array([2.0, 2.0, 5.0, l3]))
    assert np.allclose(h, [1.5 * l3, -0.5 * l3, 0.0, 2.0 / (1 + math.exp(-2.0)) * l3], rtol=1e-7)


def test_expert_ffn_gate_rows_are_first_half():
    """W13 rows [0, f) are the gate branch: a very negative gate silences the
    expert whatever the up branch; the swapped reading would not."""
    d, f = 128, 128
    x = np.ones((2, d), np.float32)
    w13 = np.zeros((2 * f, d), np.float32)
    w13[:f] = -0.25            # g = -32 for every unit
    w13[f:] = 0.0625           # u = 8
    w2 = np.full((d, f), 0.0625, np.float32)
    xq, xs = quant.quant_1x128(x)
    y, inter = layer.expert_ffn(xq, xs, *layer.quantize_expert(w13, w2))
    assert np.all(np.abs(inter["h"]) < 1e-9)
    assert np.all(np.abs(y) < 1e-8)
    w13s = np.concatenate([w13[f:], w13[:f]])
    y2, _ = layer.expert_ffn(xq, xs, *layer.quantize_expert(w13s, w2))
    assert np.all(np.abs(y2) > 1.0)


def tiny_problem(T=48, d=256, E=8, G=4, M=2, k=4, f=128, seed=0):
    cfg = configs.MoEConfig("t", T=T, d=d, E=E, G=G, M=M, k=k, f=f, seed=seed)
    x, wg, b = inputs.host_inputs(cfg)
    ex = {}

    def experts(e):
        if e not in ex:
            w13, w2 = inputs.expert_weights(cfg, e)
            ex[e] = layer.quantize_expert(w13.float().numpy(), w2.float().numpy())
        return ex[e]
    return cfg, x.float().numpy(), wg.float().numpy(), b.numpy(), experts


def test_dense_special_case_k_equals_E():
    """k = E with all groups kept selects every expert; the layer is then the
    dense gated sum over all experts plus the shared expert."""
    cfg, x, wg, b, experts = tiny_problem(E=8, G=4, M=4, k=8)
    res = layer.moe_layer(x, wg, b, experts, cfg.G, cfg.M, cfg.k, 2.5)
    assert np.all(res["route"]["idx"] == np.arange(8))
    xq, xs = quant.quant_1x128(x)
    s = R.affinity(x, wg)
    acc = np.zeros((cfg.T, cfg.d))
    for e in range(cfg.E):
        ye, _ = layer.expert_ffn(xq, xs, *experts(e))
        acc += (2.5 * s[:, e] / s.sum(axis=1)).astype(np.float32)[:, None].astype(np.float64) * ye
    ysh, _ = layer.expert_ffn(xq, xs, *experts(cfg.E))
    dense = fp8.bf16_round(acc + ysh)
    assert np.array_equal(res["out"], dense)


def test_route_scale_zero_gives_shared_expert_only():
    cfg, x, wg, b, experts = tiny_problem()
    res = layer.moe_layer(x, wg, b, experts, cfg.G, cfg.M, cfg.k, 0.0)
    xq, xs = quant.quant_1x128(x)
    ysh, _ = layer.expert_ffn(xq, xs, *experts(cfg.E))
    assert np.array_equal(res["out"], ysh)


def test_sampled_tokens_equal_full_batch():
    cfg, x, wg, b, experts = tiny_problem(T=64)
    res = layer.moe_layer(x, wg, b, experts, cfg.G, cfg.M, cfg.k, 2.5)
    sample = [0, 5, 17, 63]
    out, r, extra = layer.moe_layer_tokens(x[sample], wg, b, experts, cfg.G, cfg.M, cfg.k, 2.5)
    assert np.array_equal(out, res["out"][sample])
    assert np.array_equal(r["idx"], res["route"]["idx"][sample])
    for i, t in enumerate(sample):
        for j in range(cfg.k):
            p = res["pos"][t, j]
            assert np.array_equal(extra["inter_routed"][(i, j)]["hq"][0], res["hq"][p])
            assert np.array_equal(extra["y_routed"][i, j], res["y"][p])
        assert np.array_equal(extra["inter_shared"][i]["h"][0], res["h"][cfg.T * cfg.k + t])


def test_flop_figures(golden):
    """Per-token expert FLOPs printed on the pages: 704.6 M (top-8 routed) and
    792.72 M (with the shared expert) at d = 7168, f = 2048."""
    g = golden["expert_flops"]
    cfg = configs.get("prefill_4k")
    assert round(cfg.k * 6 * cfg.d * cfg.f / 1e6, 1) == g["routed_mflop_per_token_1dp"]
    assert round(cfg.gemm_flops() / cfg.T / 1e6, 2) == g["with_shared_mflop_per_token_2dp"]
