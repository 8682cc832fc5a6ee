"""GPU parity of the backward (scope row f2) against the backward oracle:
weight transposition, combine backward, the 128x1 regrouping, SwiGLU backward
from the FP8 cache, the Wgrad GEMM, the forward's [G, U] cache, and the tiny
layer's whole backward.

Bars: byte outputs bit-exact where both sides make the same FP32/FP64 roundings
(transposition, dY, regrouping, SwiGLU backward codes, except where an FP64
exp of the two sides differs in its last bit: at most a few codes in a
million, one step); FP32 sums within their accumulation bound; GEMM outputs
within the MFMA noise model of tests/gpu_util.py; layer gradients within
relative L2 5e-3."""

import numpy as np
import pytest
import torch

import routing_fp8_grouped_amd as moe
from routing_fp8_grouped_amd import configs, inputs
from oracle import backward as ob, fp8, quant as oq, permute as operm, layer as olayer
from tests.gpu_util import (DEV, log, to_np, code_ambiguity, check_h_codes, gemm_noise,
                            block_max_products, MAXPROD_FACTOR, device_weights, OracleExperts,
                            rel_l2_rows, random_layer_config)
from tests.test_gpu_kernels import bf16_tensor, gemm_case

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def D(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def kmajor(vals, offsets):
    """The oracle's K-major 128x1 operand of vals [rows, C] (grouped order)."""
    offsets = np.asarray(offsets)
    G = len(offsets) - 1
    rows, C = vals.shape
    kp = moe.moe_wgrad_columns(rows, G)
    q = np.zeros((C, kp), np.uint8)
    s = np.zeros((kp // 128, C), np.float32)
    col = 0
    for e in range(G):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        qe, se = ob.quant_128x1(vals[r0:r1])
        q[:, col:col + qe.shape[0]] = qe.T
        s[col // 128:col // 128 + se.shape[0]] = se
        col += qe.shape[0]
    return q, s, col


def offsets_of(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def test_transpose_fp8_blocks():
    rng = np.random.default_rng(1)
    G, N, K = 3, 256, 384
    w = rng.integers(0, 256, (G, N, K), dtype=np.uint8)
    ws = rng.uniform(0.1, 2.0, (G, N // 128, K // 128)).astype(np.float32)
    wt = torch.empty(G, K, N, dtype=torch.uint8, device=DEV)
    wts = torch.empty(G, K // 128, N // 128, dtype=torch.float32, device=DEV)
    moe.moe_transpose_fp8_blocks(D(w), D(ws), wt, wts)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(wt), w.transpose(0, 2, 1))
    assert np.array_equal(to_np(wts), ws.transpose(0, 2, 1))


def test_combine_backward():
    rng = np.random.default_rng(2)
    T, k, E, d = 37, 4, 16, 384
    idx = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)])
    _, pos, _ = operm.permute(idx, E)
    rows = T * k + T
    y = bf16_tensor(rng.standard_normal((rows, d)))
    dout = bf16_tensor(rng.standard_normal((T, d)))
    w = rng.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    dy = torch.empty(rows, d, dtype=torch.bfloat16, device=DEV)
    dw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    moe.moe_combine_backward(dout.to(DEV), y.to(DEV), D(pos), D(w), T * k, dy, dw)
    torch.cuda.synchronize()
    rdy, rdw = ob.combine_backward(dout.float().numpy(), y.float().numpy(), w, pos, T, k)
    assert np.array_equal(to_np(dy), rdy)
    # FP32 sum of d products: within d ulps of the sum of magnitudes
    bound = d * 2.0 ** -24 * np.einsum("td,tkd->tk", np.abs(dout.float().numpy()),
                                        np.abs(y.float().numpy())[pos])
    assert np.all(np.abs(to_np(dw) - rdw) <= bound + 1e-30)


@pytest.mark.parametrize("T,k,E,d", [(37, 4, 16, 384), (64, 8, 256, 7168)])
def test_combine_backward_quantising(T, k, E, d):
    """moe_combine_backward_q: the same dY and gate gradients, and the 1x128
    power-of-two copy of dY bit for bit what fp8_quant_1x128_pow2 makes of it
    and what the oracle's power-of-two rule makes of its dY."""
    log(f"combine backward with dY quantisation T={T} k={k} d={d}")
    rng = np.random.default_rng(20 + T)
    idx = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)])
    _, pos, _ = operm.permute(idx, E)
    rows = T * k + T
    y = bf16_tensor(rng.standard_normal((rows, d)))
    dout = bf16_tensor(rng.standard_normal((T, d)) * np.exp(rng.normal(0, 2, (T, 1))))
    w = rng.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    dy = torch.empty(rows, d, dtype=torch.bfloat16, device=DEV)
    dw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    dyq = torch.empty(rows, d, dtype=torch.uint8, device=DEV)
    dys = torch.empty(rows, d // 128, dtype=torch.float32, device=DEV)
    dw0 = torch.empty_like(dw)
    dy0 = torch.empty_like(dy)
    moe.moe_combine_backward(dout.to(DEV), y.to(DEV), D(pos), D(w), T * k, dy0, dw0)
    moe.moe_combine_backward(dout.to(DEV), y.to(DEV), D(pos), D(w), T * k, dy, dw, dyq=dyq, dys=dys)
    q2 = torch.empty_like(dyq)
    s2 = torch.empty_like(dys)
    moe.fp8_quant_1x128_pow2(dy, q2, s2)
    torch.cuda.synchronize()
    rdy, _ = ob.combine_backward(dout.float().numpy(), y.float().numpy(), w, pos, T, k)
    assert np.array_equal(to_np(dy), rdy)
    assert torch.equal(dy.view(torch.int16), dy0.view(torch.int16)) and torch.equal(dw, dw0)
    assert torch.equal(dyq, q2) and torch.equal(dys, s2)
    rq, rs = oq.quant_1x128(rdy, "pow2")
    assert np.array_equal(to_np(dyq), rq) and np.array_equal(to_np(dys), rs)


@pytest.mark.parametrize("quantising", [False, True])
def test_combine_backward_unassigned_slots(quantising):
    """Slots whose pos lies outside the rows (an unassigned slot, pos = -1, or
    past the end) get a zero gate gradient and write no dY row (nor its FP8
    copy); every other row is written as usual."""
    rng = np.random.default_rng(31)
    T, k, E, d = 9, 4, 16, 256
    idx = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)])
    _, pos, _ = operm.permute(idx, E)
    rows = T * k + T
    bad = [(3, 1, -1), (5, 2, rows + 7)]
    freed = [int(pos[t, j]) for t, j, _ in bad]
    for t, j, v in bad:
        pos[t, j] = v
    y = bf16_tensor(rng.standard_normal((rows, d)))
    dout = bf16_tensor(rng.standard_normal((T, d)))
    w = rng.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    sentinel = bf16_tensor(np.full((rows, d), 3.0))
    dy = sentinel.to(DEV).clone()
    dw = torch.full((T, k), 7.0, dtype=torch.float32, device=DEV)
    dyq = torch.full((rows, d), 0x55, dtype=torch.uint8, device=DEV)
    dys = torch.full((rows, d // 128), 9.0, dtype=torch.float32, device=DEV)
    if quantising:
        moe.moe_combine_backward(dout.to(DEV), y.to(DEV), D(pos), D(w), T * k, dy, dw, dyq=dyq, dys=dys)
    else:
        moe.moe_combine_backward(dout.to(DEV), y.to(DEV), D(pos), D(w), T * k, dy, dw)
    torch.cuda.synchronize()
    gdy, gdw = to_np(dy), to_np(dw)
    dn = dout.float().numpy()
    want = sentinel.float().numpy().copy()
    for t in range(T):
        for j in range(k):
            if 0 <= pos[t, j] < rows:
                want[pos[t, j]] = fp8.bf16_round(fp8.f32(np.float32(w[t, j]) * dn[t].astype(np.float32)))
        want[T * k + t] = dn[t]
    assert np.array_equal(gdy, want)
    for t, j, _ in bad:
        assert gdw[t, j] == 0.0
    assert np.all(gdw[gdw != 0.0] != 7.0)
    for r in freed:
        assert np.array_equal(gdy[r], sentinel.float().numpy()[r])
        if quantising:
            assert torch.all(dyq[r] == 0x55) and torch.all(dys[r] == 9.0)


def _routing(rng, T, k, E, empty=()):
    allowed = [e for e in range(E) if e not in empty]
    idx = np.stack([np.sort(rng.choice(allowed, k, replace=False)) for _ in range(T)])
    offsets, pos, row_token = operm.permute(idx, E)
    return offsets, pos, np.concatenate([row_token, np.arange(T)]).astype(np.int32)


def test_regroup_from_fp8_cache_and_bf16():
    rng = np.random.default_rng(3)
    T, k, E, d = 300, 3, 9, 384
    offsets, _, row_token = _routing(rng, T, k, E, empty=(2, 5))
    G, rows = E + 1, T * k + T
    x = bf16_tensor(rng.standard_normal((T, d)) * np.exp(rng.normal(0, 1.5, (T, 1))))
    xq, xs = oq.quant_1x128(x.float().numpy())
    kp = moe.moe_wgrad_columns(rows, G)
    out = torch.zeros(d, kp, dtype=torch.uint8, device=DEV)
    out_s = torch.zeros(kp // 128, d, dtype=torch.float32, device=DEV)
    moe.moe_regroup_128x1(D(offsets), G, rows, out, out_s, xq=D(xq), xs=D(xs), row_src=D(row_token))
    torch.cuda.synchronize()
    xv = fp8.f32(oq.dequant_1x128(xq, xs))[row_token]
    rq, rs, ncol = kmajor(xv, offsets)
    log(f"  regroup from the FP8 cache: {ncol} of {kp} columns")
    assert np.array_equal(to_np(out)[:, :ncol], rq[:, :ncol])
    assert np.array_equal(to_np(out_s)[:ncol // 128], rs[:ncol // 128])
    # BF16 source in grouped order (the output gradient of the experts)
    dy = bf16_tensor(rng.standard_normal((rows, d)))
    moe.moe_regroup_128x1(D(offsets), G, rows, out, out_s, x_bf16=dy.to(DEV))
    torch.cuda.synchronize()
    rq, rs, ncol = kmajor(dy.float().numpy(), offsets)
    assert np.array_equal(to_np(out)[:, :ncol], rq[:, :ncol])
    assert np.array_equal(to_np(out_s)[:ncol // 128], rs[:ncol // 128])


def _close_codes(got, ref, what, max_frac=1e-5):
    """Equal codes except a few (FP64 exp last-bit differences), each one step."""
    diff = got != ref
    n = int(diff.sum())
    if n:
        dv = np.abs(fp8.e4m3_decode(got[diff]) - fp8.e4m3_decode(ref[diff]))
        sp = np.maximum(fp8.e4m3_decode(np.maximum(got[diff] & 0x7F, ref[diff] & 0x7F)), 2.0 ** -9)
        assert np.all(dv <= sp * 0.126 + 2.0 ** -9), what
    assert n <= max(1, max_frac * got.size), (what, n)
    return n


def test_swiglu_backward():
    rng = np.random.default_rng(4)
    f = 256
    counts = [0, 130, 1, 257, 64, 128]
    offsets = offsets_of(counts)
    G, rows = len(counts), int(offsets[-1])
    gu = (rng.standard_normal((rows, 2 * f)) * np.exp(rng.normal(0, 1, (rows, 1)))).astype(np.float32)
    guq, gus = oq.quant_1x128(gu)
    dh = bf16_tensor(rng.standard_normal((rows, f)) * 0.3)
    kp = moe.moe_wgrad_columns(rows, G)
    dgu = torch.empty(rows, 2 * f, dtype=torch.uint8, device=DEV)
    dgus = torch.empty(rows, 2 * f // 128, dtype=torch.float32, device=DEV)
    dgu_t = torch.zeros(2 * f, kp, dtype=torch.uint8, device=DEV)
    dgu_ts = torch.zeros(kp // 128, 2 * f, dtype=torch.float32, device=DEV)
    h_t = torch.zeros(f, kp, dtype=torch.uint8, device=DEV)
    h_ts = torch.zeros(kp // 128, f, dtype=torch.float32, device=DEV)
    moe.moe_swiglu_backward(D(guq), D(gus), dh.to(DEV), D(offsets), G, dgu, dgus, dgu_t, dgu_ts, h_t, h_ts)
    torch.cuda.synchronize()
    gv = fp8.f32(oq.dequant_1x128(guq, gus))
    h, dg, du = (fp8.f32(v) for v in ob.swiglu_backward(gv[:, :f], gv[:, f:], dh.float().numpy()))
    dguv = np.concatenate([dg, du], axis=1)
    rq, rs = oq.quant_1x128(dguv, "pow2")
    n = _close_codes(to_np(dgu), rq, "dgu")
    assert np.array_equal(to_np(dgus), rs)
    tq, ts, ncol = kmajor(dguv, offsets)
    n += _close_codes(to_np(dgu_t)[:, :ncol], tq[:, :ncol], "dgu_t")
    assert np.array_equal(to_np(dgu_ts)[:ncol // 128], ts[:ncol // 128])
    hq, hs_, _ = kmajor(h, offsets)
    n += _close_codes(to_np(h_t)[:, :ncol], hq[:, :ncol], "h_t")
    assert np.array_equal(to_np(h_ts)[:ncol // 128], hs_[:ncol // 128])
    log(f"  swiglu backward: {n} codes differ in the last bit of FP64 exp")


def wgrad_bound(aq, as_, bq, bs, exact):
    """MFMA noise bound of a product whose operands are scaled per row and K
    block: the largest-product model of tests/gpu_util.py plus FP32
    accumulation of the chained blocks."""
    nkb = aq.shape[1] // 128
    return MAXPROD_FACTOR * block_max_products(aq, as_, bq, bs) + nkb * 2.0 ** -24 * np.abs(exact)


@pytest.mark.parametrize("counts,M,N", [([0, 5, 130, 300, 1], 256, 384), ([700, 0, 129], 512, 256)])
def test_wgrad(counts, M, N):
    rng = np.random.default_rng(sum(counts) + M)
    offsets = offsets_of(counts)
    G, rows = len(counts), int(offsets[-1])
    av = (rng.standard_normal((rows, M)) * np.exp(rng.normal(0, 1, (rows, 1)))).astype(np.float32)
    bv = rng.standard_normal((rows, N)).astype(np.float32)
    aq, as_, _ = kmajor(av, offsets)
    bq, bs, _ = kmajor(bv, offsets)
    dw = torch.full((G, M, N), 7.0, dtype=torch.float32, device=DEV)
    moe.grouped_gemm_fp8_wgrad(D(aq), D(as_), D(bq), D(bs), D(offsets), G, rows, dw)
    torch.cuda.synchronize()
    g = to_np(dw)
    col = 0
    worst = 0.0
    for e in range(G):
        n = -(-counts[e] // 128) * 128
        if n == 0:
            assert np.all(g[e] == 0.0)
            continue
        sl = slice(col, col + n)
        exact = ob.gemm_rows_scaled(aq[:, sl], as_[col // 128:(col + n) // 128].T,
                                    bq[:, sl], bs[col // 128:(col + n) // 128].T)
        bound = wgrad_bound(aq[:, sl], as_[col // 128:(col + n) // 128].T, bq[:, sl],
                            bs[col // 128:(col + n) // 128].T, exact)
        err = np.abs(g[e] - exact)
        assert np.all(err <= bound), (e, float((err / np.maximum(bound, 1e-300)).max()))
        worst = max(worst, float(np.linalg.norm(g[e] - exact) / np.linalg.norm(exact)))
        col += n
    log(f"  wgrad {counts} M={M} N={N}: relative Frobenius error max {worst:.2e}")


def test_wgrad_expert_walk():
    """The 256 x 256 kernel's workgroups walk several experts each (more
    groups than slices), across experts without rows: sampled elements of
    every expert against the oracle, empty experts all zero."""
    rng = np.random.default_rng(11)
    M, N, G = 2048, 1024, 150          # 32 tiles -> 64 slices of about 2-3 experts
    counts = rng.integers(0, 200, G)
    counts[rng.random(G) < 0.2] = 0
    counts[[0, 1, G - 1]] = [0, 0, 131]
    offsets = offsets_of(counts)
    rows = int(offsets[-1])
    av = (rng.standard_normal((rows, M)) * np.exp(rng.normal(0, 1, (rows, 1)))).astype(np.float32)
    bv = rng.standard_normal((rows, N)).astype(np.float32)
    aq, as_, _ = kmajor(av, offsets)
    bq, bs, _ = kmajor(bv, offsets)
    dw = torch.full((G, M, N), 7.0, dtype=torch.float32, device=DEV)
    moe.grouped_gemm_fp8_wgrad(D(aq), D(as_), D(bq), D(bs), D(offsets), G, rows, dw)
    torch.cuda.synchronize()
    col = 0
    worst = 0.0
    for e in range(G):
        n = -(-int(counts[e]) // 128) * 128
        if n == 0:
            assert bool((dw[e] == 0).all()), e
            continue
        mi = np.sort(rng.choice(M, 24, replace=False))
        ni = np.sort(rng.choice(N, 24, replace=False))
        got = to_np(dw[e][torch.from_numpy(mi).to(DEV)][:, torch.from_numpy(ni).to(DEV)])
        sl, ss = slice(col, col + n), slice(col // 128, (col + n) // 128)
        a_, sa = aq[mi][:, sl], as_[ss][:, mi].T.copy()
        b_, sb = bq[ni][:, sl], bs[ss][:, ni].T.copy()
        exact = ob.gemm_rows_scaled(a_, sa, b_, sb)
        err = np.abs(got - exact)
        bound = wgrad_bound(a_, sa, b_, sb, exact)
        assert np.all(err <= bound), (e, float((err / np.maximum(bound, 1e-300)).max()))
        worst = max(worst, float(np.linalg.norm(got - exact) / np.linalg.norm(exact)))
        col += n
    log(f"  wgrad walk: {G} groups ({int((counts == 0).sum())} empty), sampled relative error max {worst:.2e}")


def test_up_train_cache():
    """The training forward writes the same h as the plain one, plus [G, U] in
    1x128 FP8 tiles (the forward's amax/448 rule) within the MFMA noise."""
    rng = np.random.default_rng(5)
    counts, d, f = [40, 300, 0, 129], 384, 256
    rows = sum(counts)
    offsets, aq, as_, row_src, experts = gemm_case(rng, counts, d, f, rows + 20, True)
    W = moe.MoEWeights.empty(len(counts), d, f)
    for g, (w13q, w13s, w2q, w2s) in enumerate(experts):
        W.w13q[g].copy_(torch.from_numpy(w13q)); W.w13s[g].copy_(torch.from_numpy(w13s))
    h1 = torch.empty(rows, f, dtype=torch.uint8, device=DEV); hs1 = torch.empty(rows, f // 128, device=DEV)
    h2 = torch.empty_like(h1); hs2 = torch.empty_like(hs1)
    gu = torch.empty(rows, 2 * f, dtype=torch.uint8, device=DEV)
    gus = torch.empty(rows, 2 * f // 128, dtype=torch.float32, device=DEV)
    args = (D(aq), D(as_), D(row_src), D(offsets), W.w13q, W.w13s)
    moe.grouped_gemm_fp8_up(*args, h1, hs1)
    moe.grouped_gemm_fp8_up_train(*args, h2, hs2, gu, gus)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2) and torch.equal(hs1, hs2)
    gg, ggs = to_np(gu), to_np(gus)
    n_amb = n_diff = 0
    for e in range(len(counts)):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        w13q, w13s = experts[e][0], experts[e][1]
        a_e, s_e = aq[row_src[lo:hi]], as_[row_src[lo:hi]]
        exact = olayer.blocked_gemm(a_e, s_e, w13q, w13s)
        v = fp8.f32(exact)
        rq, rs = oq.quant_1x128(v)
        assert np.allclose(ggs[lo:hi], rs, rtol=2e-4)
        amb, step = code_ambiguity(v, gemm_noise(a_e, s_e, w13q, w13s, exact), ggs[lo:hi])
        n_diff += check_h_codes(gg[lo:hi], rq, amb, step)
        n_amb += int(amb.sum())
    log(f"  [G, U] cache: {n_amb} ambiguous codes, {n_diff} differ")


def test_tiny_layer_backward():
    """The whole backward of the tiny layer, stage by stage, each against the
    backward oracle fed with the GPU's own inputs to that stage (so every
    check is bit-exact or within one GEMM's noise), then dX end to end."""
    check_layer_backward(configs.get("tiny"), 6)


@pytest.mark.parametrize("seed", [0, 3, 5, 9, 17, 20])
def test_layer_backward_random(seed):
    """The same stage-by-stage backward checks on seeded random layers (T up
    to 300, E 8-32, d and f 128-384; the forward on the weight-streaming or
    the tiled GEMM)."""
    check_layer_backward(random_layer_config(seed), 100 + seed)


def check_layer_backward(cfg, dout_seed):
    log(f"layer backward {cfg.name}: T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} G={cfg.G} M={cfg.M} k={cfg.k}")
    x, wg, b = inputs.host_inputs(cfg)
    bf16 = {}
    W = device_weights(cfg, bf16)
    Wt = W.transposed()
    L = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.f, cfg.route_scale)
    L.forward(x.to(DEV), wg.to(DEV), b.to(DEV), W, train=True)
    rng = np.random.default_rng(dout_seed)
    dout = bf16_tensor(rng.standard_normal((cfg.T, cfg.d)))
    dx, dw13, dw2, dgate = L.backward(dout.to(DEV), Wt)
    torch.cuda.synchronize()
    T, k, E, d, f = cfg.T, cfg.k, cfg.E, cfg.d, cfg.f
    pos, off, rt = to_np(L.pos), to_np(L.offsets), to_np(L.row_token)
    # combine backward: dY bit-exact, gate gradients within the FP32 sum's bound
    rdy, rdw = ob.combine_backward(dout.float().numpy(), to_np(L.y), to_np(L.w), pos, T, k)
    assert np.array_equal(to_np(L.dy), rdy)
    assert np.allclose(to_np(dgate), rdw, rtol=1e-4, atol=1e-6)
    dyq, dys = oq.quant_1x128(rdy, "pow2")
    assert np.array_equal(to_np(L.dyq), dyq) and np.array_equal(to_np(L.dys), dys)
    oe = OracleExperts(cfg, bf16)
    oe.prepare(range(E + 1))
    gdh, gdgu, gdgus, gdx_rows = to_np(L.dh), to_np(L.dgu), to_np(L.dgus), to_np(L.dx_rows)
    gu, gus = to_np(L.gu), to_np(L.gus)
    g13, g2 = to_np(dw13), to_np(dw2)
    kp = moe.moe_wgrad_columns(T * k + T, E + 1)
    worst = {"dh": 0.0, "dx_rows": 0.0, "dw": 0.0}
    # per expert: Dgrad W2, SwiGLU backward, Dgrad W13
    for e in range(E + 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        w13q, w13s, w2q, w2s = oe(e)
        rdh = fp8.bf16_round(fp8.f32(olayer.blocked_gemm(dyq[lo:hi], dys[lo:hi], w2q.T.copy(), w2s.T.copy())))
        e_dh = rel_l2_rows(gdh[lo:hi], rdh)
        gv = fp8.f32(oq.dequant_1x128(gu[lo:hi], gus[lo:hi]))
        _, dg, du = (fp8.f32(v) for v in ob.swiglu_backward(gv[:, :f], gv[:, f:], gdh[lo:hi]))
        rq, rs = oq.quant_1x128(np.concatenate([dg, du], axis=1), "pow2")
        _close_codes(gdgu[lo:hi], rq, "dgu")
        assert np.array_equal(gdgus[lo:hi], rs)
        rdx = fp8.bf16_round(fp8.f32(olayer.blocked_gemm(gdgu[lo:hi], gdgus[lo:hi], w13q.T.copy(), w13s.T.copy())))
        e_dx = rel_l2_rows(gdx_rows[lo:hi], rdx)
        assert e_dh.max() <= TOL and e_dx.max() <= TOL, (e, e_dh.max(), e_dx.max())
        worst["dh"] = max(worst["dh"], float(e_dh.max()))
        worst["dx_rows"] = max(worst["dx_rows"], float(e_dx.max()))
    # the Wgrad operands: dY and X regrouped, [dG, dU] and h from the SwiGLU backward
    for name, vals in (("dy_t", rdy), ("x_t", fp8.f32(oq.dequant_1x128(to_np(L.xq), to_np(L.xs)))[rt])):
        q, s_, ncol = kmajor(vals, off)
        assert np.array_equal(to_np(getattr(L, name))[:, :ncol], q[:, :ncol]), name
        assert np.array_equal(to_np(getattr(L, name + "s"))[:ncol // 128], s_[:ncol // 128]), name
    # Wgrad on the GPU's operands
    ops = {n: (to_np(getattr(L, n)), to_np(getattr(L, n + "s"))) for n in ("dy_t", "h_t", "dgu_t", "x_t")}
    col = 0
    for e in range(E + 1):
        n = -(-int(off[e + 1] - off[e]) // 128) * 128
        if n == 0:
            assert np.all(g13[e] == 0) and np.all(g2[e] == 0)
            continue
        sl, ss = slice(col, col + n), slice(col // 128, (col + n) // 128)
        for got, (a, b_) in ((g2[e], ("dy_t", "h_t")), (g13[e], ("dgu_t", "x_t"))):
            aq, as_ = ops[a][0][:, sl], ops[a][1][ss].T
            bq, bs = ops[b_][0][:, sl], ops[b_][1][ss].T
            exact = ob.gemm_rows_scaled(aq, as_, bq, bs)
            err = np.abs(got - exact)
            bound = wgrad_bound(aq, as_, bq, bs, exact)
            assert np.all(err <= bound), (e, a, float((err / np.maximum(bound, 1e-300)).max()))
            worst["dw"] = max(worst["dw"], float(np.linalg.norm(got - exact) / np.linalg.norm(exact)))
        col += n
    # token gradient: the float64 sum of the GPU's rows, rounded once
    rdx_tok = ob.token_grad(gdx_rows, pos, T, k)
    assert np.array_equal(to_np(dx), rdx_tok) or rel_l2_rows(to_np(dx), rdx_tok).max() <= 2.0 ** -7
    # end to end against the oracle from the forward state only (information)
    dx_rows = np.zeros((T * k + T, d))
    xq, xs = to_np(L.xq), to_np(L.xs)
    for e in range(E + 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            w13q, w13s, w2q, w2s = oe(e)
            dx_rows[lo:hi] = ob.expert_backward((xq[rt[lo:hi]], xs[rt[lo:hi]]), (gu[lo:hi], gus[lo:hi]),
                                                rdy[lo:hi], (w13q, w13s), (w2q, w2s))["dx"]
    e2e = np.linalg.norm(to_np(dx) - ob.token_grad(dx_rows, pos, T, k)) / np.linalg.norm(ob.token_grad(dx_rows, pos, T, k))
    log(f"  relative L2 max: dH rows {worst['dh']:.2e}, dX rows {worst['dx_rows']:.2e}, "
        f"dW {worst['dw']:.2e}; token dX end to end {e2e:.2e}")
    assert e2e <= TOL


def _padded_blocks(off):
    nb = -(-np.diff(np.asarray(off, np.int64)) // 128)
    return np.concatenate([[0], np.cumsum(nb)]).astype(np.int64)


def test_v3_backward_sampled():
    """The backward at the full 16k-token V3 shape, in the configuration the
    bench times, checked on samples the oracle computes one by one: the rows of
    two tokens through every row-local stage, one 128-row block of a routed
    and of the shared expert through the regrouping and the transposed SwiGLU
    outputs, and 32 x 32 weight-gradient elements of both experts."""
    cfg = configs.get("uniform_16k")
    T, k, E, d, f = cfg.T, cfg.k, cfg.E, cfg.d, cfg.f
    log(f"layer backward {cfg.name}: T={T} d={d} E={E} f={f}")
    x, wg, b = inputs.host_inputs(cfg)
    W = device_weights(cfg)
    Wt = W.transposed()
    L = moe.MoELayer(T, d, E, cfg.G, cfg.M, k, f, cfg.route_scale)
    L.forward(x.to(DEV), wg.to(DEV), b.to(DEV), W, train=True)
    gen = torch.Generator(device=DEV).manual_seed(7)
    dout = torch.randn(T, d, generator=gen, device=DEV).to(torch.bfloat16)
    dx, dw13, dw2, dgate = L.backward(dout, Wt)
    torch.cuda.synchronize()
    log("  forward + backward done on the GPU")
    # the backward again on the same cache gives the same bytes (the gradients
    # are written, never accumulated with atomics)
    first = [t.clone() for t in (dx, dw13, dw2, dgate)]
    again = L.backward(dout, Wt)
    torch.cuda.synchronize()
    for nm, a, c in zip(("dx", "dw13", "dw2", "dgate"), first, again):
        assert torch.equal(a, c), nm
    del first
    log("  second backward identical")
    pos, off = to_np(L.pos), to_np(L.offsets)
    rt = to_np(L.row_token)
    rng = np.random.default_rng(8)
    tok = np.sort(rng.choice(T, 2, replace=False))
    ns = len(tok)
    rows = np.concatenate([pos[tok].reshape(-1), T * k + tok])
    R = torch.from_numpy(rows.astype(np.int64)).to(DEV)
    pos_l = np.arange(ns * k).reshape(ns, k)
    dout_s = dout[torch.from_numpy(tok).to(DEV)].float().cpu().numpy()
    # combine backward: dY rows bit-exact, gate gradients within the FP32 sum's bound
    ys = to_np(L.y[R])
    rdy, rdw = ob.combine_backward(dout_s, ys, to_np(L.w)[tok], pos_l, ns, k)
    assert np.array_equal(to_np(L.dy[R]), rdy)
    # FP32 dot products of length d: at most ~40 sequential roundings per element
    dw_bound = 40 * 2.0 ** -24 * np.einsum("td,tkd->tk", np.abs(dout_s), np.abs(ys[pos_l]))
    assert np.all(np.abs(to_np(dgate)[tok] - rdw) <= dw_bound)
    dyq, dys = oq.quant_1x128(rdy, "pow2")
    assert np.array_equal(to_np(L.dyq[R]), dyq) and np.array_equal(to_np(L.dys[R]), dys)
    # row-local stages on the GPU's own inputs to each stage
    experts = np.searchsorted(off, rows, side="right") - 1
    oe = OracleExperts(cfg)
    oe.prepare(sorted(set(experts.tolist())))
    log(f"  oracle: {len(set(experts.tolist()))} experts for tokens {tok.tolist()}")
    gdh, gdgu, gdgus, gdx = (to_np(getattr(L, n)[R]) for n in ("dh", "dgu", "dgus", "dx_rows"))
    gu, gus = to_np(L.gu[R]), to_np(L.gus[R])
    worst_dh = worst_dx = 0.0
    n_flip = 0
    for i, e in enumerate(experts):
        w13q, w13s, w2q, w2s = oe(int(e))
        r = slice(i, i + 1)
        rdh = fp8.bf16_round(fp8.f32(olayer.blocked_gemm(dyq[r], dys[r], w2q.T.copy(), w2s.T.copy())))
        gv = fp8.f32(oq.dequant_1x128(gu[r], gus[r]))
        _, dg, du = (fp8.f32(v) for v in ob.swiglu_backward(gv[:, :f], gv[:, f:], gdh[r]))
        rq, rs = oq.quant_1x128(np.concatenate([dg, du], axis=1), "pow2")
        n_flip += _close_codes(gdgu[r], rq, "dgu")
        assert np.array_equal(gdgus[r], rs)
        rdx = fp8.bf16_round(fp8.f32(olayer.blocked_gemm(gdgu[r], gdgus[r], w13q.T.copy(), w13s.T.copy())))
        worst_dh = max(worst_dh, float(rel_l2_rows(gdh[r], rdh).max()))
        worst_dx = max(worst_dx, float(rel_l2_rows(gdx[r], rdx).max()))
    assert worst_dh <= TOL and worst_dx <= TOL, (worst_dh, worst_dx)
    # token gradient: the float64 sum of the GPU's rows, rounded once
    rdx_tok = ob.token_grad(gdx, pos_l, ns, k)
    got_tok = to_np(dx[torch.from_numpy(tok).to(DEV)])
    assert np.array_equal(got_tok, rdx_tok) or rel_l2_rows(got_tok, rdx_tok).max() <= 2.0 ** -7
    # one 128-row block of a routed expert (its last, usually partial) and of the
    # shared expert: regrouped dY and X, transposed h and [dG, dU]
    pb = _padded_blocks(off)
    routed = int(rng.choice(np.nonzero(np.diff(off[:E + 1]))[0]))
    blocks = [(routed, int(pb[routed + 1] - pb[routed] - 1)), (E, int(rng.integers(0, pb[E + 1] - pb[E])))]
    xq, xs = L.xq, L.xs
    for e, blk in blocks:
        r0 = int(off[e]) + 128 * blk
        r1 = min(r0 + 128, int(off[e + 1]))
        c = int(pb[e]) + blk
        cols = slice(128 * c, 128 * c + 128)
        src = torch.from_numpy(rt[r0:r1].astype(np.int64)).to(DEV)
        xv = fp8.f32(oq.dequant_1x128(to_np(xq[src]), to_np(xs[src])))
        gb = to_np(L.gu[r0:r1]), to_np(L.gus[r0:r1])
        gv = fp8.f32(oq.dequant_1x128(*gb))
        h, dg, du = (fp8.f32(v) for v in ob.swiglu_backward(gv[:, :f], gv[:, f:], to_np(L.dh[r0:r1])))
        for name, vals, exact in (("dy_t", to_np(L.dy[r0:r1]), True), ("x_t", xv, True),
                                  ("h_t", h, False), ("dgu_t", np.concatenate([dg, du], axis=1), False)):
            q, s_ = ob.quant_128x1(vals)
            gq = to_np(getattr(L, name)[:, cols])
            gs = to_np(getattr(L, name + "s")[c])
            if exact:
                assert np.array_equal(gq, q.T), (name, e, blk)
            else:
                n_flip += _close_codes(gq, q.T, name)
            assert np.array_equal(gs, s_[0]), (name, e, blk)
    # weight gradients: 32 x 32 elements of each of the two experts, on the GPU's operands
    worst_dw = 0.0
    for e, _ in blocks:
        sl = slice(128 * int(pb[e]), 128 * int(pb[e + 1]))
        ss = slice(int(pb[e]), int(pb[e + 1]))
        for got_all, (a, b_), (M, N) in ((dw2, ("dy_t", "h_t"), (d, f)), (dw13, ("dgu_t", "x_t"), (2 * f, d))):
            mi = np.sort(rng.choice(M, 32, replace=False))
            ni = np.sort(rng.choice(N, 32, replace=False))
            MI, NI = (torch.from_numpy(v.astype(np.int64)).to(DEV) for v in (mi, ni))
            got = to_np(got_all[e][MI][:, NI])
            aq = to_np(getattr(L, a)[MI][:, sl])
            as_ = to_np(getattr(L, a + "s")[ss][:, MI]).T.copy()
            bq = to_np(getattr(L, b_)[NI][:, sl])
            bs = to_np(getattr(L, b_ + "s")[ss][:, NI]).T.copy()
            exact = ob.gemm_rows_scaled(aq, as_, bq, bs)
            err = np.abs(got - exact)
            bound = wgrad_bound(aq, as_, bq, bs, exact)
            assert np.all(err <= bound), (e, a, float((err / np.maximum(bound, 1e-300)).max()))
            worst_dw = max(worst_dw, float(np.linalg.norm(got - exact) / np.linalg.norm(exact)))
    log(f"  relative L2 max: dH rows {worst_dh:.2e}, dX rows {worst_dx:.2e}, dW samples {worst_dw:.2e}; "
        f"one-step code differences {n_flip}; blocks checked {blocks}")
