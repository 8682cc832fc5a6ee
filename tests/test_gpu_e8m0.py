"""GPU parity of the power-of-two (E8M0) scale variant: the _pow2 quantisers
(bit-exact), the hardware block-scaled grouped GEMMs, and the layer with
``scales="pow2"`` against the oracle run with the same rule.

H's tile scale is itself a power of two chosen from amax: where amax/448 lies
within the MFMA noise of amax from a power of two, the GPU may pick the next
power (either is a correct result of the rule).  The kernel test accepts such
a choice only on tiles where the oracle's noise band straddles the power, and
then checks the codes against the oracle's h quantised with the GPU's scale."""

import numpy as np
import pytest
import torch

import routing_fp8_grouped_amd as moe
from routing_fp8_grouped_amd import configs, inputs
from oracle import fp8, quant as oq, route as oroute, layer as olayer
from oracle.gemm import blocked_gemm
from tests.gpu_util import (rel_l2_rows, DEV, log, to_np, h_noise, h_code_ambiguity, check_h_codes,
                            pow2_scale_choices, rows_within, device_weights, OracleExperts,
                            run_layer, layer_allowance, token_allowance, chain_report,
                            stage_fed_tokens)
from tests.test_gpu_kernels import bf16_tensor, random_gemm_shape, varied_activations

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def _quant_1x128_gpu(x):
    rows, cols = x.shape
    q = torch.empty(rows, cols, dtype=torch.uint8, device=DEV)
    s = torch.empty(rows, cols // 128, dtype=torch.float32, device=DEV)
    moe.fp8_quant_1x128_pow2(x.to(DEV), q, s)
    torch.cuda.synchronize()
    return to_np(q), to_np(s)


@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 384), (256, 7168), (1000, 2048)])
def test_quant_1x128_pow2_bitexact(rows, cols):
    log(f"quant_1x128_pow2 rows={rows} cols={cols}")
    rng = np.random.default_rng(rows * 11 + cols)
    x = varied_activations(rng, rows, cols)
    q, s = _quant_1x128_gpu(x)
    rq, rs = oq.quant_1x128(x.float().numpy(), "pow2")
    assert np.array_equal(s, rs)
    assert np.array_equal(q, rq)


def test_quant_pow2_scale_edges():
    """Tiles whose amax/448 is exactly a power of two, the BF16 value just above
    and below, tiny tiles whose quotient is an FP32 subnormal (scales 2^-126 and
    the 2^-127 floor), the largest BF16 values, and an all-zero tile."""
    amaxes = []
    for j in range(-40, 40, 3):
        a = bf16_tensor(np.array([448.0 * 2.0 ** j], np.float32))
        bits = a.view(torch.int16)
        amaxes += [a, (bits + 1).view(torch.bfloat16), (bits - 1).view(torch.bfloat16)]
    amaxes = torch.cat(amaxes).float().numpy().tolist()
    amaxes += [2.0 ** -118, 2.0 ** -120, 1e-38, 9.2e-41, 3.0e38, 0.0]
    rng = np.random.default_rng(19)
    a = np.zeros((len(amaxes), 128), np.float32)
    for i, m in enumerate(amaxes):
        a[i, 1:] = rng.uniform(-1, 1, 127) * m
        a[i, 0] = -m if i % 2 else m
    x = bf16_tensor(a)
    q, s = _quant_1x128_gpu(x)
    rq, rs = oq.quant_1x128(x.float().numpy(), "pow2")
    assert np.array_equal(s, rs), np.nonzero(s != rs)
    assert np.array_equal(q, rq)
    assert s[-1, 0] == 1.0 and np.all((q[-1] & 0x7F) == 0)        # +0 and -0 only
    assert np.float32(2.0 ** -127) in set(s[:, 0].tolist())


@pytest.mark.parametrize("N,K", [(128, 128), (384, 640), (4096, 7168)])
def test_quant_128x128_pow2_bitexact(N, K):
    log(f"quant_128x128_pow2 N={N} K={K}")
    rng = np.random.default_rng(N * 3 + K)
    w = rng.standard_normal((N, K)).astype(np.float32) / np.sqrt(K)
    amp = np.exp(rng.normal(0, 1.5, (N // 128, K // 128))).astype(np.float32)
    w = (w.reshape(N // 128, 128, K // 128, 128) * amp[:, None, :, None]).reshape(N, K)
    if N * K > 128 * 128:
        w[:128, :128] = 0.0
    x = bf16_tensor(w)
    q = torch.empty(N, K, dtype=torch.uint8, device=DEV)
    s = torch.empty(N // 128, K // 128, dtype=torch.float32, device=DEV)
    moe.fp8_quant_128x128_pow2(x.to(DEV), q, s)
    torch.cuda.synchronize()
    rq, rs = oq.quant_128x128(x.float().numpy(), "pow2")
    assert np.array_equal(to_np(s), rs)
    assert np.array_equal(to_np(q), rq)


def pow2_gemm_case(rng, counts, d, f, a_rows, gather):
    G = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    a = bf16_tensor(rng.standard_normal((a_rows, d)) * np.exp(rng.normal(0, 1, (a_rows, 1))))
    aq, as_ = oq.quant_1x128(a.float().numpy(), "pow2")
    row_src = rng.integers(0, a_rows, rows).astype(np.int32) if gather else None
    experts = []
    for g in range(G):
        w13 = bf16_tensor(rng.standard_normal((2 * f, d)) / np.sqrt(d)).float().numpy()
        w2 = bf16_tensor(rng.standard_normal((d, f)) / np.sqrt(d)).float().numpy()
        experts.append(olayer.quantize_expert(w13, w2, "pow2"))
    return offsets, aq, as_, row_src, experts


def _weights(experts, d, f):
    W = moe.MoEWeights.empty(len(experts), d, f)
    for g, (w13q, w13s, w2q, w2s) in enumerate(experts):
        W.w13q[g].copy_(torch.from_numpy(w13q)); W.w13s[g].copy_(torch.from_numpy(w13s))
        W.w2q[g].copy_(torch.from_numpy(w2q)); W.w2s[g].copy_(torch.from_numpy(w2s))
    return W


@pytest.mark.parametrize("counts,d,f,gather", [
    ([0, 1, 130, 128, 257, 0], 256, 128, True),
    ([3, 0, 200, 64], 384, 256, True),
    ([129, 5], 512, 384, False),
    ([300, 520, 17], 7168, 2048, True),
    # 17 .. 192 rows per group (partial tiles)
    ([17, 192, 0, 100, 193], 640, 256, True),
    ([150, 64, 190], 7168, 2048, True),
    # at most 16 rows per group on average: the weight-streaming kernels
    ([2, 1, 3], 7168, 2048, True),
    ([0, 3, 16, 17, 1, 0], 384, 256, True),
])
def test_gemm_e8m0_parity(counts, d, f, gather):
    run_gemm_e8m0_parity(counts, d, f, gather, sum(counts) * 5 + d + f)


# the seeded random shapes of the FP32-scale GEMM test (ragged, <= 16 rows per
# group, multi-tile groups; d = 128 .. 640, f = 128 .. 384)
@pytest.mark.parametrize("seed", range(6))
def test_gemm_e8m0_parity_random(seed):
    counts, d, f, gather = random_gemm_shape(seed)
    run_gemm_e8m0_parity(counts, d, f, gather, 11 * seed + 3)


def run_gemm_e8m0_parity(counts, d, f, gather, seed):
    log(f"e8m0 grouped gemm counts={counts} d={d} f={f} gather={gather}")
    rng = np.random.default_rng(seed)
    rows = sum(counts)
    a_rows = max(rows, 40) if gather else rows
    offsets, aq, as_, row_src, experts = pow2_gemm_case(rng, counts, d, f, a_rows, gather)
    W = _weights(experts, d, f)
    h = torch.empty(rows, f, dtype=torch.uint8, device=DEV)
    hs = torch.empty(rows, f // 128, dtype=torch.float32, device=DEV)
    y = torch.empty(rows, d, dtype=torch.bfloat16, device=DEV)
    off_d = torch.from_numpy(offsets).to(DEV)
    src_d = None if row_src is None else torch.from_numpy(row_src).to(DEV)
    moe.grouped_gemm_fp8_up_e8m0(torch.from_numpy(aq).to(DEV), torch.from_numpy(as_).to(DEV), src_d,
                                 off_d, W.w13q, W.w13s, h, hs)
    moe.grouped_gemm_fp8_down_e8m0(h, hs, off_d, W.w2q, W.w2s, y)
    torch.cuda.synchronize()
    gh, ghs, gy = to_np(h), to_np(hs), to_np(y)
    src = np.arange(rows) if row_src is None else row_src
    n_amb = n_diff = n_flip = 0
    worst = 0.0
    for g in range(len(counts)):
        lo, hi = offsets[g], offsets[g + 1]
        if hi == lo:
            continue
        w13q, w13s, w2q, w2s = experts[g]
        a_g, s_g = aq[src[lo:hi]], as_[src[lo:hi]]
        _, inter = olayer.expert_ffn(a_g, s_g, *experts[g], "pow2")
        eh = h_noise(a_g, s_g, w13q, w13s, inter["g"], inter["u"], inter["h"])
        s_lo, s_hi = pow2_scale_choices(inter["h"], eh)
        gs = ghs[lo:hi]
        assert np.all((gs == s_lo) | (gs == s_hi)), "H scale outside the rule's valid choices"
        n_flip += int(np.sum(gs != inter["hs"]))
        # reference codes: the oracle's h quantised with the scale the GPU chose
        ref_q = fp8.e4m3_encode((inter["h"].reshape(hi - lo, -1, 128) / gs[:, :, None])
                                .astype(np.float32)).reshape(hi - lo, f)
        amb, sp = h_code_ambiguity(a_g, s_g, w13q, w13s, inter["g"], inter["u"], inter["h"], gs)
        n_diff += check_h_codes(gh[lo:hi], ref_q, amb, sp)
        n_amb += int(amb.sum())
        # second stage on exactly the GPU's h: only its own rounding differs
        ry = fp8.bf16_round(fp8.f32(blocked_gemm(gh[lo:hi], gs, w2q, w2s)))
        ok, err, _ = rows_within(gy[lo:hi], ry, np.zeros_like(ry), TOL)
        assert np.all(ok), (g, err.max())
        worst = max(worst, float(err.max()))
    log(f"  h: {n_flip} tile scales at the other valid power, {n_amb} ambiguous codes, "
        f"{n_diff} differ; y rel-L2 max {worst:.2e}")


def test_tiny_layer_pow2_every_token():
    cfg = configs.get("tiny")
    log(f"pow2 layer {cfg.name}")
    x, wg, b = inputs.host_inputs(cfg)
    bf16 = {}
    W = device_weights(cfg, bf16, pow2=True)
    L = run_layer(cfg, x, wg, b, W, scales="pow2")
    oe = OracleExperts(cfg, bf16, rule="pow2")
    oe.prepare(range(cfg.E + 1))
    ref = olayer.moe_layer(x.float().numpy(), wg.float().numpy(), b.numpy(), oe, cfg.G, cfg.M,
                           cfg.k, cfg.route_scale, rule="pow2")
    r = ref["route"]
    ok = ~r["near_tie"]
    assert np.array_equal(to_np(L.idx)[ok], r["idx"][ok])
    assert np.array_equal(to_np(L.xq), ref["xq"]) and np.array_equal(to_np(L.xs), ref["xs"])
    for e in range(cfg.E + 1):
        assert np.array_equal(to_np(W.w13s[e]), oe(e)[1]) and np.array_equal(to_np(W.w13q[e]), oe(e)[0])
    # stage-fed: the GPU's own routing and H through the oracle's last stages
    sf = stage_fed_tokens(L, np.arange(cfg.T), oe, cfg.E)
    err_sf = rel_l2_rows(to_np(L.out), sf)
    log(f"  stage-fed out rel-L2 max {err_sf.max():.2e} median {np.median(err_sf):.2e}")
    assert np.all(err_sf <= TOL), err_sf.max()
    allow, amb, sp = layer_allowance(ref, oe, cfg.T, cfg.k, cfg.E, rule="pow2")
    okr, err, n_allow = rows_within(to_np(L.out)[ok], ref["out"][ok], allow[ok], TOL)
    log("  " + chain_report(err, rows_within.allow_rel, TOL))
    assert np.all(okr)


@pytest.mark.parametrize("name,T", [("prefill_4k", None), ("decode_64", 17)])
def test_v3_pow2_sampled_tokens(name, T):
    """The power-of-two variant at the V3 shape: 4096 tokens (the tiled GEMMs
    on the hardware block-scaled MFMA, 64 sampled tokens, and a second run
    equal byte for byte) and 17 tokens (the weight-streaming GEMMs with
    power-of-two requantisation, every token)."""
    cfg = configs.get(name) if T is None else configs.with_tokens(configs.get(name), T)
    log(f"pow2 workload {cfg.name}: T={cfg.T}")
    x, wg, b = inputs.host_inputs(cfg)
    W = device_weights(cfg, pow2=True)
    L = run_layer(cfg, x, wg, b, W, scales="pow2")
    if T is None:
        L2 = run_layer(cfg, x, wg, b, W, scales="pow2")
        for nm in ("idx", "w", "xq", "xs", "offsets", "pos", "row_token", "h", "hs", "y", "out"):
            assert torch.equal(getattr(L, nm), getattr(L2, nm)), nm
        del L2
    xn = x.float().numpy()
    r = oroute.route(xn, wg.float().numpy(), b.numpy(), cfg.G, cfg.M, cfg.k, cfg.route_scale)
    ok = ~r["near_tie"]
    assert np.array_equal(to_np(L.idx)[ok], r["idx"][ok])
    rq, rs = oq.quant_1x128(xn, "pow2")
    assert np.array_equal(to_np(L.xq), rq) and np.array_equal(to_np(L.xs), rs)
    sample = (np.nonzero(ok)[0] if cfg.T <= 64 else
              np.sort(np.random.default_rng(4).choice(np.nonzero(ok)[0], 64, replace=False)))
    oe = OracleExperts(cfg, rule="pow2")
    oe.prepare(sorted(set(r["idx"][sample].reshape(-1).tolist()) | {cfg.E}))
    sf = stage_fed_tokens(L, sample, oe, cfg.E)
    err_sf = rel_l2_rows(to_np(L.out)[sample], sf)
    log(f"  stage-fed out rel-L2 over {sample.size} tokens: max {err_sf.max():.2e} "
        f"median {np.median(err_sf):.2e}")
    assert np.all(err_sf <= TOL), err_sf.max()
    out, rs_, extra = olayer.moe_layer_tokens(xn[sample], wg.float().numpy(), b.numpy(), oe, cfg.G,
                                              cfg.M, cfg.k, cfg.route_scale, rule="pow2")
    allow = token_allowance(extra, rs_, oe, cfg.E, rule="pow2")
    okr, err, n_allow = rows_within(to_np(L.out)[sample], out, allow, TOL)
    log(f"  {sample.size} tokens, " + chain_report(err, rows_within.allow_rel, TOL))
    assert np.all(okr)
