"""End-to-end parity of the MoE layer (route -> quant -> permute -> grouped GEMM
-> combine) against the oracle on the five seeded workloads (GPU).

Bar: routing indices, quantised bytes/scales and the permutation bit-exact
(tokens whose k-th and (k+1)-th biased scores differ by < 1e-6 excluded and
counted); layer output within relative L2 <= 5e-3 per row, plus, where an
element of the SwiGLU output h sits within the MFMA's accumulation noise of an
E4M3 rounding midpoint (two valid codes), the bounded effect of a one-step
code change (tests/gpu_util.py; the count of rows that needed it is logged).  The tiny workload
is compared on every token; the V3-shape workloads run in full on the GPU and
are compared on every token for routing and quantisation and on sampled
tokens for the output (each token's output depends on that token alone)."""

import numpy as np
import pytest
import torch

import routing_fp8_grouped_amd as moe
from routing_fp8_grouped_amd import configs, inputs
from oracle import quant as oq, route as oroute, permute as operm, layer as olayer
from tests.gpu_util import (DEV, log, to_np, rel_l2_rows, device_weights, OracleExperts,
                            run_layer, layer_allowance, token_allowance, rows_within,
                            check_h_codes)

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def check_permutation_properties(L, gi, T, k, E):
    """Properties that hold for any correct grouping of the GPU's own idx."""
    off, pos, rt = to_np(L.offsets), to_np(L.pos), to_np(L.row_token)
    counts = np.bincount(gi.reshape(-1), minlength=E)
    assert off[0] == 0 and np.array_equal(np.diff(off[:E + 1]), counts)
    assert off[E] == T * k and off[E + 1] == T * k + T
    assert sorted(pos.reshape(-1).tolist()) == list(range(T * k))
    tok = np.repeat(np.arange(T), k)
    assert np.array_equal(rt[pos.reshape(-1)], tok)
    for e in range(E):
        seg = rt[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)        # token order inside each expert
    assert np.array_equal(rt[T * k:], np.arange(T))


def test_tiny_layer_every_token():
    cfg = configs.get("tiny")
    log(f"layer {cfg.name}")
    x, wg, b = inputs.host_inputs(cfg)
    bf16 = {}
    W = device_weights(cfg, bf16)
    L = run_layer(cfg, x, wg, b, W)
    oe = OracleExperts(cfg, bf16)
    oe.prepare(range(cfg.E + 1))
    ref = olayer.moe_layer(x.float().numpy(), wg.float().numpy(), b.numpy(), oe, cfg.G, cfg.M,
                           cfg.k, cfg.route_scale)
    r = ref["route"]
    ok = ~r["near_tie"]
    gi = to_np(L.idx)
    log(f"  near-tie tokens: {int((~ok).sum())}")
    assert np.array_equal(gi[ok], r["idx"][ok])
    assert np.allclose(to_np(L.w)[ok], r["w"][ok], rtol=2e-6)
    assert np.array_equal(to_np(L.xq), ref["xq"]) and np.array_equal(to_np(L.xs), ref["xs"])
    if np.array_equal(gi, r["idx"]):
        assert np.array_equal(to_np(L.offsets), ref["offsets"])
        assert np.array_equal(to_np(L.pos), ref["pos"])
        assert np.array_equal(to_np(L.row_token)[:cfg.T * cfg.k], ref["row_token"])
    check_permutation_properties(L, gi, cfg.T, cfg.k, cfg.E)
    allow, amb, sp = layer_allowance(ref, oe, cfg.T, cfg.k, cfg.E)
    if np.array_equal(gi, r["idx"]):
        n_diff = check_h_codes(to_np(L.h), ref["hq"], amb, sp)
        log(f"  h codes: {int(amb.sum())} ambiguous, {n_diff} differ")
    okr, err, n_allow = rows_within(to_np(L.out)[ok], ref["out"][ok], allow[ok], TOL)
    log(f"  out rel-L2 max {err.max():.2e} median {np.median(err):.2e}; "
        f"rows above {TOL} within the h-code allowance: {n_allow}")
    assert np.all(okr)
    # the explicit dispatch copy gives the same bytes as the gathering GEMM
    L2 = run_layer(cfg, x, wg, b, W, dispatch=True)
    assert torch.equal(L2.out, L.out) and torch.equal(L2.h, L.h) and torch.equal(L2.y, L.y)
    assert np.array_equal(to_np(L2.xq_perm), operm.gather_rows(to_np(L.xq), to_np(L.row_token)[:cfg.T * cfg.k], cfg.T))


def test_layer_is_deterministic():
    cfg = configs.MoEConfig("det", T=600, d=1024, E=64, G=8, M=4, k=8, f=256, seed=11)
    x, wg, b = inputs.host_inputs(cfg)
    W = device_weights(cfg)
    a = run_layer(cfg, x, wg, b, W)
    c = run_layer(cfg, x, wg, b, W)
    for name in ("idx", "w", "offsets", "pos", "row_token", "h", "hs", "y", "out"):
        assert torch.equal(getattr(a, name), getattr(c, name)), name


@pytest.mark.parametrize("case", ["one_token", "hot_experts", "no_routed_weight", "k_equals_E"])
def test_degenerate_layers(case):
    """One token; a bias that sends every token to the same k experts (all
    other experts empty, full and ragged tiles); route_scale 0 (shared expert
    only); k = E with every group kept (dense)."""
    base = dict(d=256, E=16, G=4, M=2, k=4, f=256, seed=77)
    if case == "one_token":
        cfg = configs.MoEConfig(case, T=1, **base)
    elif case == "no_routed_weight":
        cfg = configs.MoEConfig(case, T=130, route_scale=0.0, **base)
    elif case == "k_equals_E":
        cfg = configs.MoEConfig(case, T=70, d=256, E=8, G=4, M=4, k=8, f=128, seed=5)
    else:
        cfg = configs.MoEConfig(case, T=300, **base)
    log(f"degenerate {case}")
    x, wg, b = inputs.host_inputs(cfg)
    if case == "hot_experts":
        b = torch.full((cfg.E,), -2.0)
        b[[1, 2, 5, 6]] = 2.0           # two experts in each of groups 0 and 1
    bf16 = {}
    W = device_weights(cfg, bf16)
    L = run_layer(cfg, x, wg, b, W)
    oe = OracleExperts(cfg, bf16)
    oe.prepare(range(cfg.E + 1))
    ref = olayer.moe_layer(x.float().numpy(), wg.float().numpy(), b.numpy(), oe, cfg.G, cfg.M,
                           cfg.k, cfg.route_scale)
    ok = ~ref["route"]["near_tie"]
    assert np.array_equal(to_np(L.idx)[ok], ref["route"]["idx"][ok])
    if case == "hot_experts":
        assert np.all(to_np(L.idx) == [1, 2, 5, 6])
        assert np.array_equal(to_np(L.offsets), ref["offsets"])
    allow, _, _ = layer_allowance(ref, oe, cfg.T, cfg.k, cfg.E)
    okr, err, n_allow = rows_within(to_np(L.out)[ok], ref["out"][ok], allow[ok], TOL)
    log(f"  out rel-L2 max {err.max():.2e}; rows above {TOL} within the h-code allowance: {n_allow}")
    assert np.all(okr)


FULL = ["decode_64", "prefill_4k", "uniform_16k", "zipf_16k"]


@pytest.mark.parametrize("name", FULL)
def test_v3_workload(name):
    cfg = configs.get(name)
    log(f"workload {name}: T={cfg.T} d={cfg.d} E={cfg.E} f={cfg.f}")
    x, wg, b = inputs.host_inputs(cfg)
    W = device_weights(cfg)
    log("  weights quantised on the GPU")
    L = run_layer(cfg, x, wg, b, W)
    log("  layer done on the GPU")
    xn = x.float().numpy()
    r = oroute.route(xn, wg.float().numpy(), b.numpy(), cfg.G, cfg.M, cfg.k, cfg.route_scale)
    gi = to_np(L.idx)
    ok = ~r["near_tie"]
    n_tie = int((~ok).sum())
    mism = int(np.sum(np.any(gi != r["idx"], axis=1)))
    log(f"  routing: near-tie tokens {n_tie}, tokens differing {mism}")
    assert np.array_equal(gi[ok], r["idx"][ok])
    assert np.allclose(to_np(L.w)[ok], r["w"][ok], rtol=2e-6)
    counts = np.bincount(gi.reshape(-1), minlength=cfg.E)
    log(f"  expert rows: max {counts.max()} min {counts.min()} distinct {int((counts > 0).sum())}")
    # quantised activations: every row when small, a seeded sample of rows otherwise
    rows = np.arange(cfg.T) if cfg.T <= 4096 else np.sort(
        np.random.default_rng(1).choice(cfg.T, 2048, replace=False))
    rq, rs = oq.quant_1x128(xn[rows])
    assert np.array_equal(to_np(L.xq)[rows], rq) and np.array_equal(to_np(L.xs)[rows], rs)
    # permutation: bit-exact against the oracle's when the selections agree
    check_permutation_properties(L, gi, cfg.T, cfg.k, cfg.E)
    if mism == 0:
        ro, rp, rt = operm.permute(r["idx"], cfg.E)
        assert np.array_equal(to_np(L.offsets), ro)
        assert np.array_equal(to_np(L.pos), rp)
        assert np.array_equal(to_np(L.row_token)[:cfg.T * cfg.k], rt)
    # layer output on sampled tokens (not near ties), evaluated by the oracle alone
    n_s = 3 if cfg.T > 64 else 4
    cand = np.nonzero(ok)[0]
    sample = np.sort(np.random.default_rng(2).choice(cand, n_s, replace=False))
    oe = OracleExperts(cfg)
    need = sorted(set(r["idx"][sample].reshape(-1).tolist()) | {cfg.E})
    log(f"  oracle: {len(need)} experts for tokens {sample.tolist()}")
    oe.prepare(need)
    out, rs_, extra = olayer.moe_layer_tokens(xn[sample], wg.float().numpy(), b.numpy(), oe, cfg.G,
                                              cfg.M, cfg.k, cfg.route_scale)
    allow = token_allowance(extra, rs_, oe, cfg.E)
    okr, err, n_allow = rows_within(to_np(L.out)[sample], out, allow, TOL)
    log(f"  out rel-L2 on sampled tokens: {np.array2string(err, precision=2)}; "
        f"above {TOL} within the h-code allowance: {n_allow}")
    assert np.all(okr)
