"""End-to-end parity of the MoE layer (route -> quant -> permute -> grouped GEMM
-> combine) against the oracle on the five seeded workloads (GPU).

Bar (spec: routing indices, quantised bytes/scales and the permutation
bit-exact outside 1e-6 near ties; relative L2 <= 5e-3 per output row):

* routing, quantisation and permutation bit-exact, near-tie tokens excluded
  and counted;
* stage-fed layer output: the GPU's own routing and FP8 H rows run through the
  oracle's down GEMM and combine; every row within 5e-3 of the GPU's output,
  with no allowance (near-tie tokens included: the routing is the GPU's);
* H codes against the oracle's from the same inputs: equal, except where the
  oracle's h lies within the MFMA's accumulation noise of an E4M3 rounding
  midpoint (two valid codes; tests/gpu_util.py);
* independent chain (the GPU layer against the oracle's own chain from x):
  rows above 5e-3 form a counted category, like near ties, whose size and
  allowance are printed; each such row must lie within the bounded effect of
  its ambiguous H codes.

The tiny workload is compared on every token; the V3-shape workloads run in
full on the GPU and are compared on every token for routing and
quantisation, and on at least 64 sampled tokens for the output (each token's
output depends on that token alone).
"""

import numpy as np
import pytest
import torch

import routing_fp8_grouped_amd as moe
from routing_fp8_grouped_amd import configs, inputs
from oracle import quant as oq, route as oroute, permute as operm, layer as olayer
from tests.gpu_util import (DEV, log, to_np, rel_l2_rows, device_weights, OracleExperts,
                            run_layer, layer_allowance, token_allowance, rows_within,
                            check_h_codes, chain_report, stage_fed_tokens)

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
    # stage-fed: the GPU's H through the oracle's down GEMM and combine, every token
    sf = stage_fed_tokens(L, np.arange(cfg.T), oe, cfg.E)
    err_sf = rel_l2_rows(to_np(L.out), sf)
    log(f"  stage-fed out rel-L2 max {err_sf.max():.2e} median {np.median(err_sf):.2e} "
        f"over {cfg.T} tokens")
    assert np.all(err_sf <= TOL), err_sf.max()
    allow, amb, sp = layer_allowance(ref, oe, cfg.T, cfg.k, cfg.E)
    if np.array_equal(gi, r["idx"]):
        n_diff = check_h_codes(to_np(L.h), ref["hq"], amb, sp)
        log(f"  h codes: {int(amb.sum())} ambiguous, {n_diff} differ")
    okr, err, n_allow = rows_within(to_np(L.out)[ok], ref["out"][ok], allow[ok], TOL)
    log("  " + chain_report(err, rows_within.allow_rel, TOL))
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
    sf = stage_fed_tokens(L, np.arange(cfg.T), oe, cfg.E)
    err_sf = rel_l2_rows(to_np(L.out), sf)
    log(f"  stage-fed out rel-L2 max {err_sf.max():.2e}")
    assert np.all(err_sf <= TOL), err_sf.max()
    allow, _, _ = layer_allowance(ref, oe, cfg.T, cfg.k, cfg.E)
    okr, err, n_allow = rows_within(to_np(L.out)[ok], ref["out"][ok], allow[ok], TOL)
    log("  " + chain_report(err, rows_within.allow_rel, TOL))
    assert np.all(okr)


@pytest.mark.parametrize("E,G,M,k", [(16, 4, 2, 4), (256, 8, 4, 8)])
def test_zero_input_ties(E, G, M, k):
    """All-zero activations with a zero bias: every logit is 0 and every
    biased score exactly sigmoid(0) = 0.5, so all groups and all experts tie.
    The tie rule (lower group index, then lower expert id) fixes the result:
    groups 0 .. M-1 are kept and the top k over their experts (the count per
    group is free) are the k lowest ids 0 .. k-1, every gate rho/k, codes and
    scales of zero tiles (code 0, scale 1) for X and H, and a zero output.
    E = 16 takes the general selection, E = 256 in 8 groups the V3 one."""
    cfg = configs.MoEConfig(f"zeros{E}", T=70, d=256, E=E, G=G, M=M, k=k, f=128, bias="zero", seed=3)
    log(f"zero input E={E} G={G} M={M} k={k}")
    _, wg, b = inputs.host_inputs(cfg)
    x = torch.zeros(cfg.T, cfg.d, dtype=torch.bfloat16)
    W = device_weights(cfg)
    L = run_layer(cfg, x, wg, b, W)
    assert k <= M * (E // G)
    want = np.arange(k, dtype=np.int32)
    r = oroute.route(x.float().numpy(), wg.float().numpy(), b.numpy(), G, M, k, cfg.route_scale)
    assert np.all(r["idx"] == want)                   # the oracle's tie rule
    assert np.all(to_np(L.idx) == want)
    assert np.all(to_np(L.w) == np.float32(cfg.route_scale / k))
    assert not to_np(L.xq).any() and np.all(to_np(L.xs) == 1.0)
    assert not to_np(L.h).any() and np.all(to_np(L.hs) == 1.0)
    assert not to_np(L.y).view(np.uint16).any()
    assert not to_np(L.out).view(np.uint16).any()


FULL = ["decode_64", "prefill_4k", "uniform_16k", "zipf_16k"]


@pytest.mark.parametrize("T", [1, 17])
def test_v3_few_tokens(T):
    """The V3 shape with 1 and 17 tokens (the weight-streaming GEMMs with
    one row per touched expert, and a ragged 16-row chunk): every token's
    routing, quantisation, and output stage-fed and on the independent chain."""
    cfg = configs.with_tokens(configs.get("decode_64"), T, f"v3_T{T}")
    log(f"workload {cfg.name}")
    x, wg, b = inputs.host_inputs(cfg)
    W = device_weights(cfg)
    L = run_layer(cfg, x, wg, b, W)
    xn = x.float().numpy()
    r = oroute.route(xn, wg.float().numpy(), b.numpy(), cfg.G, cfg.M, cfg.k, cfg.route_scale)
    ok = ~r["near_tie"]
    gi = to_np(L.idx)
    assert np.array_equal(gi[ok], r["idx"][ok])
    rq, rs = oq.quant_1x128(xn)
    assert np.array_equal(to_np(L.xq), rq) and np.array_equal(to_np(L.xs), rs)
    check_permutation_properties(L, gi, cfg.T, cfg.k, cfg.E)
    oe = OracleExperts(cfg)
    oe.prepare(sorted(set(gi.reshape(-1).tolist()) | set(r["idx"].reshape(-1).tolist()) | {cfg.E}))
    sf = stage_fed_tokens(L, np.arange(T), oe, cfg.E)
    err_sf = rel_l2_rows(to_np(L.out), sf)
    assert np.all(err_sf <= TOL), err_sf.max()
    out, rs2, extra = olayer.moe_layer_tokens(xn[ok], wg.float().numpy(), b.numpy(), oe, cfg.G, cfg.M,
                                              cfg.k, cfg.route_scale)
    allow = token_allowance(extra, rs2, oe, cfg.E)
    okr, err, _ = rows_within(to_np(L.out)[ok], out, allow, TOL)
    log(f"  stage-fed max {err_sf.max():.2e}; " + chain_report(err, rows_within.allow_rel, TOL))
    assert np.all(okr)


def test_v3_max_tokens():
    """65536 tokens at the V3 shape: 589824 grouped rows, whose FP8 rows and
    BF16 outputs reach 98% of the 4 GiB the kernels' 32-bit byte offsets
    address (the entry points refuse more).  Routing and quantisation on a
    sample of 2048 tokens, the permutation's properties on all of them, and
    the layer output of 64 tokens (among them the last four, whose rows lie
    at the top of the offset range) stage-fed and on the independent chain."""
    cfg = configs.with_tokens(configs.get("prefill_4k"), 65536, "prefill_64k")
    assert 0.98 < cfg.rows * cfg.d / 2 ** 32 < 1.0
    log(f"workload {cfg.name}: T={cfg.T} rows={cfg.rows}")
    x, wg, b = inputs.host_inputs(cfg)
    W = device_weights(cfg)
    L = run_layer(cfg, x, wg, b, W)
    log("  layer done on the GPU")
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([rng.choice(cfg.T - 4, 2044, replace=False), np.arange(cfg.T - 4, cfg.T)]))
    xn = x[torch.from_numpy(rows)].float().numpy()
    r = oroute.route(xn, wg.float().numpy(), b.numpy(), cfg.G, cfg.M, cfg.k, cfg.route_scale)
    gi_all = to_np(L.idx)
    gi = gi_all[rows]
    ok = ~r["near_tie"]
    assert np.array_equal(gi[ok], r["idx"][ok])
    assert np.allclose(to_np(L.w)[rows][ok], r["w"][ok], rtol=2e-6)
    rq, rs = oq.quant_1x128(xn)
    assert np.array_equal(to_np(L.xq)[rows], rq) and np.array_equal(to_np(L.xs)[rows], rs)
    check_permutation_properties(L, gi_all, cfg.T, cfg.k, cfg.E)
    sample = np.sort(np.concatenate([rng.choice(cfg.T - 4, 60, replace=False), np.arange(cfg.T - 4, cfg.T)]))
    oe = OracleExperts(cfg)
    oe.prepare(sorted(set(gi_all[sample].reshape(-1).tolist()) | {cfg.E}))
    sf = stage_fed_tokens(L, sample, oe, cfg.E)
    err_sf = rel_l2_rows(to_np(L.out)[sample], sf)
    log(f"  stage-fed out rel-L2 over {sample.size} tokens: max {err_sf.max():.2e}")
    assert np.all(err_sf <= TOL), err_sf.max()
    xs_ = x[torch.from_numpy(sample)].float().numpy()
    rr = oroute.route(xs_, wg.float().numpy(), b.numpy(), cfg.G, cfg.M, cfg.k, cfg.route_scale)
    okt = ~rr["near_tie"]
    oe.prepare(sorted(set(rr["idx"][okt].reshape(-1).tolist())))
    out, rs2, extra = olayer.moe_layer_tokens(xs_[okt], wg.float().numpy(), b.numpy(), oe, cfg.G, cfg.M,
                                              cfg.k, cfg.route_scale)
    allow = token_allowance(extra, rs2, oe, cfg.E)
    okr, err, _ = rows_within(to_np(L.out)[sample[okt]], out, allow, TOL)
    log(f"  {int(okt.sum())} tokens, " + chain_report(err, rows_within.allow_rel, TOL))
    assert np.all(okr)


@pytest.mark.parametrize("name", FULL)
def test_v3_workload(name):
    cfg = configs.get(name)
    log(f"workload {name}: T={cfg.T} d={cfg.d} E={cfg.E} f={cfg.f}")
    x, wg, b = inputs.host_inputs(cfg)
    W = device_weights(cfg)
    log("  weights quantised on the GPU")
    L = run_layer(cfg, x, wg, b, W)
    log("  layer done on the GPU")
    # a second run of the same step in a fresh layer gives the same bytes in
    # every buffer (no order-dependent atomics; integer counters only)
    L2 = run_layer(cfg, x, wg, b, W)
    for nm in ("idx", "w", "xq", "xs", "offsets", "pos", "row_token", "h", "hs", "y", "out"):
        assert torch.equal(getattr(L, nm), getattr(L2, nm)), nm
    del L2
    log("  second run identical in every buffer")
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
    # layer output on sampled tokens: every token of a decode batch; otherwise
    # 64 tokens, among them tokens of the most loaded expert and the last token
    if cfg.T <= 64:
        sample = np.arange(cfg.T)
    else:
        rng = np.random.default_rng(2)
        hot = int(np.argmax(counts))
        hot_tokens = np.nonzero(np.any(gi == hot, axis=1))[0]
        pick = set(rng.choice(hot_tokens, min(8, hot_tokens.size), replace=False).tolist())
        pick |= {cfg.T - 1, cfg.T - 2}
        rest = np.setdiff1d(np.arange(cfg.T), sorted(pick))
        pick |= set(rng.choice(rest, 64 - len(pick), replace=False).tolist())
        sample = np.array(sorted(pick))
        log(f"  sample: {sample.size} tokens, {min(8, hot_tokens.size)} of them on expert {hot} "
            f"({counts[hot]} rows)")
    oe = OracleExperts(cfg)
    need = sorted(set(gi[sample].reshape(-1).tolist()) | set(r["idx"][sample].reshape(-1).tolist())
                  | {cfg.E})
    log(f"  oracle: quantising {len(need)} experts")
    oe.prepare(need)
    # stage-fed: the GPU's own routing and H rows through the oracle's last stages
    sf = stage_fed_tokens(L, sample, oe, cfg.E)
    got = to_np(L.out)[sample]
    err_sf = rel_l2_rows(got, sf)
    log(f"  stage-fed out rel-L2 over {sample.size} tokens: max {err_sf.max():.2e} "
        f"median {np.median(err_sf):.2e}")
    assert np.all(err_sf <= TOL), err_sf.max()
    # independent chain on the sampled tokens that are not near ties
    sample_ok = sample[ok[sample]]
    out, rs_, extra = olayer.moe_layer_tokens(xn[sample_ok], wg.float().numpy(), b.numpy(), oe, cfg.G,
                                              cfg.M, cfg.k, cfg.route_scale)
    allow = token_allowance(extra, rs_, oe, cfg.E)
    okr, err, n_allow = rows_within(to_np(L.out)[sample_ok], out, allow, TOL)
    log(f"  {sample_ok.size} tokens, " + chain_report(err, rows_within.allow_rel, TOL))
    assert np.all(okr)
