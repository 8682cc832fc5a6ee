"""Randomised tier of the dispatch path (GPU): seeded draws of (T, d, E, G, M,
k, route scale) run the router, the permutation and the combine through the
C ABI in sequence, each stage fed with the previous GPU stage's output, and
each compared with the oracle on the same inputs: the selection bit for bit
(tokens at a near tie excluded, with the routing invariants still checked on
them), gates within 2e-6 relative, the permutation bit for bit, the combine
within the bound of test_combine_parity.  The fixed parameter lists of
test_gpu_kernels.py cover chosen shapes; these cover the space between them
(group sizes from 1 to 64 experts, 1 to 16 experts per token, ragged T).

A second sweep runs the whole layer (router, 1x128 quantisation, permutation,
both expert GEMMs, combine) on seeded draws of T in [1, 300], E in {8, 16,
32} with G dividing E, and d, f in {128, 256, 384}: the small draws take the
weight-streaming GEMM, the larger ones the tiled GEMM.  Each is held to the
bar of the tiny layer in test_gpu_layer.py on every token: routing and
quantisation bit for bit outside near ties, the permutation's properties,
the stage-fed output within 5e-3 per row, H codes equal where unambiguous,
and the independent chain within its counted allowance.

Router: "DeepSeek-V3" summary page, section 1 (DeepSeekMoE, node-limited
routing) and section 2 (routing-only bias); dispatch and combine: the book's
chapter 15 "What dispatch must do", chapter 7 "Selecting and combining
experts"; the expert GEMMs: summary page section 6, the book's chapter 16
"Periodic high-precision promotion".
"""

import numpy as np
import pytest
import torch

import routing_fp8_grouped_amd as moe
from routing_fp8_grouped_amd import configs, inputs
from oracle import route as oroute, permute as operm, layer as olayer
from tests.gpu_util import (DEV, log, to_np, rel_l2_rows, device_weights, OracleExperts, run_layer,
                            layer_allowance, rows_within, check_h_codes, chain_report,
                            stage_fed_tokens, random_layer_config)

pytestmark = pytest.mark.gpu
N_CASES = 24
N_LAYERS = 16
TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def bf16_tensor(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def draw_config(seed):
    """A routing configuration the C ABI accepts: E <= 256 in G <= 64 equal
    groups, k = M * n (n <= experts per group, k <= 16)."""
    r = np.random.default_rng(4242 + seed)
    G = int(r.choice([1, 2, 3, 4, 8, 16, 32, 64]))
    per = int(r.integers(1, 256 // G + 1))
    E = G * per
    M = int(r.integers(1, min(G, 16) + 1))
    n_top = int(r.integers(1, min(per, 16 // M) + 1))
    k = M * n_top
    T = int(r.integers(1, 300))
    d = int(r.choice([128, 256, 384, 640]))
    rho = float(r.choice([1.0, 2.5]))
    return r, T, d, E, G, M, k, rho


@pytest.mark.parametrize("seed", range(N_CASES))
def test_dispatch_chain_random(seed):
    r, T, d, E, G, M, k, rho = draw_config(seed)
    log(f"fuzz seed={seed}: T={T} d={d} E={E} G={G} M={M} k={k} rho={rho}")
    x = bf16_tensor(r.standard_normal((T, d)))
    wg = bf16_tensor(r.standard_normal((E, d)) / np.sqrt(d))
    bias = torch.from_numpy(r.uniform(-0.05, 0.05, E).astype(np.float32)) if seed % 3 else None

    # ---- router ----
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    moe.moe_route(x.to(DEV), wg.to(DEV), None if bias is None else bias.to(DEV), G, M, k, rho, idx, w)
    torch.cuda.synchronize()
    ref = oroute.route(x.float().numpy(), wg.float().numpy(), None if bias is None else bias.numpy(),
                       G, M, k, rho)
    gi, gw = to_np(idx), to_np(w)
    ok = ~ref["near_tie"]
    assert np.array_equal(gi[ok], ref["idx"][ok])
    assert np.allclose(gw[ok], ref["w"][ok], rtol=2e-6, atol=1e-7)
    per = E // G
    for t in range(T):
        assert len(set(gi[t].tolist())) == k and np.all(np.diff(gi[t]) > 0)
        assert len(set((gi[t] // per).tolist())) <= M
    assert np.allclose(gw.astype(np.float64).sum(1), rho, rtol=1e-5)

    # ---- permutation of the GPU's selection ----
    rows = T * k + T
    offsets = torch.empty(E + 2, dtype=torch.int32, device=DEV)
    pos = torch.empty(T, k, dtype=torch.int32, device=DEV)
    row_token = torch.empty(rows, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(16, moe.moe_permute_workspace_bytes(T, k, E)), dtype=torch.uint8, device=DEV)
    moe.moe_permute(idx, E, offsets, pos, row_token, ws)
    torch.cuda.synchronize()
    ro, rp, rt = operm.permute(gi, E)
    assert np.array_equal(to_np(offsets), ro)
    assert np.array_equal(to_np(pos), rp)
    assert np.array_equal(to_np(row_token)[:T * k], rt)
    assert np.array_equal(to_np(row_token)[T * k:], np.arange(T))

    # ---- combine of random expert outputs with the GPU's gates ----
    y = bf16_tensor(r.standard_normal((rows, d)))
    out = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    moe.moe_combine(y.to(DEV), pos, w, T * k, out)
    torch.cuda.synchronize()
    yn = y.float().numpy()
    p64 = rp.astype(np.int64)
    want = olayer.combine(yn[p64], gw, yn[T * k:])
    got = to_np(out).astype(np.float64)
    terms = np.einsum("tk,tkd->td", np.abs(gw.astype(np.float64)), np.abs(yn[p64])) + np.abs(yn[T * k:])
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 16 * 2.0 ** -24 * terms)
    log(f"  near-tie tokens: {int((~ok).sum())} of {T}; groups used max "
        f"{max(len(set((gi[t] // per).tolist())) for t in range(T))} of {M}")


def run_random_layer(cfg, rule):
    small = cfg.rows <= 16 * (cfg.E + 1)
    log(f"layer fuzz {cfg.name} ({rule} scales): T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} G={cfg.G} "
        f"M={cfg.M} k={cfg.k} rho={cfg.route_scale} ({'weight-streaming' if small else 'tiled'} GEMM)")
    x, wg, b = inputs.host_inputs(cfg)
    bf16 = {}
    W = device_weights(cfg, bf16, pow2=rule == "pow2")
    L = run_layer(cfg, x, wg, b, W, scales=rule)
    oe = OracleExperts(cfg, bf16, rule=rule)
    oe.prepare(range(cfg.E + 1))
    ref = olayer.moe_layer(x.float().numpy(), wg.float().numpy(), b.numpy(), oe, cfg.G, cfg.M,
                           cfg.k, cfg.route_scale, rule=rule)
    return L, ref, oe


@pytest.mark.parametrize("seed", range(N_LAYERS))
def test_layer_random(seed):
    cfg = random_layer_config(seed)
    L, ref, oe = run_random_layer(cfg, "fp32")
    r = ref["route"]
    ok = ~r["near_tie"]
    gi = to_np(L.idx)
    assert np.array_equal(gi[ok], r["idx"][ok])
    assert np.allclose(to_np(L.w)[ok], r["w"][ok], rtol=2e-6, atol=1e-7)
    assert np.array_equal(to_np(L.xq), ref["xq"]) and np.array_equal(to_np(L.xs), ref["xs"])
    same_route = np.array_equal(gi, r["idx"])
    if same_route:
        assert np.array_equal(to_np(L.offsets), ref["offsets"])
        assert np.array_equal(to_np(L.pos), ref["pos"])
        assert np.array_equal(to_np(L.row_token)[:cfg.T * cfg.k], ref["row_token"])
    # stage-fed: the GPU's routing and H through the oracle's down GEMM and combine
    sf = stage_fed_tokens(L, np.arange(cfg.T), oe, cfg.E)
    err_sf = rel_l2_rows(to_np(L.out), sf)
    assert np.all(err_sf <= TOL), err_sf.max()
    allow, amb, sp = layer_allowance(ref, oe, cfg.T, cfg.k, cfg.E)
    n_diff = check_h_codes(to_np(L.h), ref["hq"], amb, sp) if same_route else -1
    okr, err, _ = rows_within(to_np(L.out)[ok], ref["out"][ok], allow[ok], TOL)
    log(f"  near ties {int((~ok).sum())}; stage-fed rel-L2 max {err_sf.max():.2e}; h codes "
        f"{int(amb.sum())} ambiguous, {n_diff} differ; " + chain_report(err, rows_within.allow_rel, TOL))
    assert np.all(okr)


@pytest.mark.parametrize("seed", range(N_LAYERS, N_LAYERS + 8))
def test_layer_random_pow2(seed):
    """The power-of-two scale variant (hardware block-scaled MFMA) on further
    draws, against the oracle run with the power-of-two rule: routing and
    quantisation bit for bit, the stage-fed output within 5e-3 per row, the
    independent chain within its counted allowance."""
    cfg = random_layer_config(seed)
    L, ref, oe = run_random_layer(cfg, "pow2")
    r = ref["route"]
    ok = ~r["near_tie"]
    assert np.array_equal(to_np(L.idx)[ok], r["idx"][ok])
    assert np.array_equal(to_np(L.xq), ref["xq"]) and np.array_equal(to_np(L.xs), ref["xs"])
    sf = stage_fed_tokens(L, np.arange(cfg.T), oe, cfg.E)
    err_sf = rel_l2_rows(to_np(L.out), sf)
    assert np.all(err_sf <= TOL), err_sf.max()
    allow, _, _ = layer_allowance(ref, oe, cfg.T, cfg.k, cfg.E, rule="pow2")
    okr, err, _ = rows_within(to_np(L.out)[ok], ref["out"][ok], allow[ok], TOL)
    log(f"  near ties {int((~ok).sum())}; stage-fed rel-L2 max {err_sf.max():.2e}; "
        + chain_report(err, rows_within.allow_rel, TOL))
    assert np.all(okr)
