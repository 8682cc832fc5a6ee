"""Stage parity of each HIP kernel against the oracle, element by element, on the
same seeded inputs (GPU).  Integer and byte outputs must match bit for bit;
floating-point outputs within the bounds stated in each test."""

import numpy as np
import pytest
import torch

import routing_fp8_grouped_amd as moe
from oracle import fp8, quant as oq, route as oroute, permute as operm, layer as olayer
from tests.gpu_util import (DEV, log, to_np, rel_l2_rows, h_code_ambiguity, check_h_codes,
                            y_allowance, rows_within)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def bf16_tensor(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)


def varied_activations(rng, rows, cols):
    """N(0,1) rows with log-normal per-tile amplitudes, some all-zero tiles,
    some outliers and some tiny tiles (subnormal E4M3 codes)."""
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    amp = np.exp(rng.normal(0, 2, (rows, cols // 128))).astype(np.float32)
    a = (a.reshape(rows, -1, 128) * amp[:, :, None]).reshape(rows, cols)
    if rows * cols >= 1024:
        flat = a.reshape(-1)
        flat[rng.choice(flat.size, max(1, flat.size // 500), replace=False)] *= 300
        a.reshape(rows, -1, 128)[rng.random((rows, cols // 128)) < 0.03] = 0.0
    return bf16_tensor(a)


@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 384), (256, 7168), (1000, 2048)])
def test_quant_1x128_bitexact(rows, cols):
    log(f"quant_1x128 rows={rows} cols={cols}")
    rng = np.random.default_rng(rows * 7 + cols)
    x = varied_activations(rng, rows, cols)
    q = torch.empty(rows, cols, dtype=torch.uint8, device=DEV)
    s = torch.empty(rows, cols // 128, dtype=torch.float32, device=DEV)
    moe.fp8_quant_1x128(x.to(DEV), q, s)
    torch.cuda.synchronize()
    rq, rs = oq.quant_1x128(x.float().numpy())
    assert np.array_equal(to_np(s), rs)
    assert np.array_equal(to_np(q), rq)


def test_quant_conversion_grid():
    """Tiles whose amax is 448 have scale exactly 1, so every other entry is
    converted as is: all E4M3 values, all midpoints between neighbouring codes
    (round-to-nearest-even ties) and their BF16 neighbours, both signs, zeros."""
    vals = np.unique(np.abs(fp8.e4m3_decode(np.arange(256, dtype=np.uint8))))
    vals = vals[np.isfinite(vals)]
    mids = (vals[:-1] + vals[1:]) / 2
    b = bf16_tensor(mids).float().numpy()
    up = torch.from_numpy(b).to(torch.bfloat16).view(torch.int16) + 1
    dn = torch.from_numpy(b).to(torch.bfloat16).view(torch.int16) - 1
    pts = np.concatenate([vals, mids, up.view(torch.bfloat16).float().numpy(),
                          dn.view(torch.bfloat16).float().numpy(), [0.0, -0.0, 1e-6, 460.0]])
    pts = np.concatenate([pts, -pts]).astype(np.float32)
    pts = bf16_tensor(pts).float().numpy()
    pts = np.clip(pts, -448, 448)
    n_per = 127
    rows = -(-pts.size // n_per)
    body = np.zeros(rows * n_per, np.float32)
    body[:pts.size] = pts
    a = np.zeros((rows, 128), np.float32)
    a[:, 0] = 448.0
    a[:, 1:] = body.reshape(rows, n_per)
    x = bf16_tensor(a)
    q = torch.empty(rows, 128, dtype=torch.uint8, device=DEV)
    s = torch.empty(rows, 1, dtype=torch.float32, device=DEV)
    moe.fp8_quant_1x128(x.to(DEV), q, s)
    torch.cuda.synchronize()
    rq, rs = oq.quant_1x128(x.float().numpy())
    assert np.all(rs == 1.0) and np.all(to_np(s) == 1.0)
    assert np.array_equal(to_np(q), rq)


@pytest.mark.parametrize("N,K", [(128, 128), (384, 640), (4096, 7168)])
def test_quant_128x128_bitexact(N, K):
    log(f"quant_128x128 N={N} K={K}")
    rng = np.random.default_rng(N + K)
    w = rng.standard_normal((N, K)).astype(np.float32) / np.sqrt(K)
    amp = np.exp(rng.normal(0, 1.5, (N // 128, K // 128))).astype(np.float32)
    w = (w.reshape(N // 128, 128, K // 128, 128) * amp[:, None, :, None]).reshape(N, K)
    if N * K > 128 * 128:
        w[:128, :128] = 0.0
    x = bf16_tensor(w)
    q = torch.empty(N, K, dtype=torch.uint8, device=DEV)
    s = torch.empty(N // 128, K // 128, dtype=torch.float32, device=DEV)
    moe.fp8_quant_128x128(x.to(DEV), q, s)
    torch.cuda.synchronize()
    rq, rs = oq.quant_128x128(x.float().numpy())
    assert np.array_equal(to_np(s), rs)
    assert np.array_equal(to_np(q), rq)


ROUTE_CASES = [
    # T, d, E, G, M, k, route_scale
    (256, 256, 16, 4, 2, 4, 2.5),
    (300, 7168, 256, 8, 4, 8, 2.5),
    (64, 7168, 256, 8, 4, 8, 2.5),
    (100, 256, 8, 4, 2, 4, 1.0),
    (100, 384, 12, 3, 1, 2, 1.0),
    (130, 512, 64, 8, 4, 8, 2.5),
    (70, 256, 256, 16, 4, 16, 2.5),
    (65, 256, 32, 32, 8, 8, 1.0),
    (1, 128, 4, 1, 1, 4, 2.5),
    (50, 256, 64, 2, 1, 16, 2.5),      # group score over k/M = 16 experts
    (90, 256, 256, 8, 2, 6, 1.0),      # 8 groups of 32, k < 8
]


@pytest.mark.parametrize("T,d,E,G,M,k,rho", ROUTE_CASES)
def test_route_parity(T, d, E, G, M, k, rho):
    log(f"route T={T} d={d} E={E} G={G} M={M} k={k}")
    rng = np.random.default_rng(T * 1000 + E + d)
    x = bf16_tensor(rng.standard_normal((T, d)))
    wg = bf16_tensor(rng.standard_normal((E, d)) / np.sqrt(d))
    b = torch.from_numpy(rng.uniform(-0.05, 0.05, E).astype(np.float32))
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    moe.moe_route(x.to(DEV), wg.to(DEV), b.to(DEV), G, M, k, rho, idx, w)
    torch.cuda.synchronize()
    r = oroute.route(x.float().numpy(), wg.float().numpy(), b.numpy(), G, M, k, rho)
    gi, gw = to_np(idx), to_np(w)
    ok = ~r["near_tie"]
    log(f"  near-tie tokens excluded: {int((~ok).sum())} of {T}")
    assert np.array_equal(gi[ok], r["idx"][ok])
    assert np.allclose(gw[ok], r["w"][ok], rtol=2e-6, atol=1e-7)
    # every token (near ties included) still satisfies the routing invariants
    per = E // G
    for t in range(T):
        assert len(set(gi[t])) == k and list(gi[t]) == sorted(gi[t])
        assert len(set(gi[t] // per)) <= M
    assert np.allclose(gw.astype(np.float64).sum(1), rho, rtol=1e-5)


@pytest.mark.parametrize("T,d,E,G,M,k", [
    (1, 7168, 256, 8, 4, 8), (64, 7168, 256, 8, 4, 8), (100, 7168, 256, 8, 4, 8),
    (1024, 7168, 256, 8, 4, 8), (1025, 7168, 256, 8, 4, 8), (4096, 7168, 256, 8, 4, 8),
    (8192, 512, 256, 8, 4, 8), (8193, 256, 64, 8, 4, 8), (300, 384, 12, 3, 1, 2),
    (70, 256, 256, 16, 4, 16), (65, 128, 40, 8, 2, 4)])
def test_route_ws_matches_single_kernel(T, d, E, G, M, k):
    """The two-kernel router (workspace) returns moe_route's result bit for bit:
    the same logit arithmetic, the same selection code (with a bias, and
    without one on odd T)."""
    log(f"route_ws T={T} d={d} E={E} G={G} M={M} k={k}")
    rng = np.random.default_rng(T + 7 * E + d)
    x = bf16_tensor(rng.standard_normal((T, d))).to(DEV)
    wg = bf16_tensor(rng.standard_normal((E, d)) / np.sqrt(d)).to(DEV)
    b = torch.from_numpy(rng.uniform(-0.05, 0.05, E).astype(np.float32)).to(DEV) if T % 2 == 0 else None
    out = []
    for ws in (None, torch.empty(max(16, moe.moe_route_workspace_bytes(T, E)), dtype=torch.uint8, device=DEV)):
        idx = torch.full((T, k), -1, dtype=torch.int32, device=DEV)
        w = torch.full((T, k), -1.0, dtype=torch.float32, device=DEV)
        moe.moe_route(x, wg, b, G, M, k, 2.5, idx, w, workspace=ws)
        out.append((idx, w))
    torch.cuda.synchronize()
    assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1])


def test_route_bias_only_moves_selection():
    """A bias that pushes every unselected expert down keeps the selection and
    leaves the gates bit-identical (the bias never enters the weights)."""
    rng = np.random.default_rng(3)
    T, d, E, G, M, k = 64, 256, 64, 8, 4, 8
    x = bf16_tensor(rng.standard_normal((T, d))).to(DEV)
    wg = bf16_tensor(rng.standard_normal((E, d)) / 16).to(DEV)
    idx0 = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w0 = torch.empty(T, k, dtype=torch.float32, device=DEV)
    moe.moe_route(x, wg, None, G, M, k, 2.5, idx0, w0)
    for t in range(0, T, 9):
        bias = torch.full((E,), -1.0, device=DEV)
        bias[idx0[t].long()] = 0.5
        idx1 = torch.empty(1, k, dtype=torch.int32, device=DEV)
        w1 = torch.empty(1, k, dtype=torch.float32, device=DEV)
        moe.moe_route(x[t:t + 1].contiguous(), wg, bias, G, M, k, 2.5, idx1, w1)
        assert torch.equal(idx1[0], idx0[t]) and torch.equal(w1[0], w0[t])


def random_idx(rng, T, E, k, skew=False):
    if skew:
        hot = rng.choice(E, min(E, k + 3), replace=False)
        return np.stack([np.sort(rng.choice(hot, k, replace=False)) for _ in range(T)]).astype(np.int32)
    return np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,k,E,skew,d", [(1, 4, 16, False, 256), (255, 8, 256, False, 256),
                                           (256, 8, 256, False, 128), (1000, 8, 256, True, 256),
                                           (4097, 6, 64, False, 128), (37, 1, 1, False, 128)])
def test_permute_parity(T, k, E, skew, d):
    log(f"permute T={T} k={k} E={E} skew={skew}")
    rng = np.random.default_rng(T + k + E)
    idx = random_idx(rng, T, E, k, skew)
    xq = torch.from_numpy(rng.integers(0, 256, (T, d), dtype=np.uint8))
    xs = torch.from_numpy(rng.random((T, d // 128)).astype(np.float32))
    rows = T * k + T
    offsets = torch.empty(E + 2, dtype=torch.int32, device=DEV)
    pos = torch.empty(T, k, dtype=torch.int32, device=DEV)
    row_token = torch.empty(rows, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(16, moe.moe_permute_workspace_bytes(T, k, E)), dtype=torch.uint8, device=DEV)
    xq_perm = torch.empty(rows, d, dtype=torch.uint8, device=DEV)
    xs_perm = torch.empty(rows, d // 128, dtype=torch.float32, device=DEV)
    moe.moe_permute(torch.from_numpy(idx).to(DEV), E, offsets, pos, row_token, ws,
                    xq.to(DEV), xs.to(DEV), xq_perm, xs_perm)
    torch.cuda.synchronize()
    ro, rp, rt = operm.permute(idx, E)
    assert np.array_equal(to_np(offsets), ro)
    assert np.array_equal(to_np(pos), rp)
    assert np.array_equal(to_np(row_token)[:T * k], rt)
    assert np.array_equal(to_np(row_token)[T * k:], np.arange(T))
    assert np.array_equal(to_np(xq_perm), operm.gather_rows(xq.numpy(), rt, T))
    assert np.array_equal(to_np(xs_perm), operm.gather_rows(xs.numpy(), rt, T))


def gemm_case(rng, counts, d, f, a_rows, gather):
    """Quantised activations, group offsets, source rows and per-group weights,
    all produced by the oracle from seeded BF16 data."""
    G = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    a = rng.standard_normal((a_rows, d)).astype(np.float32)
    a = bf16_tensor(a).float().numpy()
    aq, as_ = oq.quant_1x128(a)
    row_src = rng.integers(0, a_rows, rows).astype(np.int32) if gather else None
    experts = []
    for g in range(G):
        w13 = bf16_tensor(rng.standard_normal((2 * f, d)) / np.sqrt(d)).float().numpy()
        w2 = bf16_tensor(rng.standard_normal((d, f)) / np.sqrt(d)).float().numpy()
        experts.append(olayer.quantize_expert(w13, w2))
    return offsets, aq, as_, row_src, experts


@pytest.mark.parametrize("counts,d,f,gather", [
    ([0, 1, 130, 128, 257, 0], 256, 128, True),
    ([3, 0, 200, 64], 384, 256, True),
    ([129, 5], 512, 384, False),
    ([300, 520, 17], 7168, 2048, True),     # the V3 shape on the tiled kernel
    # 17 .. 192 rows per group (prefill sizes): partial 256-row tiles whose
    # waves past the group's end skip the multiply, an empty group, a partial
    # 256-row block of W2 at d = 640, K = 7168 with 56 promotions
    ([17, 192, 0, 100, 193], 640, 256, True),
    ([150, 64, 190], 7168, 2048, True),
    ([40, 33], 128, 384, False),
    # at most 16 rows per group on average: the weight-streaming kernels
    # (chunks of 16 rows, a partial 256-row block of W2 at d = 384)
    ([2, 1, 3], 7168, 2048, True),
    ([0, 3, 16, 17, 1, 0], 384, 256, True),
    ([5, 0, 2], 256, 128, False),
])
def test_gemm_parity(counts, d, f, gather):
    run_gemm_parity(counts, d, f, gather, sum(counts) + d + f)


def random_gemm_shape(seed):
    """Seeded group sizes and widths: seed % 3 picks ragged groups on the tiled
    kernel, at most 16 rows per group (the weight-streaming kernels), or
    groups of several tiles (the balanced row split); d = 640 leaves a
    half-empty last column tile in the second GEMM."""
    r = np.random.default_rng(1000 + seed)
    G = int(r.integers(1, 10))
    d = (128, 640, 384, 256, 512)[seed % 5]   # d = 128: a single K block in the first GEMM
    f = (384, 128, 256)[(seed // 3) % 3]
    if seed % 3 == 0:
        counts = r.integers(0, 300, G)
    elif seed % 3 == 1:
        counts = r.integers(0, 17, G)
    else:
        counts = np.where(r.random(G) < 0.3, 0, r.integers(200, 600, G))
    counts = [int(c) for c in counts]
    if sum(counts) == 0:
        counts[0] = 1
    return counts, d, f, bool(r.integers(0, 2))


@pytest.mark.parametrize("seed", range(9))
def test_gemm_parity_random(seed):
    counts, d, f, gather = random_gemm_shape(seed)
    run_gemm_parity(counts, d, f, gather, 7 * seed + 1)


@pytest.mark.parametrize("hi_rows,gather", [(41, True), (13, False)])
def test_gemm_parity_max_groups(hi_rows, gather):
    """The largest group count the GEMM entry points accept (1024): the tile
    list's prefix over 16 chunks of 64 groups, about a fifth of the groups
    empty.  Up to 40 rows per group (about 20 on average) takes the tiled
    kernel, up to 12 the weight-streaming one."""
    r = np.random.default_rng(4000 + hi_rows)
    counts = [int(c) if r.random() > 0.2 else 0 for c in r.integers(1, hi_rows, 1024)]
    run_gemm_parity(counts, 128, 128, gather, hi_rows)


def run_gemm_parity(counts, d, f, gather, seed):
    log(f"grouped gemm counts={counts} d={d} f={f} gather={gather}")
    rng = np.random.default_rng(seed)
    rows = sum(counts)
    a_rows = max(rows, 40) if gather else rows
    offsets, aq, as_, row_src, experts = gemm_case(rng, counts, d, f, a_rows, gather)
    G = len(counts)
    W = moe.MoEWeights.empty(G, d, f)
    for g, (w13q, w13s, w2q, w2s) in enumerate(experts):
        W.w13q[g].copy_(torch.from_numpy(w13q)); W.w13s[g].copy_(torch.from_numpy(w13s))
        W.w2q[g].copy_(torch.from_numpy(w2q)); W.w2s[g].copy_(torch.from_numpy(w2s))
    h = torch.empty(rows, f, dtype=torch.uint8, device=DEV)
    hs = torch.empty(rows, f // 128, dtype=torch.float32, device=DEV)
    y = torch.empty(rows, d, dtype=torch.bfloat16, device=DEV)
    moe.grouped_gemm_fp8_swiglu(torch.from_numpy(aq).to(DEV), torch.from_numpy(as_).to(DEV),
                                None if row_src is None else torch.from_numpy(row_src).to(DEV),
                                torch.from_numpy(offsets).to(DEV), W.w13q, W.w13s, W.w2q, W.w2s,
                                h, hs, y)
    torch.cuda.synchronize()
    gh, ghs, gy = to_np(h), to_np(hs), to_np(y)
    src = np.arange(rows) if row_src is None else row_src
    n_amb = n_diff = n_allow = 0
    worst = 0.0
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi == lo:
            continue
        w13q, w13s, w2q, w2s = experts[g]
        ry, inter = olayer.expert_ffn(aq[src[lo:hi]], as_[src[lo:hi]], *experts[g])
        amb, sp = h_code_ambiguity(aq[src[lo:hi]], as_[src[lo:hi]], w13q, w13s, inter["g"],
                                   inter["u"], inter["h"], inter["hs"])
        # scales: amax/448 of h, within the same noise (a few 1e-5 relative)
        assert np.allclose(ghs[lo:hi], inter["hs"], rtol=2e-4)
        n_diff += check_h_codes(gh[lo:hi], inter["hq"], amb, sp)
        n_amb += int(amb.sum())
        ok, err, na = rows_within(gy[lo:hi], ry, y_allowance(amb, sp, inter["hs"], w2q, w2s), 5e-3)
        assert np.all(ok), (g, err.max())
        n_allow += na
        worst = max(worst, float(err.max()))
    log(f"  h codes: {n_amb} ambiguous, {n_diff} differ; y rel-L2 max {worst:.2e}, "
        f"rows above 5e-3 (within the ambiguity allowance): {n_allow}/{rows}")


# k = 8 takes the unrolled kernel, other k the generic one; a row's 16-byte
# chunks go to 224 threads x 4 at d = 7168 and 144 x 1 at d = 1152, while
# d = 512 (64 chunks) runs 256 threads
@pytest.mark.parametrize("T,k,E,d,with_residual", [
    (300, 8, 64, 512, False),
    (300, 8, 64, 512, True),
    (70, 8, 256, 7168, False),
    (90, 6, 64, 1152, True),
    (33, 16, 256, 7168, False),
])
def test_combine_parity(T, k, E, d, with_residual):
    log(f"combine T={T} k={k} d={d} (residual: {with_residual})")
    rng = np.random.default_rng(5 + T + k)
    idx = random_idx(rng, T, E, k)
    offsets, pos, rt = operm.permute(idx, E)
    rows = T * k + T
    y = bf16_tensor(rng.standard_normal((rows, d)))
    w = rng.random((T, k)).astype(np.float32)
    w = (2.5 * w / w.sum(1, keepdims=True)).astype(np.float32)
    res = bf16_tensor(rng.standard_normal((T, d)) * 3.0) if with_residual else None
    out = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    moe.moe_combine(y.to(DEV), torch.from_numpy(pos).to(DEV), torch.from_numpy(w).to(DEV), T * k, out,
                    residual=None if res is None else res.to(DEV))
    torch.cuda.synchronize()
    yn = y.float().numpy()
    rn = None if res is None else res.float().numpy()
    ref = olayer.combine(yn[pos.astype(np.int64)], w, yn[T * k:], rn)
    got = to_np(out)
    # FP32 sum in slot order vs the float64 sum: one BF16 step where the two
    # land on different sides of a rounding boundary, plus the FP32 sum's own
    # error where the terms cancel
    diff = np.abs(got.astype(np.float64) - ref)
    terms = np.einsum("tk,tkd->td", np.abs(w), np.abs(yn[pos.astype(np.int64)])) + np.abs(yn[T * k:])
    if rn is not None:
        terms += np.abs(rn)
    assert np.all(diff <= np.abs(ref) * 2.0 ** -7 + 16 * 2.0 ** -24 * terms)
    assert np.mean(got != ref) < 0.01
