"""Shared helpers of the GPU parity tests: device inputs, FP8 weights through the
HIP path, and the oracle's view of the same seeded inputs."""

import concurrent.futures as cf
import os
import sys
import time

import numpy as np
import torch

import routing_fp8_grouped_amd as moe
from routing_fp8_grouped_amd import configs, inputs
from oracle import layer as olayer

DEV = "cuda"


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_np(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy()
    return t.numpy()


def rel_l2_rows(a, b):
    """Per-row relative L2 error of a against reference b."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    num = np.linalg.norm(a - b, axis=-1)
    den = np.linalg.norm(b, axis=-1)
    return num / np.maximum(den, 1e-30)


def device_weights(cfg, bf16_cache=None, pow2=False):
    """Generate every expert's BF16 weights on the GPU (seeded per expert) and
    quantise them with the library's 128x128 kernel (the offline step; the
    power-of-two scale rule when ``pow2``)."""
    W = moe.MoEWeights.empty(cfg.E + 1, cfg.d, cfg.f)
    for e in range(cfg.E + 1):
        w13, w2 = inputs.expert_weights(cfg, e, DEV)
        W.quantize_expert(e, w13, w2, pow2=pow2)
        if bf16_cache is not None:
            bf16_cache[e] = (w13, w2)
    torch.cuda.synchronize()
    return W


class OracleExperts:
    """The oracle's quantised weights of the experts it needs, quantised by the
    oracle from the same BF16 weights the GPU quantised (regenerated per expert
    with the same seed, copied to the host)."""

    # quantised experts of the most recently used weight sets, keyed by
    # (expert seed, d, f, rule) and shared by every test in the process, so
    # the V3 workloads, which draw their experts from one seed, quantise each
    # expert once; least recently used sets go first once the sets hold more
    # than CACHE_BYTES (a whole V3 set is about 11 GB)
    _sets = {}
    CACHE_BYTES = 24 << 30

    def __init__(self, cfg, bf16_cache=None, rule="fp32"):
        self.cfg = cfg
        self.bf16 = bf16_cache
        self.rule = rule
        self.key = (cfg.expert_seed, cfg.d, cfg.f, rule)
        sets = OracleExperts._sets
        sets[self.key] = sets.pop(self.key, {})     # most recently used last
        self.cache = sets[self.key]

    def _trim(self):
        sets = OracleExperts._sets
        size = lambda c: sum(a.nbytes for q in c.values() for a in q)
        total = sum(size(c) for c in sets.values())
        for k in list(sets):
            if total <= OracleExperts.CACHE_BYTES:
                break
            if k != self.key:
                total -= size(sets.pop(k))

    def _host(self, e):
        if self.bf16 is not None and e in self.bf16:
            w13, w2 = self.bf16[e]
        else:
            w13, w2 = inputs.expert_weights(self.cfg, e, DEV)
        return w13.float().cpu().numpy(), w2.float().cpu().numpy()

    def prepare(self, ids, workers=None):
        ids = [int(e) for e in ids if int(e) not in self.cache]
        if not ids:
            return
        host = {e: self._host(e) for e in ids}
        workers = workers or min(16, os.cpu_count() or 4)
        with cf.ThreadPoolExecutor(workers) as ex:
            res = ex.map(lambda e: (e, olayer.quantize_expert(*host[e], self.rule)), ids)
            for e, q in res:
                self.cache[e] = q
        self._trim()

    def __call__(self, e):
        if int(e) not in self.cache:
            self.prepare([e])
        return self.cache[int(e)]


def host_inputs(cfg):
    x, wg, b = inputs.host_inputs(cfg)
    return x, wg, b


def random_layer_config(seed):
    """A whole-layer configuration: T in [1, 300], E in {8, 16, 32}, G | E,
    M <= G, k = M * n <= min(M * E / G, 16), d and f in {128, 256, 384}."""
    r = np.random.default_rng(9000 + seed)
    E = int(r.choice([8, 16, 32]))
    G = int(r.choice([g for g in (1, 2, 4, 8) if E % g == 0]))
    per = E // G
    M = int(r.integers(1, G + 1))
    n_top = int(r.integers(1, min(per, 16 // M) + 1))
    T = int(r.integers(1, 301))
    d = int(r.choice([128, 256, 384]))
    f = int(r.choice([128, 256, 384]))
    rho = float(r.choice([1.0, 2.5]))
    return configs.MoEConfig(f"fuzz{seed}", T=T, d=d, E=E, G=G, M=M, k=M * n_top, f=f,
                             route_scale=rho, bias="zero" if seed % 4 == 0 else "uniform",
                             seed=31000 + seed)


def run_layer(cfg, x, wg, b, W, dispatch=False, scales="fp32"):
    L = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.f, cfg.route_scale,
                     dispatch=dispatch, scales=scales)
    L.forward(x.to(DEV), wg.to(DEV), b.to(DEV), W)
    torch.cuda.synchronize()
    return L


# ---- codes of h with two valid values ------------------------------------------
#
# The GPU computes each 128-wide K block's partial sum with one E4M3 MFMA, which
# sums its 128 products with an unbiased error of RMS 1.87e-6 of sum|a*b|, and
# at most 1.75e-5 of it over 3 x 1M dot products of E4M3 codes of Gaussian
# tiles (measured on gfx950 by tests/test_gpu_mfma_noise.py; the tail is heavy:
# 9.6 RMS).  MFMA_BLOCK_MAX takes 1.4 times that maximum.  G and U, and
# so h = SiLU(G) * U, therefore differ from the oracle's exact blocked sums by a
# small, bounded amount, and an element of h that lies that close to an E4M3
# rounding midpoint has two correct codes.  These helpers flag such elements
# from oracle quantities alone and bound what a one-step code change can do to
# the expert output, the way near-tie tokens are handled for routing.

from oracle import fp8 as ofp8, quant as oquant, gemm as ogemm

MFMA_BLOCK_RMS = 1.87e-6   # RMS of (block sum - exact) / sum|a*b|
MFMA_BLOCK_MAX = 2.5e-5    # bound on |block sum - exact| / sum|a*b| (measured max 1.75e-5)


def block_abs_sums(aq_rows, as_rows, wq, ws):
    """Per output element, over the 128-wide K blocks kb of sa*sw*sum|a||w|:
    returns (sqrt of the sum of squares, the largest one)."""
    a = ofp8.e4m3_decode(np.asarray(aq_rows) & 0x7F)
    w = ofp8.e4m3_decode(np.asarray(wq) & 0x7F)
    sa = np.asarray(as_rows, np.float64)
    sw = np.repeat(np.asarray(ws, np.float64), 128, axis=0)
    ss = np.zeros((a.shape[0], w.shape[0]))
    mx = np.zeros_like(ss)
    for kb in range(a.shape[1] // 128):
        blk = slice(kb * 128, (kb + 1) * 128)
        p = (a[:, blk] @ w[:, blk].T) * sa[:, kb:kb + 1] * sw[None, :, kb]
        ss += p * p
        np.maximum(mx, p, out=mx)
    return np.sqrt(ss), mx


# Over 56 K blocks (K = 7168) on E4M3 codes of Gaussian data, measured on
# gfx950 over 131,072 outputs (tests/test_gpu_mfma_noise.py): |error| has RMS
# 1.07 sigma (sigma = the RMS above times the root-sum-square of the blocks'
# s*sum|a*b|) and a maximum of 6.6 sigma, and stays within 1.1 times the
# single-block bound MFMA_BLOCK_MAX * max over blocks of s*sum|a*b|; chaining
# the accumulator through the block-scaled instruction gives the same errors
# as promoting each partial in FP32.  The band takes 8 sigma and twice the
# single-block bound, for a margin over the tails of the ~10^6 outputs of a
# test.
NOISE_SIGMAS = 8.0
NOISE_BLOCKS = 2.0


def gemm_noise(aq_rows, as_rows, wq, ws, acc):
    """Bound on |GPU - exact| of a blocked GEMM output: NOISE_SIGMAS RMS of the
    independent block errors, at least NOISE_BLOCKS times the worst
    single-block error, plus FP32 accumulation."""
    root, mx = block_abs_sums(aq_rows, as_rows, wq, ws)
    kb = np.asarray(aq_rows).shape[1] // 128
    return (np.maximum(NOISE_SIGMAS * MFMA_BLOCK_RMS * root, NOISE_BLOCKS * MFMA_BLOCK_MAX * mx)
            + kb * 2.0 ** -24 * np.abs(acc))


# The MFMA's error per 128-product block also scales with the block's largest
# product (its sum is formed on the exponent of the largest term): over 131,072
# outputs of 56-block chains on uniform codes, Gaussian codes and 128x1 tiles
# of tokens with log-normal amplitudes, |error| / sqrt(sum over blocks of
# (max|a b| * s)^2) had RMS 3.6e-5 .. 6.8e-5 and maximum 2.1e-4 .. 3.4e-4,
# whatever the spread of magnitudes inside a block (where the model above, in
# sum|a b|, does not hold).  The bound takes 8e-4.
MAXPROD_FACTOR = 8e-4


def block_max_products(aq, sa, bq, sb):
    """sqrt over K blocks of (max over the block of |a b| * sa * sb)^2 [M, N],
    both operands scaled per row and block (sa [M, K/128], sb [N, K/128])."""
    a = np.abs(ofp8.e4m3_decode(np.asarray(aq))); b = np.abs(ofp8.e4m3_decode(np.asarray(bq)))
    sa = np.asarray(sa, np.float64); sb = np.asarray(sb, np.float64)
    M, N = a.shape[0], b.shape[0]
    out = np.zeros((M, N))
    for kb in range(a.shape[1] // 128):
        blk = slice(kb * 128, (kb + 1) * 128)
        for m0 in range(0, M, 32):
            mp = np.max(a[m0:m0 + 32, None, blk] * b[None, :, blk], axis=2)
            out[m0:m0 + 32] += (mp * sa[m0:m0 + 32, kb:kb + 1] * sb[None, :, kb]) ** 2
    return np.sqrt(out)


def e4m3_spacing(v):
    """Distance between neighbouring E4M3 values at magnitude |v|."""
    v = np.abs(np.asarray(v, np.float64))
    _, p = np.frexp(np.maximum(v, 1e-300))
    return np.ldexp(1.0, np.maximum(p - 1, -6) - 3)


def h_noise(aq_rows, as_rows, w13q, w13s, g, u, h):
    """Bound on |GPU h - oracle h| per element, from oracle quantities."""
    f = w13q.shape[0] // 2
    g = np.asarray(g, np.float64); u = np.asarray(u, np.float64); h = np.asarray(h, np.float64)
    e = gemm_noise(aq_rows, as_rows, w13q, w13s, np.concatenate([g, u], axis=1))
    eg, eu = e[:, :f], e[:, f:]
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    return np.abs(u) * np.abs(dsilu) * eg + np.abs(g * sig) * eu + SWIGLU_REL * np.abs(h)


# The kernels' SwiGLU is g / (1 + exp(-g)) * u in FP32: exp within one ulp, then
# a correctly rounded sum, quotient and product, so h is within 2.5 ulp (at
# most 2.5 * 2^-23 relative) of fl32(SiLU(g) * u) for the same g and u.  The
# h/scale division of the requantisation is correctly rounded, as in the
# oracle.
SWIGLU_REL = 2.0 ** -21


def pow2_scale_choices(h, eh):
    """Per 1x128 tile of h: the power-of-two scales the GPU may legitimately
    pick (lowest, highest).  They differ where amax/448 lies within the noise
    of amax from a power of two; then either choice is correct."""
    rows = h.shape[0]
    ht = np.abs(np.asarray(h, np.float64)).reshape(rows, -1, 128)
    et = np.asarray(eh, np.float64).reshape(rows, -1, 128)
    lo = np.max(np.maximum(ht - et, 0.0), -1).astype(np.float32)
    hi = np.max(ht + et, -1).astype(np.float32)
    return oquant.scale_from_amax(lo, "pow2"), oquant.scale_from_amax(hi, "pow2")


def code_ambiguity(v, ev, scales):
    """(amb, step) for the 1x128 codes of values v [rows, C] whose GPU values may
    differ by up to ev: amb marks elements whose scaled value lies within the
    noise band of an E4M3 rounding midpoint (the tile scale, amax/448 of
    equally noisy values, moves with them); step bounds how far in scaled
    units a valid code of such an element can be from the oracle's: the GPU
    code rounds some value inside the band, so the two differ by at most twice
    the band plus one grid spacing (near zero the band can cover several
    subnormal steps)."""
    v = np.asarray(v, np.float64); ev = np.asarray(ev, np.float64)
    rows = v.shape[0]
    vt = np.abs(v).reshape(rows, -1, 128)
    et = ev.reshape(rows, -1, 128)
    amax = vt.max(-1)
    scale_rel = (np.max(vt + et, -1) - amax + np.max(et, -1)) / np.maximum(amax, 1e-300)
    sx = np.repeat(np.asarray(scales, np.float64), 128, axis=1)
    y = np.abs(v) / sx
    band = ev / sx + y * np.repeat(scale_rel, 128, axis=1)
    sp = e4m3_spacing(y)
    lo = np.floor(y / sp) * sp
    sp_below = e4m3_spacing(np.maximum(lo - sp / 4, 0.0))
    dist = np.minimum(np.abs(y - (lo + sp / 2)), np.abs(y - (lo - sp_below / 2)))
    step = 2.0 * band + e4m3_spacing(y + band)
    code_ambiguity.margin = dist / np.maximum(band, 1e-300)   # for failure reports
    code_ambiguity.y = y
    code_ambiguity.band = band
    return dist <= band, step


def h_code_ambiguity(aq_rows, as_rows, w13q, w13s, g, u, h, hs, rule="fp32"):
    """code_ambiguity of the rows' h codes, with the noise of h propagated from
    G and U.  With the power-of-two rule a tile whose scale may legitimately
    be the next power up or down is ambiguous as a whole: its GPU values sit
    on a grid up to twice as coarse, i.e. within twice the band plus three
    spacings of the oracle's (in the oracle's scaled units)."""
    g = np.asarray(g, np.float64); u = np.asarray(u, np.float64); h = np.asarray(h, np.float64)
    eh = h_noise(aq_rows, as_rows, w13q, w13s, g, u, h)
    amb, step = code_ambiguity(h, eh, hs)
    if rule == "pow2":
        y, band = code_ambiguity.y, code_ambiguity.band
        s_lo, s_hi = pow2_scale_choices(h, eh)
        flip = np.repeat(s_lo != s_hi, 128, axis=1)
        amb = amb | flip
        step = np.where(flip, 2.0 * band + 3.0 * e4m3_spacing(2.0 * (y + band)), step)
    return amb, step


def check_h_codes(gh, hq, amb, step):
    """Unambiguous codes equal; ambiguous ones within their allowed step.  The
    two zero codes (+0, -0) count as equal: a value that rounds to zero has the
    sign of an h that is itself within noise of zero."""
    from oracle import fp8 as ofp8
    same = (gh == hq) | (((gh & 0x7F) == 0) & ((hq & 0x7F) == 0))
    bad = ~same & ~amb
    if np.any(bad):
        m = getattr(code_ambiguity, "margin", None)
        if m is not None and m.shape == bad.shape:
            yv = code_ambiguity.y
            print("  codes outside the band: distance to midpoint / band =",
                  np.array2string(m[bad][:10], precision=3), "scaled value",
                  np.array2string(yv[bad][:10], precision=4), "gpu", gh[bad][:10], "oracle", hq[bad][:10],
                  flush=True)
    assert np.all(same | amb), int(np.sum(bad))
    dv = np.abs(ofp8.e4m3_decode(gh) - ofp8.e4m3_decode(hq))
    assert np.all(dv[~same] <= 1.001 * step[~same])
    return int(np.sum(~same))


def y_allowance(amb, step, hs, w2q, w2s):
    """Elementwise bound on |delta y| [rows, d] from the ambiguous h codes
    taking another valid value."""
    W2 = oquant.dequant_128x128(w2q, w2s)
    delta = amb * step * np.repeat(np.asarray(hs, np.float64), 128, axis=1)
    return delta @ np.abs(W2).T


def rows_within(got, ref, allow, tol):
    """Per-row check ||got - ref|| <= tol * ||ref|| + ||allow||; returns
    (ok mask, relative errors, number of rows that needed the allowance)."""
    got = np.asarray(got, np.float64); ref = np.asarray(ref, np.float64)
    err = np.linalg.norm(got - ref, axis=-1)
    nref = np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    nall = np.linalg.norm(allow, axis=-1)
    ok = err <= tol * nref + nall
    rows_within.allow_rel = nall / nref     # for reports
    return ok, err / nref, int(np.sum(err > tol * nref))


def chain_report(err, allow_rel, tol):
    """One line on the independent chain (GPU layer against the oracle's own
    chain): rows above tol form a counted category, like near-tie tokens,
    each explained by SwiGLU outputs within the MFMA's noise of an E4M3
    rounding midpoint; the size of that allowance is printed."""
    over = err > tol
    return (f"independent chain: rel-L2 max {err.max():.2e} median {np.median(err):.2e}; "
            f"rows above {tol:.0e}: {int(over.sum())} of {err.size} (max {err.max():.2e}); "
            f"allowance ||allow||/||ref|| median {np.median(allow_rel):.2e} max {allow_rel.max():.2e}"
            + (f", on those rows max {allow_rel[over].max():.2e}" if over.any() else ""))


# ---- stage-fed check: the GPU's own H through the oracle's last stages ----------

def oracle_down_rows(hq, hs, experts_of_rows, experts):
    """The oracle's down projection of H rows given as codes and scales
    (e.g. the GPU's own): y = BF16(fl32(blocked GEMM with W2 of each row's
    expert)), float32 [rows, d]."""
    hq = np.asarray(hq); hs = np.asarray(hs, np.float32)
    ids = np.asarray(experts_of_rows)
    out = None
    for e in np.unique(ids):
        sel = np.nonzero(ids == e)[0]
        _, _, w2q, w2s = experts(int(e))
        y = ofp8.bf16_round(ofp8.f32(ogemm.blocked_gemm(hq[sel], hs[sel], w2q, w2s)))
        if out is None:
            out = np.zeros((ids.size, y.shape[1]), np.float32)
        out[sel] = y
    return out


def stage_fed_tokens(L, tokens, experts, E):
    """Layer output of ``tokens`` from the GPU's own routing (idx, w, pos) and
    its own FP8 H rows, through the oracle's down GEMM and combine: what the
    GPU's last two stages must reproduce within the layer tolerance."""
    T, k = L.idx.shape
    tokens = np.asarray(tokens)
    idx = to_np(L.idx)[tokens]; w = to_np(L.w)[tokens]; pos = to_np(L.pos)[tokens]
    rows = np.concatenate([pos.reshape(-1), T * k + tokens])
    ids = np.concatenate([idx.reshape(-1), np.full(tokens.size, E)])
    hq = L.h.index_select(0, torch.as_tensor(rows, device=L.h.device, dtype=torch.long)).cpu().numpy()
    hs = L.hs.index_select(0, torch.as_tensor(rows, device=L.hs.device, dtype=torch.long)).cpu().numpy()
    y = oracle_down_rows(hq, hs, ids, experts)
    n = tokens.size
    return olayer.combine(y[:n * k].reshape(n, k, -1), w, y[n * k:])


def layer_allowance(res, experts, T, k, E, rule="fp32"):
    """Bound on |delta out| [T, d] of a whole-batch oracle result (moe_layer)
    from the ambiguous h codes of every expert row, combined with the gates."""
    rows, d = res["y"].shape
    allow = np.zeros((rows, d))
    amb_all = np.zeros(res["hq"].shape, bool)
    sp_all = np.zeros(res["hq"].shape)
    off = res["offsets"]
    for e in range(E + 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        w13q, w13s, w2q, w2s = experts(e)
        amb, sp = h_code_ambiguity(res["xq_perm"][lo:hi], res["xs_perm"][lo:hi], w13q, w13s,
                                   res["g"][lo:hi], res["u"][lo:hi], res["h"][lo:hi],
                                   res["hs"][lo:hi], rule)
        amb_all[lo:hi], sp_all[lo:hi] = amb, sp
        allow[lo:hi] = y_allowance(amb, sp, res["hs"][lo:hi], w2q, w2s)
    w = np.asarray(res["route"]["w"], np.float64)
    out_allow = np.einsum("tk,tkd->td", np.abs(w), allow[np.asarray(res["pos"], np.int64)])
    out_allow += allow[T * k:T * k + T]
    return out_allow, amb_all, sp_all


def token_allowance(extra, r, experts, E, rule="fp32"):
    """The same bound for tokens evaluated on their own (moe_layer_tokens),
    batched per expert: the (token, slot) rows of one expert share its
    dequantised W2."""
    n, k = r["idx"].shape
    d = extra["y_shared"].shape[1]
    out = np.zeros((n, d))
    by_e = {}
    for t in range(n):
        for j in range(k):
            by_e.setdefault(int(r["idx"][t, j]), []).append((t, extra["inter_routed"][(t, j)],
                                                            abs(float(r["w"][t, j]))))
        by_e.setdefault(E, []).append((t, extra["inter_shared"][t], 1.0))
    for e, items in by_e.items():
        w13q, w13s, w2q, w2s = experts(e)
        ts = [t for t, _, _ in items]
        cat = {key: np.concatenate([it[key] for _, it, _ in items]) for key in ("g", "u", "h", "hs")}
        amb, sp = h_code_ambiguity(extra["xq"][ts], extra["xs"][ts], w13q, w13s, cat["g"], cat["u"],
                                   cat["h"], cat["hs"], rule)
        ya = y_allowance(amb, sp, cat["hs"], w2q, w2s)
        for i, (t, _, wt) in enumerate(items):
            out[t] += wt * ya[i]
    return out
