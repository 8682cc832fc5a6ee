"""The accumulation error of gfx950's FP8 MFMA, measured through the C ABI: the
measurement behind the noise constants of tests/gpu_util.py (MFMA_BLOCK_RMS,
MFMA_BLOCK_MAX, NOISE_SIGMAS, NOISE_BLOCKS, MAXPROD_FACTOR) that every
floating-point band of the GEMM parity tests is built from (GPU).

The method promotes each 128-wide K block's partial sum into FP32 because the
matrix unit's own accumulation is not exact ("DeepSeek-V3" summary page,
section 6 (b) "Higher-precision accumulation", limited accumulator precision
of about 14 bits on H800, up to ~2% error at K = 4096; the book's chapter 16
"Multiplication error and accumulation error differ").  On gfx950 one
v_mfma_scale_f32_16x16x128_f8f6f4 sums exactly one such block: its products of
E4M3 codes are exact, its 128-term sum is not.

Measured here with grouped_gemm_fp8_wgrad, whose output is FP32: with every
scale 1 (E8M0 code 127) and groups of exactly 128 rows, each output is one
MFMA's block sum; with groups of 7168 rows it is a chain of 56 blocks
accumulated through the instruction (the forward's FP32 promotion of each
partial gives the same errors, which the chain's model also bounds).  The
exact sums are integers times 2^-18 and are computed exactly in float64.
Operands are the E4M3 codes of N(0, 1) data quantised in 1x128 tiles (the
forward's operand distribution), seeded.
"""

import numpy as np
import pytest
import torch

import routing_fp8_grouped_amd as moe
from oracle import fp8, quant as oq
from tests.gpu_util import (DEV, log, MFMA_BLOCK_RMS, MFMA_BLOCK_MAX, NOISE_SIGMAS, NOISE_BLOCKS,
                            MAXPROD_FACTOR)

pytestmark = pytest.mark.gpu
M = N = 256


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def codes(rng, rows, K):
    """E4M3 codes [rows, K] of N(0, 1) data quantised in 1x128 tiles along K."""
    q, _ = oq.quant_1x128(rng.standard_normal((rows, K)).astype(np.float32))
    return q


def run_wgrad(aq, bq, group_rows):
    """dw [G, M, N] of grouped_gemm_fp8_wgrad on K-major codes aq [M, K],
    bq [N, K] split into groups of group_rows rows (multiples of 128), all
    scales 1."""
    K = aq.shape[1]
    G = K // group_rows
    kp = moe.moe_wgrad_columns(K, G)
    a_t = torch.zeros(M, kp, dtype=torch.uint8)
    b_t = torch.zeros(N, kp, dtype=torch.uint8)
    a_t[:, :K] = torch.from_numpy(aq)
    b_t[:, :K] = torch.from_numpy(bq)
    ones_a = torch.ones(kp // 128, M, dtype=torch.float32, device=DEV)
    ones_b = torch.ones(kp // 128, N, dtype=torch.float32, device=DEV)
    offsets = torch.arange(0, K + 1, group_rows, dtype=torch.int32, device=DEV)
    dw = torch.empty(G, M, N, dtype=torch.float32, device=DEV)
    moe.grouped_gemm_fp8_wgrad(a_t.to(DEV), ones_a, b_t.to(DEV), ones_b, offsets, G, K, dw)
    torch.cuda.synchronize()
    return dw.cpu().numpy().astype(np.float64)


def block_stats(a, b):
    """Per block kb and output (m, n): the exact sum, sum |a b| and max |a b|."""
    nb = a.shape[1] // 128
    exact = np.zeros((nb, M, N)); sabs = np.zeros_like(exact); mx = np.zeros_like(exact)
    for kb in range(nb):
        blk = slice(kb * 128, (kb + 1) * 128)
        exact[kb] = a[:, blk] @ b[:, blk].T
        sabs[kb] = np.abs(a[:, blk]) @ np.abs(b[:, blk]).T
        for m0 in range(0, M, 32):
            mx[kb, m0:m0 + 32] = np.max(np.abs(a[m0:m0 + 32, None, blk] * b[None, :, blk]), axis=2)
    return exact, sabs, mx


def test_single_block_error():
    """1,048,576 single-block sums (16 groups of 128 rows, 256 x 256 outputs
    each): the error relative to sum|a b| has the RMS and maximum that
    MFMA_BLOCK_RMS and MFMA_BLOCK_MAX state."""
    rng = np.random.default_rng(20241227)
    G = 16
    aq, bq = codes(rng, M, 128 * G), codes(rng, N, 128 * G)
    got = run_wgrad(aq, bq, 128)
    a, b = fp8.e4m3_decode(aq), fp8.e4m3_decode(bq)
    exact, sabs, mxp = block_stats(a, b)
    r = (got - exact) / sabs
    rms, mx = float(np.sqrt(np.mean(r * r))), float(np.max(np.abs(r)))
    frac_exact = float(np.mean(got == exact))
    by_max = float(np.max(np.abs(got - exact) / mxp))
    log(f"single block: rel error RMS {rms:.3e} (constant {MFMA_BLOCK_RMS:.3e}), max {mx:.3e} "
        f"(bound {MFMA_BLOCK_MAX:.3e}), mean {float(np.mean(r)):.2e}, exact in FP32 {frac_exact:.1%}; "
        f"error / max|a b| max {by_max:.2e} (bound {MAXPROD_FACTOR:.0e})")
    assert 0.5 * MFMA_BLOCK_RMS <= rms <= 1.25 * MFMA_BLOCK_RMS
    assert mx <= MFMA_BLOCK_MAX
    assert by_max < MAXPROD_FACTOR
    assert abs(float(np.mean(r))) < 0.05 * rms     # unbiased


def test_chain_error_model():
    """131,072 chains of 56 blocks (K = 7168, two groups of 7168 rows): the
    error against the RMS model sigma = MFMA_BLOCK_RMS * sqrt(sum over blocks
    of (sum|a b|)^2) stays below NOISE_SIGMAS sigma, at most NOISE_BLOCKS
    times the single-block bound, and below MAXPROD_FACTOR times the root-sum
    of the blocks' largest products."""
    rng = np.random.default_rng(20241228)
    K, G = 7168, 2
    aq, bq = codes(rng, M, K * G), codes(rng, N, K * G)
    got = run_wgrad(aq, bq, K)
    a, b = fp8.e4m3_decode(aq), fp8.e4m3_decode(bq)
    z_all, blk_all, mp_all = [], [], []
    for g in range(G):
        cols = slice(g * K, (g + 1) * K)
        exact, sabs, mx = block_stats(a[:, cols], b[:, cols])
        err = np.abs(got[g] - exact.sum(0))
        root = np.sqrt(np.sum(sabs * sabs, axis=0))
        # the bound of tests/gpu_util.gemm_noise, with FP32 accumulation
        bound = (np.maximum(NOISE_SIGMAS * MFMA_BLOCK_RMS * root, NOISE_BLOCKS * MFMA_BLOCK_MAX * sabs.max(0))
                 + (K // 128) * 2.0 ** -24 * np.abs(exact.sum(0)))
        assert np.all(err <= bound), float(np.max(err / bound))
        z_all.append(err / (MFMA_BLOCK_RMS * root))
        blk_all.append(err / (MFMA_BLOCK_MAX * sabs.max(0)))
        mp_all.append(err / np.sqrt(np.sum(mx * mx, axis=0)))
    z, bl, mp = (np.concatenate([v.reshape(-1) for v in x]) for x in (z_all, blk_all, mp_all))
    z_rms = float(np.sqrt(np.mean(z * z)))
    mp_rms = float(np.sqrt(np.mean(mp * mp)))
    log(f"56-block chains: error / sigma RMS {z_rms:.3f} max {z.max():.2f} (band {NOISE_SIGMAS}); "
        f"error / single-block bound max {bl.max():.2f} (band {NOISE_BLOCKS}); "
        f"error / root-sum of max products RMS {mp_rms:.2e} max {mp.max():.2e} (bound {MAXPROD_FACTOR:.0e})")
    assert 0.5 <= z_rms <= 1.5
    assert z.max() < NOISE_SIGMAS
    assert bl.max() < NOISE_BLOCKS
    assert mp.max() < MAXPROD_FACTOR
