"""Pins of the power-of-two (E8M0) scale rule of the oracle quantiser."""

import numpy as np

from oracle import fp8, quant
from oracle import layer as olayer


def _pow2(a):
    return quant.scale_from_amax(np.float32(a), "pow2")


def test_pow2_scale_by_hand():
    assert _pow2(448.0) == 1.0                       # amax/448 is exactly 1
    assert _pow2(449.0) == 2.0                       # just above: the next power up
    assert _pow2(224.0) == 0.5
    assert _pow2(300.0) == 1.0
    assert _pow2(448.0 * 2.0 ** -10) == 2.0 ** -10
    assert _pow2(0.0) == 1.0                         # all-zero tile
    # 2^-118 / 448 = 1.14 * 2^-127 (an FP32 subnormal): next power of two 2^-126
    assert _pow2(2.0 ** -118) == np.float32(2.0 ** -126)
    # far below E8M0's smallest value: clamped to 2^-127
    assert _pow2(1e-40) == np.float32(2.0 ** -127)


def _brute(amax):
    """Smallest 2^k (k = -127 .. 127) not below fl32(amax/448), by enumeration."""
    if amax == 0:
        return 1.0
    s = float(np.float32(np.float32(amax) / np.float32(448.0)))
    for k in range(-127, 128):
        if 2.0 ** k >= s:
            return 2.0 ** k
    raise AssertionError


def test_pow2_scale_matches_enumeration():
    rng = np.random.default_rng(3)
    exps = rng.integers(-130, 120, 4000)
    vals = (rng.uniform(1.0, 2.0, 4000) * 2.0 ** exps).astype(np.float32)
    # powers of two times 448, their float32 neighbours, and BF16-looking values
    edges = [np.float32(448.0 * 2.0 ** j) for j in range(-20, 20)]
    edges += [np.nextafter(e, np.float32(np.inf)) for e in edges]
    edges += [np.nextafter(e, np.float32(0)) for e in edges[:40]]
    allv = np.concatenate([vals, np.asarray(edges, np.float32), [0.0]]).astype(np.float32)
    got = quant.scale_from_amax(allv, "pow2")
    want = np.array([_brute(a) for a in allv], np.float64)
    assert np.array_equal(got.astype(np.float64), want)


def test_pow2_bounds_on_normal_tiles():
    rng = np.random.default_rng(5)
    x = fp8.bf16_round(rng.standard_normal((512, 1024)) * np.exp(rng.uniform(-8, 8, (512, 1)))).astype(np.float32)
    q2, s2 = quant.quant_1x128(x, "pow2")
    _, s1 = quant.quant_1x128(x, "fp32")
    m, _ = np.frexp(s2.astype(np.float64))
    assert np.all(m == 0.5)                                   # powers of two
    assert np.all(s2 >= s1) and np.all(s2 < 2 * s1)           # at most one octave coarser
    y = x.reshape(512, 8, 128) / s2[:, :, None]
    assert np.abs(y).max() <= 448.0                           # nothing saturates
    assert np.array_equal(q2.reshape(512, 8, 128), fp8.e4m3_encode(y.astype(np.float32)))


def test_pow2_equals_fp32_rule_when_quotient_is_a_power_of_two():
    rng = np.random.default_rng(7)
    x = fp8.bf16_round(rng.uniform(-1, 1, (64, 256))).astype(np.float32)
    j = rng.integers(-6, 6, (64, 2))
    t = x.reshape(64, 2, 128)
    t[:, :, 0] = 448.0 * 2.0 ** j                             # amax/448 = 2^j exactly
    t[:, :, 1:] = np.clip(t[:, :, 1:], -1, 1) * 2.0 ** j[:, :, None]
    x = t.reshape(64, 256)
    qa, sa = quant.quant_1x128(x, "fp32")
    qb, sb = quant.quant_1x128(x, "pow2")
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb)


def test_pow2_error_within_one_octave_of_fp32_rule():
    rng = np.random.default_rng(11)
    x = fp8.bf16_round(rng.standard_normal((2048, 128))).astype(np.float32)
    e = {}
    for rule in ("fp32", "pow2"):
        q, s = quant.quant_1x128(x, rule)
        r = quant.dequant_1x128(q, s)
        e[rule] = np.sqrt(np.mean((r - x) ** 2) / np.mean(x.astype(np.float64) ** 2))
    # coarser by the per-tile factor s_pow2 / s_fp32 in [1, 2)
    assert e["fp32"] < e["pow2"] < 2 * e["fp32"]


def test_pow2_128x128_on_grid_roundtrip_catches_transpose():
    rng = np.random.default_rng(13)
    n, k = 256, 384
    codes = rng.integers(0, 0x7E, (n, k)).astype(np.uint8) | (rng.integers(0, 2, (n, k)).astype(np.uint8) << 7)
    ex = rng.integers(-12, 4, (n // 128, k // 128))
    for bi in range(n // 128):
        for bj in range(k // 128):
            codes[bi * 128 + 5, bj * 128 + 7] = 0x7E       # 448 in every block: amax/448 = 2^ex
    vals = fp8.e4m3_decode(codes) * np.repeat(np.repeat(2.0 ** ex, 128, 0), 128, 1)
    q, s = quant.quant_128x128(vals.astype(np.float32), "pow2")
    assert np.array_equal(s, (2.0 ** ex).astype(np.float32))
    assert np.array_equal(q, codes)


def test_pow2_layer_scales_are_powers_of_two():
    rng = np.random.default_rng(17)
    T, d, E, f = 8, 256, 4, 128
    x = fp8.bf16_round(rng.standard_normal((T, d))).astype(np.float32)
    wg = fp8.bf16_round(rng.standard_normal((E, d)) / 16).astype(np.float32)
    ex = [olayer.quantize_expert(fp8.bf16_round(rng.standard_normal((2 * f, d)) / 16).astype(np.float32),
                                 fp8.bf16_round(rng.standard_normal((d, f)) / 16).astype(np.float32), "pow2")
          for _ in range(E + 1)]
    r = olayer.moe_layer(x, wg, np.zeros(E, np.float32), lambda e: ex[e], 2, 1, 2, 2.5, rule="pow2")
    for s in [r["xs"], r["hs"]] + [w[1] for w in ex] + [w[3] for w in ex]:
        m, _ = np.frexp(np.asarray(s, np.float64))
        assert np.all(m == 0.5)
