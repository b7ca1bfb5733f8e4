"""Pins of the oracle's expert FFN (two expert matmuls with the clamped SwiGLU
between them: MegaMoE bullet, section 2.3 of the HyperParallel page; clamp
limit L = 10 on gate and up before SwiGLU is the workload's parameter).

- bf16 rounding against exact rational rounding (ties to even, subnormals,
  overflow).
- The grouped FFN against a numpy fp64 dense FFN (textbook matmuls) per group.
- The clamp against its closed form on saturating inputs: with |G|, |U| > L
  every h is bf16(silu(+-L) * (+-L)).
- L = inf disables the clamp; clamp mode 1 clamps the gate from above only.
"""
from fractions import Fraction
import math

import numpy as np
import pytest


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_round_np(v):
    """bf16 RNE of finite fp64 values (numpy, independent of the C oracle):
    8 significant bits in the normal range, spacing 2^-133 below 2^-126."""
    m, e = np.frexp(v)
    normal = np.ldexp(np.rint(m * 256.0), e - 8)
    sub = np.ldexp(np.rint(np.ldexp(v, 133)), -133)
    return np.where(np.abs(v) < 2.0 ** -126, sub, normal)


def exact_bf16_bits(v: float) -> int:
    if math.isnan(v):
        return 0x7FC0
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    if math.isinf(v):
        return sign | 0x7F80
    a = Fraction(abs(v))
    if a == 0:
        return sign
    if a < Fraction(2) ** -126:
        q = round(a / Fraction(2) ** -133) * Fraction(2) ** -133
    else:
        e = math.frexp(abs(v))[1] - 1            # 2^e <= a < 2^(e+1)
        ulp = Fraction(2) ** (e - 7)
        q = round(a / ulp) * ulp                 # Fraction round: half to even
    if q > (2 - Fraction(2) ** -7) * Fraction(2) ** 127:
        return sign | 0x7F80
    f = np.float32(float(q))
    return sign | (int(f.view(np.uint32)) >> 16)


def test_bf16_rounding_exact(orc):
    rng = np.random.default_rng(1)
    vals = list(rng.normal(0, 1, 2000) * np.exp2(rng.integers(-140, 130, 2000)))
    for e in (-130, -127, -126, -20, 0, 5, 127):
        for m in (256, 257, 258, 511):          # exact midpoints: ties to even
            vals.append((m + 0.5) * 2.0 ** (e - 8))
            vals.append(-(m + 0.5) * 2.0 ** (e - 8))
    vals += [0.0, -0.0, 1e-45, 3.3e38, 3.4e38, -3.5e38, 1e300, float("inf"), 2.0 ** -133,
             1.5 * 2.0 ** -133, 2.5 * 2.0 ** -133]
    for v in vals:
        assert orc.f64_to_bf16(float(v)) == exact_bf16_bits(float(v)), v
    assert orc.f64_to_bf16(float("nan")) & 0x7F80 == 0x7F80


def _weights(rng, G, F, d, scale_x=1.0):
    def bf(shape, std):
        v = (rng.normal(0, std, shape)).astype(np.float32)
        return (v.view(np.uint32) >> 16).astype(np.uint16)   # truncation: any bf16 values do
    return (bf((G, F, d), 1 / math.sqrt(d)), bf((G, F, d), 1 / math.sqrt(d)),
            bf((G, d, F), 1 / math.sqrt(F)))


def _ref_ffn(a64, wg, wu, wd, L, mode):
    G = a64 @ bf16_to_f64(wg).T
    U = a64 @ bf16_to_f64(wu).T
    if mode == 0:
        G = np.clip(G, -L, L)
    else:
        G = np.minimum(G, L)
    U = np.clip(U, -L, L)
    pre = G / (1.0 + np.exp(-G)) * U
    return pre, bf16_round_np(pre)


def _check_group(orc, a, offsets, wg, wu, wd, L, mode, h, y):
    a64 = bf16_to_f64(a)
    for g in range(len(offsets) - 1):
        lo, hi = offsets[g], offsets[g + 1]
        if hi == lo:
            continue
        pre, href = _ref_ffn(a64[lo:hi], wg[g], wu[g], wd[g], L, mode)
        hgot = bf16_to_f64(h[lo:hi])
        bad = hgot != href
        if bad.any():
            # only values within rounding noise of a bf16 midpoint may differ
            mid = (np.abs(hgot - href) <= np.abs(href) * 2.0 ** -7) & \
                  (np.abs(np.abs(pre) - (np.abs(hgot) + np.abs(href)) / 2) <=
                   1e-12 * np.abs(pre))
            assert np.all(mid[bad])
        yref = hgot @ bf16_to_f64(wd[g]).T
        scale = np.abs(hgot) @ np.abs(bf16_to_f64(wd[g])).T
        assert np.all(np.abs(y[lo:hi] - yref) <= 1e-12 * scale + 1e-300)


@pytest.mark.parametrize("mode", [0, 1])
def test_grouped_ffn_matches_dense(orc, mode):
    rng = np.random.default_rng(20 + mode)
    G, d, F, rows = 5, 64, 48, 90
    wg, wu, wd = _weights(rng, G, F, d)
    a = (rng.normal(0, 1, (rows, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    offsets = np.array([0, 10, 10, 45, 80, 90], np.int32)      # includes an empty expert
    h, y = orc.expert_ffn(a, offsets, wg, wu, wd, 10.0, mode)
    _check_group(orc, a, offsets, wg, wu, wd, 10.0, mode, h, y)


def test_clamp_closed_form(orc):
    rng = np.random.default_rng(30)
    G, d, F, rows, L = 1, 64, 64, 40, 10.0
    wg, wu, wd = _weights(rng, G, F, d)
    x = (rng.normal(0, 30, (rows, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    h, _ = orc.expert_ffn(x, np.array([0, rows], np.int32), wg, wu, wd, L, 0)
    a64 = bf16_to_f64(x)
    Gf = a64 @ bf16_to_f64(wg[0]).T
    Uf = a64 @ bf16_to_f64(wu[0]).T
    sat = (np.abs(Gf) > L) & (np.abs(Uf) > L)
    assert sat.sum() > 300

    def silu(z):
        return z / (1.0 + math.exp(-z))
    closed = {(sg, su): exact_bf16_bits(silu(sg * L) * su * L)
              for sg in (-1, 1) for su in (-1, 1)}
    # silu(10)*10 = 99.99546..., silu(-10)*10 = -4.5397868e-3
    assert abs(silu(L) * L - 99.99546021312976) < 1e-12
    assert abs(silu(-L) * L + 4.539786870243439e-3) < 1e-15
    for r, f in zip(*np.nonzero(sat)):
        want = closed[(int(np.sign(Gf[r, f])), int(np.sign(Uf[r, f])))]
        assert int(h[r, f]) == want


def test_no_clamp_when_limit_infinite(orc):
    rng = np.random.default_rng(31)
    G, d, F, rows = 2, 64, 32, 30
    wg, wu, wd = _weights(rng, G, F, d)
    x = (rng.normal(0, 30, (rows, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    offsets = np.array([0, 13, 30], np.int32)
    h, y = orc.expert_ffn(x, offsets, wg, wu, wd, float("inf"), 0)
    _check_group(orc, x, offsets, wg, wu, wd, float("inf"), 0, h, y)


def test_rows_variant_matches_grouped(orc):
    rng = np.random.default_rng(32)
    G, d, F, rows = 3, 64, 32, 24
    wg, wu, wd = _weights(rng, G, F, d)
    a = (rng.normal(0, 1, (rows, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    offsets = np.array([0, 5, 17, 24], np.int32)
    h, y = orc.expert_ffn(a, offsets, wg, wu, wd, 10.0)
    sel = np.array([0, 6, 23, 16], np.int64)
    ex = np.array([0, 1, 2, 1], np.int32)
    h2, y2 = orc.expert_ffn_rows(a, sel, ex, wg, wu, wd, 10.0)
    assert np.array_equal(h2, h[sel]) and np.array_equal(y2, y[sel])
