"""Pins of the oracle's MXFP4 expert-weight encoding (OCP Microscaling: blocks
of 32 values along K sharing one power-of-two scale X = floor(log2 amax) - 2,
elements OCP E2M1 floats: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, saturating).

Anchors: the E2M1 value table the OCP specification prints (torch has no
float4 conversion to compare with), brute force over all 16 codes for the
rounding (nearest value, ties to the code with mantissa bit 0), numpy's
frexp for the block exponent.
"""
import numpy as np
import pytest

import oracle

SPEC_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # OCP E2M1, codes 0-7


def test_decode_matches_spec_table():
    for c in range(16):
        v = oracle.e2m1_decode(c)
        assert abs(v) == SPEC_MAGNITUDES[c & 7]
        assert np.signbit(v) == bool(c & 8)


def brute_encode(v):
    """nearest of the 16 codes; among equally near ones the even code."""
    vals = np.array([oracle.e2m1_decode(c) for c in range(16)])
    v = float(np.clip(v, -6.0, 6.0))
    d = np.abs(vals - v)
    best = [c for c in range(16) if d[c] == d.min()]
    # a value equally near +0 and -0 keeps its sign; otherwise the even code
    best = [c for c in best if np.signbit(vals[c]) == np.signbit(v) or vals[c] != 0.0] or best
    even = [c for c in best if c % 2 == 0]
    return (even or best)[0]


def test_encode_against_brute_force():
    rng = np.random.default_rng(3)
    mids = [(a + b) / 2 for a, b in zip(SPEC_MAGNITUDES[:-1], SPEC_MAGNITUDES[1:])]
    vals = np.concatenate([SPEC_MAGNITUDES, mids, rng.uniform(-8, 8, 4000),
                           np.array(mids) * -1, [7.0, -9.0, 1e30]])
    for v in vals:
        assert oracle.e2m1_encode(v) == brute_encode(v), v


def test_ties_to_even_and_saturation():
    # midpoints between neighbours: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2,
    # 2.5 -> 2, 3.5 -> 4, 5 -> 4 (the neighbour whose code has mantissa bit 0)
    for v, want in ((0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0), (3.5, 4.0),
                    (5.0, 4.0), (6.5, 6.0), (1e9, 6.0)):
        assert oracle.e2m1_decode(oracle.e2m1_encode(v)) == want
        assert oracle.e2m1_decode(oracle.e2m1_encode(-v)) == -want


@pytest.mark.parametrize("K", [64, 1024])
def test_mx_block_quantisation(K):
    rng = np.random.default_rng(K + 1)
    R = 24
    w = (rng.standard_normal((R, K)) / np.sqrt(K)).astype(np.float32)
    w[2, :32] = 0.0                                   # all-zero block
    w[4] *= 2.0 ** 30                                 # large row
    w[5] *= 2.0 ** -110                               # exponent clamped at -110
    w[6, :32] = 7.0 * 2.0 ** -3                       # saturating block: amax / 2^X = 7 > 6
    w[6, 3] = 1.0 * 2.0 ** -3
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    wf = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q, x = oracle.quant_mxfp4(wb)
    blocks = wf.reshape(R, K // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    _, ex = np.frexp(amax)
    want_x = np.where(amax > 0, np.clip(ex - 1 - 2, -110, 110), 0)
    assert np.array_equal(x, want_x)
    scaled = (blocks / 2.0 ** x[:, :, None]).reshape(R, K)
    assert q.max() < 16
    sample = rng.choice(R * K, min(3000, R * K), replace=False)
    for i in sample:
        assert q.ravel()[i] == brute_encode(scaled.ravel()[i])
    assert q[6, 0] == 7                               # saturated to 6
    deq = oracle.dequant_mxfp4(q, x)
    dv = (deq.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    dec = np.array([oracle.e2m1_decode(c) for c in range(16)])[q]
    scale = np.repeat(2.0 ** x, 32, axis=1)
    assert np.array_equal(dv, dec * scale)           # exact bf16 values
    # error: half the E2M1 spacing at the value (0.25 below 2, 0.5 below 4,
    # 1 above) times the scale, unless saturated
    a = np.abs(wf) / scale
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0)) * scale
    sat = a > 6
    assert np.all((np.abs(dv - wf) <= half) | sat)
