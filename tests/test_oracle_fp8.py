"""Pins of the oracle's fp8 expert-weight encoding: OCP MXFP8 (blocks of 32
values along K sharing one power-of-two scale X = floor(log2 amax) - 8,
elements OCP 8-bit floats E4M3: bias 7, subnormals, no infinities, largest
finite 448, saturating), the format the pages' "MxFP8" names.

External anchors: torch's float8_e4m3fn dtype, an independent library
implementation of the same OCP element format (decode of every code, and the
round-to-nearest-even cast of values inside the finite range), numpy's frexp
for the block exponent, plus the format's fixed points (1.0, 448, the
smallest normal and subnormal values).
"""
import math

import numpy as np
import pytest
import torch

import oracle

F8 = torch.float8_e4m3fn


def torch_decode(codes):
    return torch.tensor(np.asarray(codes, np.uint8)).view(F8).float().double().numpy()


def torch_encode(v):
    return torch.tensor(np.asarray(v, np.float32)).to(F8).view(torch.uint8).numpy()


def test_decode_every_code_matches_library():
    ref = torch_decode(np.arange(256))
    for c in range(256):
        got = oracle.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c] and math.copysign(1, got) == math.copysign(1, ref[c]), c


def test_format_fixed_points():
    assert oracle.e4m3_decode(0x38) == 1.0
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6
    assert oracle.e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert math.isnan(oracle.e4m3_decode(0x7F)) and math.isnan(oracle.e4m3_decode(0xFF))
    assert oracle.e4m3_encode(448.0) == 0x7E and oracle.e4m3_encode(-448.0) == 0xFE
    assert oracle.e4m3_encode(1e9) == 0x7E            # saturation
    assert oracle.e4m3_encode(-0.0) == 0x80


def test_encode_roundtrips_every_finite_code():
    for c in range(256):
        v = oracle.e4m3_decode(c)
        if not math.isnan(v):
            assert oracle.e4m3_encode(v) == c, c


def test_encode_midpoints_round_to_even():
    vals = sorted({oracle.e4m3_decode(c) for c in range(0x7F) if c != 0x7F})
    for a, b in zip(vals[:-1], vals[1:]):
        mid = (a + b) / 2
        ca, cb = oracle.e4m3_encode(a), oracle.e4m3_encode(b)
        want = ca if ca % 2 == 0 else cb
        assert oracle.e4m3_encode(mid) == want, (a, b)
        assert oracle.e4m3_encode(-mid) == want | 0x80


def test_encode_matches_library_cast():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000),
                        rng.standard_normal(20000) * 2.0 ** -7,
                        (rng.integers(-3600, 3600, 20000) + 0.5) * 2.0 ** -10])
    v = v.astype(np.float32)
    got = np.array([oracle.e4m3_encode(float(x)) for x in v], np.uint8)
    assert np.array_equal(got, torch_encode(v))


@pytest.mark.parametrize("K", [64, 2048])
def test_mx_block_quantisation(K):
    rng = np.random.default_rng(K)
    R = 40
    w = (rng.standard_normal((R, K)) / np.sqrt(K)).astype(np.float32)
    w[3, :32] = 0.0                                   # all-zero block
    w[5] *= 2.0 ** 20                                 # large row
    w[6] *= 2.0 ** -110                               # tiny row: exponent clamped at -110
    w[7, :32] = 500.0 * 2.0 ** -4                     # saturating block: amax / 2^X = 500 > 448
    w[7, 1] = 1.0 * 2.0 ** -4
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)  # bf16 (truncated) bits
    wf = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q, x = oracle.quant_mxfp8(wb)
    assert x.shape == (R, K // 32)
    blocks = wf.reshape(R, K // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    _, ex = np.frexp(amax)                            # amax = f * 2^ex, f in [0.5, 1)
    want_x = np.where(amax > 0, np.clip(ex - 1 - 8, -110, 110), 0)
    assert np.array_equal(x, want_x)
    assert x[6].max() == -110 and x[3, 0] == 0
    # codes: the library's RNE cast of v / 2^X after saturation to +-448
    scaled = np.clip(blocks / 2.0 ** x[:, :, None], -448, 448).reshape(R, K)
    assert np.array_equal(q, torch_encode(scaled).reshape(R, K))
    assert q[7, 0] == 0x7E                            # saturated to 448
    deq = oracle.dequant_mxfp8(q, x)
    dv = (deq.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    scale = np.repeat(2.0 ** x, 32, axis=1)
    # dequantised weights are exactly decode(q) * 2^X (bf16-exact)
    assert np.array_equal(dv, torch_decode(q.ravel()).reshape(R, K) * scale)
    # error: half an E4M3 ulp (relative 2^-4 normal, 2^-10 * 2^X subnormal)
    # unless saturated (|v| / 2^X in (448, 512))
    sat = np.abs(wf) / scale > 448
    bound = np.maximum(np.abs(wf) * 2.0 ** -4, scale * 2.0 ** -10)
    assert np.all((np.abs(dv - wf) <= bound) | sat)
    assert np.all(np.abs(dv[sat]) == 448 * scale[sat])
