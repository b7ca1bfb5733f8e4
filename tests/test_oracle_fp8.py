"""Pins of the oracle's fp8 expert-weight encoding (OCP 8-bit floating point,
E4M3 with bias 7, subnormals, no infinities, largest finite 448; one
power-of-two scale per output row - the reading of the pages' FP8 weights).

External anchors: torch's float8_e4m3fn dtype, an independent library
implementation of the same OCP format (decode of every code, and the
round-to-nearest-even cast of values inside the finite range), plus the
format's fixed points (1.0, 448, the smallest normal and subnormal values).
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
def test_row_quantisation(K):
    rng = np.random.default_rng(K)
    w = (rng.standard_normal((40, K)) / np.sqrt(K)).astype(np.float32)
    w[3] = 0.0                                        # all-zero row
    w[5] *= 2.0 ** 20                                 # large row
    w[6, :] = w[6, :] * 2.0 ** -30                    # tiny row (subnormal codes)
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)  # bf16 (truncated) bits
    wf = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q, e = oracle.quant_fp8_rows(wb)
    amax = np.abs(wf).max(axis=1)
    for r in range(w.shape[0]):
        if amax[r] == 0:
            assert e[r] == 0 and not q[r].any()
            continue
        # the smallest e with amax <= 448 * 2^e
        assert amax[r] <= 448 * 2.0 ** e[r] < 2 * amax[r]
        # codes are the library's RNE cast of w / 2^e
        assert np.array_equal(q[r], torch_encode(wf[r] / 2.0 ** e[r]))
    deq = oracle.dequant_fp8_rows(q, e)
    dv = (deq.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # dequantised weights are exactly decode(q) * 2^e (bf16-exact)
    assert np.array_equal(dv, torch_decode(q.ravel()).reshape(q.shape) * 2.0 ** e[:, None])
    # error: half an E4M3 ulp (relative 2^-4 in the normal range, 2^-10 * 2^e below)
    bound = np.maximum(np.abs(wf) * 2.0 ** -4, 2.0 ** (e[:, None] - 10.0))
    assert np.all(np.abs(dv - wf) <= bound)
