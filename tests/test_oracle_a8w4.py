"""Pins of the oracle's A8W4 layer ("CANN DeepSeek-V4 training optimisation",
outlook, functional-expansion bullets: A8W4 low-precision training on MxFP8 /
MxFP4): the routed expert matmuls take MXFP8 activations (x along d before
gate/up, the bf16 h along F before down), the routed weights are MXFP4
values, everything else is the bf16 layer.

External anchors: the MX format's own properties (a block already on the MX
grid quantises to itself; every quantised block lies on the E4M3 grid scaled
by 2^X with X = floor(log2 amax) - 8 from numpy's frexp, within half a grid
step of the input or saturated), invariance of the routed part under any
change of x that leaves its quantisation unchanged, identity down weights
that expose h's quantisation, and the unquantised shared expert.
"""
import math

import numpy as np
import torch

from test_oracle_ffn import bf16_to_f64
from test_oracle_forward import _bf, _problem

F8 = torch.float8_e4m3fn


def _on_grid_and_near(v_bits, q_bits):
    """every 32-block of q lies on the E4M3 grid x 2^X, X from v's block
    maximum, and is within half a grid step of v (or saturated at 448 2^X)"""
    v = bf16_to_f64(v_bits).reshape(-1, 32)
    q = bf16_to_f64(q_bits).reshape(-1, 32)
    for vb, qb in zip(v, q):
        amax = np.abs(vb).max()
        if amax == 0:
            assert np.all(qb == 0)
            continue
        X = np.frexp(amax)[1] - 1 - 8
        s = qb * 2.0 ** -X
        back = torch.tensor(s, dtype=torch.float64).to(torch.float32).to(F8).double().numpy()
        assert np.array_equal(back, s)                       # on the E4M3 grid
        a = np.abs(vb * 2.0 ** -X)
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
        step = 2.0 ** (e - 3)                                 # E4M3 spacing (subnormal: 2^-9)
        err = np.abs(s - vb * 2.0 ** -X)
        assert np.all((err <= step / 2) | ((a > 448) & (np.abs(s) == 448)))


def test_quant_dequant_is_idempotent_and_on_grid(orc):
    rng = np.random.default_rng(3)
    v = _bf(rng, (64, 256), 1.0)
    v[1, :32] = 0                                             # an all-zero block
    v[2, 32:64] = _bf(rng, (32,), 1e-3)                       # small values
    v[3] = _bf(rng, (256,), 300.0)                            # large values
    q = orc.quant_dequant_mxfp8(v)
    assert np.array_equal(orc.quant_dequant_mxfp8(q), q)
    _on_grid_and_near(v, q)


def _a8(orc, p, logits, k, scale, shared=True, **kw):
    return orc.forward_a8w4(p["x"], logits, k, scale, p["w_gate"], p["w_up"], p["w_down"],
                            p["s_gate"] if shared else None, p["s_up"] if shared else None,
                            p["s_down"] if shared else None, 10.0, 0, **kw)


def test_routed_part_sees_only_the_quantised_x(orc):
    T, d, E, k, F = 48, 64, 8, 2, 64
    p = _problem(5, T, d, E, k, F)
    logits = orc.gate_logits(p["x"], p["wg"])
    q = orc.quant_dequant_mxfp8(p["x"])
    # flip the last mantissa bit of every element whose quantised value stays
    # (with its block's exponent unchanged each element quantises alone)
    xa = p["x"] ^ np.uint16(1)
    qa = orc.quant_dequant_mxfp8(xa)
    same_x = np.repeat(orc.quant_mxfp8(xa)[1] == orc.quant_mxfp8(p["x"])[1], 32, axis=1)
    x2 = np.where(same_x & (qa == q), xa, p["x"]).astype(np.uint16)
    assert np.array_equal(orc.quant_dequant_mxfp8(x2), q) and np.count_nonzero(x2 != p["x"]) > T * d // 2
    r1 = _a8(orc, p, logits, k, 2.5)
    r2 = _a8(orc, dict(p, x=x2), logits, k, 2.5)
    assert np.array_equal(r1["x_perm"], q[r1["src"][r1["src"] >= 0]])
    assert np.array_equal(r1["y_perm"], r2["y_perm"])
    # the bf16 layer does see the change
    b1 = orc.forward(p["x"], logits, k, 2.5, p["w_gate"], p["w_up"], p["w_down"])
    b2 = orc.forward(x2, logits, k, 2.5, p["w_gate"], p["w_up"], p["w_down"])
    assert not np.array_equal(b1["y_perm"], b2["y_perm"])


def test_h_is_quantised_along_F(orc):
    # F = d = 32 and identity down weights: y_perm is the quantised h itself
    T, d, E, k, F = 40, 32, 4, 2, 32
    p = _problem(7, T, d, E, k, F)
    eye = (np.eye(32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    p["w_down"] = np.repeat(eye[None], E, axis=0)
    logits = orc.gate_logits(p["x"], p["wg"])
    r = _a8(orc, p, logits, k, 1.0, shared=False)
    n = int(r["offsets"][-1])
    h8 = bf16_to_f64(r["h8"][:n])
    assert np.array_equal(r["y_perm"][:n], h8)
    _on_grid_and_near(r["h"][:n], r["h8"][:n])
    assert not np.array_equal(h8, bf16_to_f64(r["h"][:n]))


def test_shared_expert_and_routing_are_the_bf16_layers(orc):
    T, d, E, k, F = 40, 64, 8, 3, 64
    p = _problem(9, T, d, E, k, F)
    logits = orc.gate_logits(p["x"], p["wg"])
    a = _a8(orc, p, logits, k, 2.5)
    b = orc.forward(p["x"], logits, k, 2.5, p["w_gate"], p["w_up"], p["w_down"], p["s_gate"],
                    p["s_up"], p["s_down"], 10.0, 0)
    assert np.array_equal(a["ysh"], b["ysh"])
    for key in ("ids", "w", "dest", "src", "offsets"):
        assert np.array_equal(a[key], b[key])


def test_token_form_matches_the_chain(orc):
    T, d, E, k, F = 60, 64, 8, 3, 64
    p = _problem(11, T, d, E, k, F)
    logits = orc.gate_logits(p["x"], p["wg"])
    a = _a8(orc, p, logits, k, 2.5)
    toks = np.array([0, 5, 17, 59])
    y = orc.tokens_forward_a8w4(p["x"], toks, a["ids"], a["w"], p["w_gate"], p["w_up"],
                                p["w_down"], p["s_gate"], p["s_up"], p["s_down"], 10.0, 0)
    assert np.allclose(y, a["y"][toks], rtol=1e-12, atol=1e-12 * np.abs(a["y"]).max())
