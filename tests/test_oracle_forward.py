"""Pins of the oracle's router projection, combine and whole-layer chain.

- Router logits against a numpy fp64 matmul (<= 1 binary32 ulp).
- Dense reductions of the combine ("merged by routing weight" plus the
  always-on shared expert):
  (i)  k = 1 and a bias that forces expert e0: y = Ysh + scale * FFN_e0(x);
  (ii) all experts identical: y = Ysh + (sum_j w_j) * FFN(x) for any routing;
  (iii) scale = 0: y = Ysh;
  (iv) E = 1, k = 1: y = Ysh + scale * FFN(x);
  each FFN computed by numpy fp64 dense matmuls.
- The token-level form (used for sampled checks) equals the permuted chain.
"""
import math

import numpy as np
import pytest

from test_oracle_ffn import bf16_to_f64, bf16_round_np


def _bf(rng, shape, std):
    v = rng.normal(0, std, shape).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def _problem(seed, T, d, E, k, F, same_experts=False):
    rng = np.random.default_rng(seed)
    p = dict(x=_bf(rng, (T, d), 1.0), wg=_bf(rng, (E, d), 1 / math.sqrt(d)),
             w_gate=_bf(rng, (E, F, d), 1 / math.sqrt(d)), w_up=_bf(rng, (E, F, d), 1 / math.sqrt(d)),
             w_down=_bf(rng, (E, d, F), 1 / math.sqrt(F)), s_gate=_bf(rng, (F, d), 1 / math.sqrt(d)),
             s_up=_bf(rng, (F, d), 1 / math.sqrt(d)), s_down=_bf(rng, (d, F), 1 / math.sqrt(F)),
             bias=rng.uniform(-0.1, 0.1, (1, E)).astype(np.float32))
    if same_experts:
        for key in ("w_gate", "w_up", "w_down"):
            p[key][:] = p[key][0]
    return p


def dense_ffn(x_bits, wg, wu, wd, L=10.0):
    a = bf16_to_f64(x_bits)
    G = np.clip(a @ bf16_to_f64(wg).T, -L, L)
    U = np.clip(a @ bf16_to_f64(wu).T, -L, L)
    h = bf16_round_np(G / (1 + np.exp(-G)) * U)
    return h @ bf16_to_f64(wd).T


def test_gate_logits_vs_numpy(orc):
    p = _problem(1, 40, 256, 24, 2, 32)
    off = np.random.default_rng(2).normal(0, 2, 24).astype(np.float32)
    got = orc.gate_logits(p["x"], p["wg"], off)
    ref = (bf16_to_f64(p["x"]) @ bf16_to_f64(p["wg"]).T + off).astype(np.float32)
    ulp = np.spacing(np.abs(ref))
    assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp)


def _fwd(orc, p, logits, k, scale, shared=True, **kw):
    return orc.forward(p["x"], logits, k, scale, p["w_gate"], p["w_up"], p["w_down"],
                       p["s_gate"] if shared else None, p["s_up"] if shared else None,
                       p["s_down"] if shared else None, 10.0, 0, **kw)


def test_single_forced_expert(orc):
    T, d, E, k, F, e0 = 30, 64, 6, 1, 32, 4
    p = _problem(3, T, d, E, k, F)
    logits = orc.gate_logits(p["x"], p["wg"])
    bias = np.zeros((1, E), np.float32)
    bias[0, e0] = 1000.0
    out = _fwd(orc, p, logits, k, 2.5, bias=bias)
    assert np.all(out["ids"] == e0)
    ref = dense_ffn(p["x"], p["s_gate"], p["s_up"], p["s_down"]) + \
        2.5 * dense_ffn(p["x"], p["w_gate"][e0], p["w_up"][e0], p["w_down"][e0])
    assert np.allclose(out["y"], ref, rtol=1e-10, atol=1e-10)
    out2 = _fwd(orc, p, logits, k, 2.5, shared=False, bias=bias)
    assert np.allclose(out2["y"], 2.5 * dense_ffn(p["x"], p["w_gate"][e0], p["w_up"][e0],
                                                  p["w_down"][e0]), rtol=1e-10, atol=1e-10)


def test_identical_experts(orc):
    T, d, E, k, F = 50, 64, 8, 3, 32
    p = _problem(4, T, d, E, k, F, same_experts=True)
    logits = orc.gate_logits(p["x"], p["wg"])
    out = _fwd(orc, p, logits, k, 1.7, bias=p["bias"])
    ysh = dense_ffn(p["x"], p["s_gate"], p["s_up"], p["s_down"])
    fx = dense_ffn(p["x"], p["w_gate"][0], p["w_up"][0], p["w_down"][0])
    ref = ysh + out["w"].astype(np.float64).sum(axis=1, keepdims=True) * fx
    assert np.allclose(out["y"], ref, rtol=1e-10, atol=1e-10)


def test_scale_zero(orc):
    p = _problem(5, 20, 64, 8, 2, 32)
    out = _fwd(orc, p, orc.gate_logits(p["x"], p["wg"]), 2, 0.0, bias=p["bias"])
    ysh = dense_ffn(p["x"], p["s_gate"], p["s_up"], p["s_down"])
    assert np.allclose(out["y"], ysh, rtol=1e-10, atol=1e-12)


def test_single_expert_layer(orc):
    p = _problem(6, 25, 64, 1, 1, 32)
    out = _fwd(orc, p, orc.gate_logits(p["x"], p["wg"]), 1, 2.5)
    ref = dense_ffn(p["x"], p["s_gate"], p["s_up"], p["s_down"]) + \
        2.5 * dense_ffn(p["x"], p["w_gate"][0], p["w_up"][0], p["w_down"][0])
    assert np.allclose(out["y"], ref, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("shared", [True, False])
def test_token_form_equals_chain(orc, shared):
    T, d, E, k, F = 70, 64, 8, 2, 32
    p = _problem(7, T, d, E, k, F)
    logits = orc.gate_logits(p["x"], p["wg"])
    out = _fwd(orc, p, logits, k, 1.0, shared=shared, bias=p["bias"])
    tok = np.array([0, 5, 69, 33], np.int64)
    y = orc.tokens_forward(p["x"], tok, out["ids"], out["w"], p["w_gate"], p["w_up"],
                           p["w_down"], p["s_gate"] if shared else None,
                           p["s_up"] if shared else None, p["s_down"] if shared else None, 10.0)
    assert np.allclose(y, out["y"][tok], rtol=1e-12, atol=1e-13)
