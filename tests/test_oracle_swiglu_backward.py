"""Pins of the oracle's clamped-SwiGLU backward against torch's fp64 autograd
of clamp -> silu -> product (torch's own silu and clamp), and against the
cases the clamp fixes."""
import numpy as np
import pytest
import torch

import oracle


def _autograd(g, u, dh, L, mode):
    G = torch.tensor(g, dtype=torch.float64, requires_grad=True)
    U = torch.tensor(u, dtype=torch.float64, requires_grad=True)
    gc = torch.clamp(G, -L, L) if mode == 0 else torch.clamp(G, max=L)
    h = torch.nn.functional.silu(gc) * torch.clamp(U, -L, L)
    h.backward(torch.tensor(dh, dtype=torch.float64))
    return G.grad.numpy(), U.grad.numpy()


@pytest.mark.parametrize("L,mode,spread", [(10.0, 0, 3.0), (0.5, 0, 1.0), (0.5, 1, 1.0),
                                           (float("inf"), 0, 4.0), (2.0, 1, 6.0)])
def test_matches_autograd(L, mode, spread):
    rng = np.random.default_rng(int(spread * 10) + mode)
    g = rng.normal(0, spread, (64, 96)).astype(np.float32)
    u = rng.normal(0, spread, (64, 96)).astype(np.float32)
    dh = rng.normal(0, 1, (64, 96)).astype(np.float32)
    dg, du = oracle.swiglu_backward(g, u, dh, L, mode)
    rg, ru = _autograd(g, u, dh, L, mode)
    # relative to the size of the terms: silu' = s (1 + z (1 - s)) cancels to
    # 0 near z = -1.28, where only an absolute bound holds
    mag = np.abs(dh.astype(np.float64)) * (np.minimum(np.abs(u), L) + 1) * (1 + np.abs(g))
    assert np.all(np.abs(dg - rg) <= 1e-12 * mag)
    assert np.all(np.abs(du - ru) <= 1e-12 * mag)


def test_clamped_inputs_get_no_gradient():
    L = 1.0
    g = np.array([[-3.0, -1.0, 0.5, 1.0, 2.5]], np.float32)
    u = np.array([[0.5, -2.0, 3.0, 1.0, -1.0]], np.float32)
    dh = np.ones_like(g)
    dg, du = oracle.swiglu_backward(g, u, dh, L, 0)
    assert dg[0, 0] == 0.0 and dg[0, 4] == 0.0          # gate outside [-L, L]
    assert du[0, 1] == 0.0 and du[0, 2] == 0.0          # up outside [-L, L]
    assert dg[0, 1] != 0.0 and dg[0, 3] != 0.0          # at the limits: passed
    dg1, _ = oracle.swiglu_backward(g, u, dh, L, 1)     # gate clamped above only
    assert dg1[0, 0] != 0.0 and dg1[0, 4] == 0.0


def test_silu_derivative_special_values():
    """silu'(0) = 1/2 and silu'(z) -> 1 for large z: with U = 1 inside the
    clamp, dG is dh times those values and dU is dh silu(G)."""
    g = np.array([[0.0, 30.0, -30.0]], np.float32)
    u = np.ones_like(g)
    dh = np.full_like(g, 2.0)
    dg, du = oracle.swiglu_backward(g, u, dh, float("inf"), 0)
    assert dg[0, 0] == 1.0 and abs(dg[0, 1] - 2.0) < 1e-10 and abs(dg[0, 2]) < 1e-10
    assert du[0, 0] == 0.0 and abs(du[0, 1] - 60.0) < 1e-10
