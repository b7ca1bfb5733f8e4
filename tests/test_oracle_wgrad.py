"""Pins of the oracle's grouped weight gradient dw[g] = dy_g^T a_g (the weight
gradient of out = a W_g^T per group): numpy's fp64 matmul per group, torch
fp64 autograd of the grouped matmul itself (so the transposition and the
group boundaries follow from the forward, not from a retyped formula), the
adjoint identity <dw, V> = sum_r <dy[r], a[r] V_g^T>, zero gradients for
empty groups, and the sampled-entries variant against the whole gradient."""
import numpy as np
import torch

import oracle


def _bf16(rng, shape, std):
    return (rng.normal(0, std, shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _val(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _case(seed=3, counts=(0, 37, 1, 90, 0, 5), M=48, K=80):
    rng = np.random.default_rng(seed)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offs[-1])
    return rng, offs, _bf16(rng, (rows, M), 1.0), _bf16(rng, (rows, K), 1.0)


def test_matches_numpy_per_group_and_empty_groups_are_zero():
    _, offs, dy, a = _case()
    dw = oracle.grouped_wgrad(dy, a, offs)
    assert dw.shape == (len(offs) - 1, dy.shape[1], a.shape[1])
    for g in range(len(offs) - 1):
        lo, hi = offs[g], offs[g + 1]
        if hi == lo:
            assert np.all(dw[g] == 0.0)
        ref = _val(dy[lo:hi]).T @ _val(a[lo:hi])
        assert np.allclose(dw[g], ref, rtol=1e-13, atol=1e-12)


def test_is_the_autograd_of_the_grouped_matmul():
    """out = a W_g^T on each group's rows (the expert matmul); backpropagating
    dy gives dW_g, which must equal the oracle's gradient."""
    rng, offs, dy, a = _case(seed=4)
    G, M, K = len(offs) - 1, dy.shape[1], a.shape[1]
    W = torch.tensor(_val(_bf16(rng, (G, M, K), 0.1)), requires_grad=True)
    A = torch.tensor(_val(a))
    outs = [A[offs[g]:offs[g + 1]] @ W[g].T for g in range(G)]
    torch.cat(outs).backward(torch.tensor(_val(dy)))
    dw = oracle.grouped_wgrad(dy, a, offs)
    assert np.allclose(dw, W.grad.numpy(), rtol=1e-13, atol=1e-12)


def test_adjoint_identity():
    """<dw, V> = sum_r <dy[r], a[r] V_g^T> for any V: dw is the adjoint of the
    grouped matmul applied to dy."""
    rng, offs, dy, a = _case(seed=5, counts=(12, 0, 33), M=32, K=64)
    V = rng.normal(0, 1, (len(offs) - 1, dy.shape[1], a.shape[1]))
    dw = oracle.grouped_wgrad(dy, a, offs)
    lhs = float((dw * V).sum())
    rhs = 0.0
    for g in range(len(offs) - 1):
        lo, hi = offs[g], offs[g + 1]
        rhs += float((_val(dy[lo:hi]) * (_val(a[lo:hi]) @ V[g].T)).sum())
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(rhs))


def test_entries_match_the_whole_gradient():
    rng, offs, dy, a = _case(seed=6)
    dw = oracle.grouped_wgrad(dy, a, offs)
    n = 200
    g = rng.integers(0, len(offs) - 1, n)
    m = rng.integers(0, dy.shape[1], n)
    k = rng.integers(0, a.shape[1], n)
    got = oracle.grouped_wgrad_entries(dy, a, offs, g, m, k)
    assert np.array_equal(got, dw[g, m, k])
