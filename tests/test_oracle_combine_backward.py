"""Pins of the oracle's combine backward against torch's fp64 autograd of the
combine (gather, weight, sum), written independently of the oracle, and
against the identity that the routed part of the output is linear in the
routing weights."""
import numpy as np
import torch

import oracle


def _case(T, d, k, seed, E=None):
    rng = np.random.default_rng(seed)
    E = E or 4 * k
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    _, _, dest, _, _ = oracle.permute(ids, E)
    rows = T * k
    yp = rng.normal(0, 1, (rows, d)).astype(np.float32)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    dy = rng.normal(0, 1, (T, d)).astype(np.float32)
    return dy, yp, dest.reshape(T, k), w


def _autograd(dy, yp, dest, w):
    Y = torch.tensor(yp, dtype=torch.float64, requires_grad=True)
    W = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    idx = torch.tensor(dest, dtype=torch.int64)
    y = (W.unsqueeze(-1) * Y[idx]).sum(dim=1)          # [T, d]
    y.backward(torch.tensor(dy, dtype=torch.float64))
    return Y.grad.numpy(), W.grad.numpy()


def test_matches_autograd():
    for T, d, k in ((40, 64, 6), (17, 200, 2), (8, 1024, 8)):
        dy, yp, dest, w = _case(T, d, k, T + d + k)
        gy, gw = oracle.combine_backward(dy, yp, dest, w)
        ry, rw = _autograd(dy, yp, dest, w)
        assert np.allclose(gy, ry, rtol=1e-15, atol=0)
        assert np.allclose(gw, rw, rtol=1e-12, atol=1e-12)


def test_linear_in_weights():
    """y - y_shared = sum_j w_j Y[dest_j] is linear in w, so
    sum_j w_j dw_j = <dy, y - y_shared> for every token."""
    dy, yp, dest, w = _case(32, 128, 4, 5)
    _, gw = oracle.combine_backward(dy, yp, dest, w)
    y = oracle.combine(yp.astype(np.float64), dest.ravel(), w)
    lhs = np.sum(w.astype(np.float64) * gw, axis=1)
    rhs = np.sum(dy.astype(np.float64) * y, axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_invalid_dest_and_untouched_rows():
    dy, yp, dest, w = _case(6, 32, 2, 9)
    dest = dest.copy()
    lost = int(dest[2, 1])
    dest[2, 1] = -1
    keep = np.full((yp.shape[0], yp.shape[1]), 7.0)
    gy, gw = oracle.combine_backward(dy, yp, dest, w, dy_perm=keep)
    assert gw[2, 1] == 0.0
    assert np.all(gy[lost] == 7.0)                    # no pair maps to it any more
    assert np.array_equal(gy[dest[0, 0]], w[0, 0].astype(np.float64) * dy[0].astype(np.float64))
