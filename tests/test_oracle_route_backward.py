"""Pins of the oracle's routing backward (gradient of the routing weights
with respect to the router logits) against torch's fp64 autograd of the
same forward, written independently of the oracle (sigmoid, gather,
normalise, scale), and against invariants the formula must satisfy."""
import numpy as np
import pytest
import torch

import oracle


def _autograd(logits, ids, dw, scale):
    """fp64 autograd of w = scale * g / sum(g), g = sigmoid(l)[ids]: returns
    the gradient w.r.t. the logits [T,E] and w.r.t. g scattered to [T,E]."""
    l = torch.tensor(logits, dtype=torch.float64, requires_grad=True)
    idx = torch.tensor(ids, dtype=torch.int64)
    g = torch.gather(torch.sigmoid(l), 1, idx)
    g.retain_grad()
    w = scale * g / g.sum(dim=1, keepdim=True)
    w.backward(torch.tensor(dw, dtype=torch.float64))
    dg = torch.zeros_like(l).scatter_(1, idx, g.grad)
    return l.grad.numpy(), dg.detach().numpy()


def _close(dl, ref, dg):
    """The oracle takes the logistic derivative at the forward's binary32
    score s: s and 1 - s carry up to ~4 x 2^-24 of absolute error there (the
    rounding of s plus the sigmoid's 3 ulp), which dominates in the tails;
    everything else agrees to fp64 rounding plus S's relative error."""
    tol = 8 * 2.0 ** -24 * np.abs(dg) + 1e-5 * np.abs(ref) + 1e-15
    return np.all(np.abs(dl - ref) <= tol)


def _case(T, E, k, seed, hash_ids=False, spread=1.5):
    rng = np.random.default_rng(seed)
    lg = rng.normal(0, spread, (T, E)).astype(np.float32)
    if hash_ids:     # any distinct ids, not the top-k of the scores
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    else:
        ids, _, _ = oracle.route(lg, k, 1.0, bias=rng.uniform(-0.1, 0.1, E).astype(np.float32))
    dw = rng.normal(0, 1, (T, k)).astype(np.float32)
    return lg, ids, dw


@pytest.mark.parametrize("T,E,k,scale,hash_ids", [(64, 32, 4, 2.5, False), (50, 384, 6, 2.5, False),
                                                  (40, 16, 8, 1.0, False), (30, 64, 6, 1.0, True)])
def test_matches_autograd(T, E, k, scale, hash_ids):
    lg, ids, dw = _case(T, E, k, T + E + k, hash_ids)
    dl, flags = oracle.route_backward(lg, ids, dw, scale)
    ref, dg = _autograd(lg, ids, dw, scale)
    assert flags == 0
    assert _close(dl, ref, dg)


def test_only_selected_logits_get_gradient():
    lg, ids, dw = _case(32, 64, 6, 7)
    dl, _ = oracle.route_backward(lg, ids, dw, 2.5)
    mask = np.zeros_like(dl, dtype=bool)
    np.put_along_axis(mask, ids.astype(np.int64), True, axis=1)
    assert np.all(dl[~mask] == 0.0)
    assert np.count_nonzero(dl[mask]) > 0.9 * mask.sum()


def test_scale_invariance():
    """w is unchanged when every selected score is multiplied by one factor,
    so the gradient along g vanishes: sum_j g_j dg_j = 0."""
    lg, ids, dw = _case(64, 48, 6, 11)
    dl, _ = oracle.route_backward(lg, ids, dw, 2.5)
    g = oracle.score(np.take_along_axis(lg, ids.astype(np.int64), axis=1)).astype(np.float64)
    dg = np.take_along_axis(dl, ids.astype(np.int64), axis=1) / (g * (1.0 - g))
    lhs = np.sum(g * dg, axis=1)
    assert np.all(np.abs(lhs) <= 1e-12 * 2.5 * np.abs(dw).sum(axis=1))


def test_constant_weights_have_no_gradient():
    lg, ids, _ = _case(16, 32, 1, 3)
    dl, _ = oracle.route_backward(lg, ids, np.random.default_rng(1).normal(0, 1, (16, 1))
                                  .astype(np.float32), 2.5)
    assert np.all(dl == 0.0)                  # k = 1: w = scale whatever the logits
    lg, ids, _ = _case(16, 32, 6, 4)
    dl, _ = oracle.route_backward(lg, ids, np.full((16, 6), 0.75, np.float32), 2.5)
    assert np.all(dl == 0.0)                  # equal dw: sum_j w_j = scale is constant


def test_invalid_ids_zero_row_and_flag():
    lg, ids, dw = _case(4, 8, 2, 5)
    ids = ids.copy()
    ids[1, 0] = -1
    ids[3, 1] = 8
    dl, flags = oracle.route_backward(lg, ids, dw, 1.0)
    assert flags == oracle.FLAG_BAD_EXPERT_ID
    assert np.all(dl[1] == 0.0) and np.all(dl[3] == 0.0)
    assert np.any(dl[0] != 0.0) and np.any(dl[2] != 0.0)


def test_saturated_scores():
    """Logits far out in both tails: the logistic derivative underflows to
    nothing on the negative side and the result still matches autograd."""
    lg, ids, dw = _case(20, 16, 4, 9, spread=30.0)
    dl, _ = oracle.route_backward(lg, ids, dw, 2.5)
    ref, dg = _autograd(lg, ids, dw, 2.5)
    assert np.all(np.isfinite(dl))
    assert _close(dl, ref, dg)
