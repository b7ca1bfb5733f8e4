"""Pins of the oracle's grouped matmul against numpy's fp64 matmul per group
(and, for the backward reading, against torch autograd of the expert FFN's
second matmul: dH = dY W_down is the grouped matmul with W_down^T)."""
import numpy as np
import torch

import oracle


def _bf16(rng, shape, std):
    return (rng.normal(0, std, shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _val(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_matches_numpy_per_group():
    rng = np.random.default_rng(1)
    G, K, N = 4, 128, 96
    counts = [0, 37, 1, 90]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offs[-1]) + 3                        # three rows outside every group
    a = _bf16(rng, (rows, K), 1.0)
    w = _bf16(rng, (G, N, K), 0.1)
    out = oracle.grouped_gemm(a, offs, w, out=np.full((rows, N), 5.0))
    for g in range(G):
        lo, hi = offs[g], offs[g + 1]
        ref = _val(a[lo:hi]) @ _val(w[g]).T
        assert np.allclose(out[lo:hi], ref, rtol=1e-13, atol=1e-13)
    assert np.all(out[offs[-1]:] == 5.0)


def test_is_the_down_projection_input_gradient():
    """For y = h W_down^T (one expert), dL/dh = dy W_down: the grouped matmul
    with the transposed matrix W_down^T ([F, d] -> stored [d, F]^T)."""
    rng = np.random.default_rng(2)
    rows, d, F = 20, 64, 48
    dy = _bf16(rng, (rows, d), 1.0)
    wd = _bf16(rng, (1, d, F), 0.1)                  # W_down [d, F]
    H = torch.zeros((rows, F), dtype=torch.float64, requires_grad=True)
    y = H @ torch.tensor(_val(wd[0])).T
    y.backward(torch.tensor(_val(dy)))
    wdT = np.ascontiguousarray(np.swapaxes(wd, 1, 2))    # [1, F, d]
    dh = oracle.grouped_gemm(dy, np.array([0, rows], np.int32), wdT)
    assert np.allclose(dh, H.grad.numpy(), rtol=1e-13, atol=1e-13)
