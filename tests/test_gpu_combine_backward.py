"""moe_combine_backward against the oracle: the expert-output gradient
w * dy bit for bit (one fp32 rounding of an exact product), the routing
weights' gradient within the bound of its fp32 sums, rows no pair maps to
untouched, invalid dest pairs dropped; up to the 384-expert layer's full
shape (T = 8192, d = 4096, k = 6), checked on sampled tokens."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import host
from sparse_moe_layer_04_amd import ops

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def _dw_bound(dy, yp, dest, d):
    """fp32 error bound of d_topk_w: each thread sums n_p = 4 ceil(d / 1024)
    products by fma, the workgroup adds the 256 partials in an 8-level tree:
    at most (n_p + 8) 2^-24 sum_o |dy y| (the test allows 2 more)."""
    n_p = 4 * -(-d // 1024)
    T, k = dest.shape
    mag = np.zeros((T, k))
    for j in range(k):
        r = dest[:, j]
        ok = r >= 0
        mag[ok, j] = np.sum(np.abs(dy[ok].astype(np.float64) * yp[r[ok]].astype(np.float64)),
                            axis=1)
    return (n_p + 10) * 2.0 ** -24 * mag


@pytest.mark.parametrize("T,d,k,E", [(64, 4096, 6, 384), (100, 1032, 8, 64), (1, 8, 1, 4),
                                     (257, 2048, 6, 64)])
def test_combine_backward(T, d, k, E):
    rng = np.random.default_rng(T + d + k)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    _, _, dest, _, _ = oracle.permute(ids, E)
    dest = dest.reshape(T, k)
    rows = T * k + 5                                   # five rows no pair maps to
    yp = rng.normal(0, 1, (rows, d)).astype(np.float32)
    w = rng.uniform(0, 2.5, (T, k)).astype(np.float32)
    dy = rng.normal(0, 1, (T, d)).astype(np.float32)
    if T > 2:                                          # invalid pairs: dropped
        dest[1, 0] = -1
        dest[2, k - 1] = rows
    init = np.full((rows, d), 7.0, np.float32)
    dyp, dw = ops.combine_backward(torch.from_numpy(dy).to(DEV), torch.from_numpy(yp).to(DEV),
                                   torch.from_numpy(dest).to(DEV), torch.from_numpy(w).to(DEV),
                                   dy_perm=torch.from_numpy(init).to(DEV))
    torch.cuda.synchronize()
    ry, rw = oracle.combine_backward(dy, yp, dest, w, dy_perm=init)
    assert np.array_equal(host(dyp), ry.astype(np.float32))
    valid = np.where((dest >= 0) & (dest < rows), dest, -1)
    assert np.all(host(dw)[valid < 0] == 0.0)
    assert np.all(np.abs(host(dw) - rw) <= _dw_bound(dy, yp, valid, d))


def test_combine_backward_full_size_sampled():
    """The 384-expert layer's shapes (T = 8192, d = 4096, k = 6) on the GPU;
    64 sampled tokens checked against the oracle."""
    T, d, k, E = 8192, 4096, 6, 384
    gen = torch.Generator(device=DEV)
    gen.manual_seed(21)
    logits = torch.randn((T, E), generator=gen, device=DEV)
    ids, w = ops.route(logits, k, 2.5)
    perm = ops.permute(ids, torch.zeros((T, 8), dtype=torch.bfloat16, device=DEV), E)
    dest = perm["dest"].view(T, k)
    yp = torch.randn((T * k, d), generator=gen, device=DEV)
    dy = torch.randn((T, d), generator=gen, device=DEV)
    dyp, dw = ops.combine_backward(dy, yp, dest, w)
    torch.cuda.synchronize()
    tok = np.sort(np.random.default_rng(3).choice(T, 64, replace=False))
    dest_s = host(dest)[tok]
    rows_s = dest_s.ravel()
    # the oracle on the sampled tokens, their source rows renumbered 0 .. 6*64-1
    yp_s = host(yp[torch.from_numpy(rows_s.astype(np.int64)).to(DEV)])
    local = np.arange(rows_s.size, dtype=np.int32).reshape(dest_s.shape)
    ry, rw = oracle.combine_backward(host(dy)[tok], yp_s, local, host(w)[tok])
    got_rows = host(dyp[torch.from_numpy(rows_s.astype(np.int64)).to(DEV)])
    assert np.array_equal(got_rows, ry.astype(np.float32))
    assert np.all(np.abs(host(dw)[tok] - rw) <= _dw_bound(host(dy)[tok], yp_s, local, d))


def test_gather_backward_is_combine_with_unit_weights():
    """The backward of the dispatch gather (x_perm[row] = x[src[row]]) adds
    each token's k row gradients: moe_combine with unit weights and no shared
    term, checked against fp64 autograd of the gather."""
    T, d, k, E = 300, 256, 6, 64
    rng = np.random.default_rng(8)
    ids = torch.from_numpy(np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
                           .astype(np.int32)).to(DEV)
    perm = ops.permute(ids, torch.zeros((T, 8), dtype=torch.bfloat16, device=DEV), E)
    dxp = rng.normal(0, 1, (T * k, d)).astype(np.float32)
    dx = ops.combine(torch.from_numpy(dxp).to(DEV), perm["dest"],
                     torch.ones((T, k), dtype=torch.float32, device=DEV), out_dtype=ops.OUT_F32)
    torch.cuda.synchronize()
    X = torch.zeros((T, d), dtype=torch.float64, requires_grad=True)
    src = torch.from_numpy(host(perm["src"]).astype(np.int64))
    (X[src] * torch.from_numpy(dxp.astype(np.float64))).sum().backward()
    ref = X.grad.numpy()
    mag = np.zeros((T, d))
    np.add.at(mag, host(perm["src"]), np.abs(dxp.astype(np.float64)))
    assert np.all(np.abs(host(dx) - ref) <= k * 2.0 ** -24 * mag)
