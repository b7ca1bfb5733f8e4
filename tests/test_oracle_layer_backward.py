"""Pin of the oracle's whole-layer backward chain (oracle.layer_backward)
against torch fp64 autograd of the layer forward written out in the pages'
order: router projection -> sigmoid scores -> gather of the selected experts'
unbiased scores -> normalise -> scale; per routed pair the clamped-SwiGLU
expert FFN (h rounded to bf16 on the way to the down projection, with the
gradient passed straight through the rounding, as the chain does); the shared
expert; the combine by routing weight.  The expert choice is piecewise
constant in the logits, so autograd runs with the oracle's routes.

x enters the autograd graph as three separate leaves (router, routed experts,
shared expert), so each of the chain's three parts of dx is checked on its
own as well as their sum.

Tolerance: the chain feeds gradients to the products as bf16 (relative error
2^-9 per operand) where autograd stays in fp64, so each gradient is compared
as max |chain - autograd| <= 2e-2 * max |autograd| with a relative Frobenius
error below 5e-3; a wiring mistake (a transposed or swapped operand, a
missing path, a wrong sign) gives errors of order one."""
import numpy as np
import pytest
import torch

import oracle


def _bf16(rng, shape, std):
    return (rng.normal(0, std, shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _v(b):
    return torch.tensor((b.astype(np.uint32) << 16).view(np.float32).astype(np.float64))


def _round_bf16(t):
    b = oracle.round_bf16(t.detach().numpy())
    return _v(b)


def _case(seed, T=16, d=64, E=8, k=2, F=64, Fs=64, xscale=1.0, mode=oracle.MODE_TOPK):
    rng = np.random.default_rng(seed)
    c = dict(T=T, d=d, E=E, k=k, F=F, Fs=Fs, mode=mode)
    c["x"] = _bf16(rng, (T, d), xscale)
    c["w_g"] = _bf16(rng, (E, d), d ** -0.5)
    c["w_gate"] = _bf16(rng, (E, F, d), d ** -0.5)
    c["w_up"] = _bf16(rng, (E, F, d), d ** -0.5)
    c["w_down"] = _bf16(rng, (E, d, F), F ** -0.5)
    c["s_gate"] = _bf16(rng, (Fs, d), d ** -0.5)
    c["s_up"] = _bf16(rng, (Fs, d), d ** -0.5)
    c["s_down"] = _bf16(rng, (d, Fs), Fs ** -0.5)
    c["bias"] = rng.uniform(-0.1, 0.1, (1, E)).astype(np.float32)
    c["dy"] = rng.normal(0, 1, (T, d)).astype(np.float32)
    if mode == oracle.MODE_HASH:
        V = 50
        c["tid2eid"] = np.stack([rng.choice(E, k, replace=False) for _ in range(V)]).astype(np.int32)
        c["input_ids"] = rng.integers(0, V, T).astype(np.int32)
    return c


def _autograd(c, ids, scale, L, cmode):
    T, E, k = c["T"], c["E"], c["k"]
    xr, xe, xs = (_v(c["x"]).requires_grad_() for _ in range(3))
    wg = _v(c["w_g"]).requires_grad_()
    wgate, wup, wdown = (_v(c[n]).requires_grad_() for n in ("w_gate", "w_up", "w_down"))
    sg, su, sd = (_v(c[n]).requires_grad_() for n in ("s_gate", "s_up", "s_down"))
    ids_t = torch.tensor(ids, dtype=torch.int64)

    def clamps(G, U):
        Gc = torch.clamp(G, -L, L) if cmode == 0 else torch.clamp(G, max=L)
        return Gc, torch.clamp(U, -L, L)

    def ffn(xrow, Wg, Wu, Wd):
        Gc, Uc = clamps(xrow @ Wg.T, xrow @ Wu.T)
        h = torch.nn.functional.silu(Gc) * Uc
        h = h + (_round_bf16(h) - h).detach()       # bf16 h, gradient passed through
        return h @ Wd.T

    logits = xr @ wg.T
    s = torch.sigmoid(logits)
    g = s.gather(1, ids_t)
    w = g / g.sum(dim=1, keepdim=True) * scale
    rows = []
    for t in range(T):
        yt = ffn(xs[t], sg, su, sd)
        for j in range(k):
            e = int(ids[t, j])
            yt = yt + w[t, j] * ffn(xe[t], wgate[e], wup[e], wdown[e])
        rows.append(yt)
    y = torch.stack(rows)
    (y * torch.tensor(c["dy"].astype(np.float64))).sum().backward()
    return dict(dx_router=xr.grad, dx_routed=xe.grad, dx_shared=xs.grad,
                dx=xr.grad + xe.grad + xs.grad, dw_g=wg.grad, dw_gate=wgate.grad,
                dw_up=wup.grad, dw_down=wdown.grad, ds_gate=sg.grad, ds_up=su.grad,
                ds_down=sd.grad)


@pytest.mark.parametrize("name,seed,xscale,L,cmode,mode", [
    ("topk", 1, 1.0, 10.0, 0, oracle.MODE_TOPK),
    ("topk-saturating", 2, 30.0, 10.0, 0, oracle.MODE_TOPK),
    ("topk-saturating-gate-upper", 3, 30.0, 10.0, 1, oracle.MODE_TOPK),
    ("hash", 4, 1.0, 10.0, 0, oracle.MODE_HASH),
])
def test_chain_matches_autograd(name, seed, xscale, L, cmode, mode):
    c = _case(seed, xscale=xscale, mode=mode)
    scale = 2.5
    x64 = (c["x"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wg64 = (c["w_g"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    logits = (x64 @ wg64.T).astype(np.float32)
    hashed = mode == oracle.MODE_HASH
    ids, _, _ = oracle.route(logits, c["k"], scale, bias=None if hashed else c["bias"],
                             input_ids=c.get("input_ids"), tid2eid=c.get("tid2eid"), mode=mode)
    got = oracle.layer_backward(c["x"], logits, c["k"], scale, c["w_g"], c["w_gate"], c["w_up"],
                                c["w_down"], c["s_gate"], c["s_up"], c["s_down"], c["dy"], L,
                                cmode, bias=None if hashed else c["bias"],
                                input_ids=c.get("input_ids"), tid2eid=c.get("tid2eid"),
                                mode=mode)
    ref = _autograd(c, ids, scale, L, cmode)
    for key, r in ref.items():
        r = r.numpy()
        gk = got[key]
        scale_ref = np.abs(r).max()
        assert scale_ref > 0, key
        err = np.abs(gk - r).max()
        fro = np.linalg.norm(gk - r) / np.linalg.norm(r)
        assert err <= 2e-2 * scale_ref and fro <= 5e-3, (key, err / scale_ref, fro)
