"""ctypes marshalling for the C oracle (moe_oracle.c).  TEST INFRASTRUCTURE ONLY.

Arrays are numpy; bf16 tensors travel as their uint16 bit patterns.  No
arithmetic of the method lives here: every function forwards to the C
definition of the same name (``orc_*``), except ``forward``, which only
chains those calls in the pages' order (route -> permute -> gather -> expert
FFN -> shared FFN -> combine).
"""
import ctypes
import os

import numpy as np

MODE_TOPK = 0
MODE_HASH = 1
FLAG_BAD_INPUT_ID = 1
FLAG_BAD_EXPERT_ID = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    # MOE_ORACLE_LIBRARY: another build of the same source (the sanitizer
    # build of tests/test_sanitizers.py)
    return os.environ.get("MOE_ORACLE_LIBRARY", os.path.join(_HERE, "libmoe_oracle.so"))


def load():
    """Load (building first if absent) the oracle shared library."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    I64 = ctypes.c_int64
    F = ctypes.c_float
    D = ctypes.c_double
    lib.orc_f64_to_bf16.argtypes = [D]
    lib.orc_f64_to_bf16.restype = ctypes.c_uint16
    lib.orc_score.argtypes = [F]
    lib.orc_score.restype = F
    lib.orc_score_array.argtypes = [P, P, I64]
    lib.orc_score_array.restype = None
    lib.orc_gate_logits.argtypes = [P, P, P, I, I, I, P]
    lib.orc_gate_logits.restype = None
    lib.orc_route.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, P, P]
    lib.orc_route.restype = ctypes.c_uint
    lib.orc_route_backward.argtypes = [P, P, P, I, I, I, F, P]
    lib.orc_route_backward.restype = ctypes.c_uint
    lib.orc_permute.argtypes = [P, I, I, I, P, P, P, P]
    lib.orc_permute.restype = ctypes.c_uint
    lib.orc_gather.argtypes = [P, P, I64, I, P]
    lib.orc_gather.restype = None
    lib.orc_expert_ffn.argtypes = [P, P, I, I, I, P, P, P, D, I, P, P]
    lib.orc_expert_ffn.restype = None
    lib.orc_expert_ffn_rows.argtypes = [P, P, P, I, I, I, P, P, P, D, I, P, P]
    lib.orc_expert_ffn_rows.restype = None
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = D
    lib.orc_e4m3_encode.argtypes = [D]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_quant_mxfp8.argtypes = [P, I64, I, P, P]
    lib.orc_quant_mxfp8.restype = None
    lib.orc_dequant_mxfp8.argtypes = [P, P, I64, I, P]
    lib.orc_dequant_mxfp8.restype = None
    lib.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e2m1_decode.restype = D
    lib.orc_e2m1_encode.argtypes = [D]
    lib.orc_e2m1_encode.restype = ctypes.c_uint8
    lib.orc_quant_mxfp4.argtypes = [P, I64, I, P, P]
    lib.orc_quant_mxfp4.restype = None
    lib.orc_dequant_mxfp4.argtypes = [P, P, I64, I, P]
    lib.orc_dequant_mxfp4.restype = None
    lib.orc_combine.argtypes = [P, P, P, P, I, I, I, P]
    lib.orc_combine.restype = None
    lib.orc_combine_backward.argtypes = [P, P, P, P, I, I, I, I, P, P]
    lib.orc_swiglu_backward.argtypes = [P, P, P, I64, D, I, P, P]
    lib.orc_grouped_gemm.argtypes = [P, P, I, I, I, P, P]
    lib.orc_grouped_gemm.restype = None
    lib.orc_router_backward.argtypes = [P, P, P, I, I, I, P, P]
    lib.orc_router_backward.restype = None
    lib.orc_round_bf16_array.argtypes = [P, I64, P]
    lib.orc_round_bf16_array.restype = None
    lib.orc_add_f64.argtypes = [P, P, I64, P]
    lib.orc_add_f64.restype = None
    lib.orc_grouped_wgrad.argtypes = [P, P, P, I, I, I, P]
    lib.orc_grouped_wgrad.restype = None
    lib.orc_grouped_wgrad_entries.argtypes = [P, P, P, I, I, P, P, P, I64, P]
    lib.orc_grouped_wgrad_entries.restype = None
    lib.orc_swiglu_backward.restype = None
    lib.orc_combine_backward.restype = None
    lib.orc_tokens_forward.argtypes = [P, P, I, I, I, I, P, P, P, P, P, P, P, P, I, D, I, P]
    lib.orc_tokens_forward.restype = None
    _LIB = lib
    return lib


def _c(a, dtype):
    """Contiguous array of the given dtype (None passes through)."""
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data


def _bf16(a):
    """bf16 payload as uint16 bits (accepts uint16 arrays or torch bf16 tensors)."""
    if a is None:
        return None
    if hasattr(a, "view") and hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        import torch
        return a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 arrays are passed as uint16 bit patterns")
    return np.ascontiguousarray(a)


def f64_to_bf16(v: float) -> int:
    return int(load().orc_f64_to_bf16(float(v)))


def score(x):
    """Pinned binary32 sigmoid S(x), elementwise."""
    x = _c(x, np.float32)
    out = np.empty_like(x)
    load().orc_score_array(_p(x), _p(out), x.size)
    return out


def gate_logits(x, wg, off=None):
    x, wg, off = _bf16(x), _bf16(wg), _c(off, np.float32)
    T, d = x.shape
    E = wg.shape[0]
    out = np.empty((T, E), np.float32)
    load().orc_gate_logits(_p(x), _p(wg), _p(off), T, d, E, _p(out))
    return out


def route(logits, k, scale, bias=None, modality=None, input_ids=None, tid2eid=None,
          mode=MODE_TOPK):
    """Returns (ids[T,k] int32, w[T,k] float32, flags)."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    bias = _c(bias, np.float32)
    if bias is not None:
        bias = bias.reshape(-1, E)
    n_bias = 0 if bias is None else bias.shape[0]
    modality = _c(modality, np.uint8)
    input_ids = _c(input_ids, np.int32)
    tid2eid = _c(tid2eid, np.int32)
    V = 0 if tid2eid is None else tid2eid.shape[0]
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    flags = load().orc_route(_p(logits), _p(bias), _p(modality), _p(input_ids), _p(tid2eid),
                             T, E, k, n_bias, V, mode, float(scale), _p(ids), _p(w))
    return ids, w, int(flags)


def route_backward(logits, ids, dw, scale):
    """Gradient of the routing weights w.r.t. the logits (orc_route_backward):
    returns (dlogits[T,E] float64, flags)."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = _c(ids, np.int32)
    dw = _c(dw, np.float32)
    k = ids.shape[1]
    assert ids.shape == (T, k) and dw.shape == (T, k) and k <= 64
    dl = np.empty((T, E), np.float64)
    flags = load().orc_route_backward(_p(logits), _p(ids), _p(dw), T, E, k, float(scale), _p(dl))
    return dl, int(flags)


def permute(ids, E):
    """Returns (counts[E], offsets[E+1], dest[T*k], src[T*k], flags)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    dest = np.empty(T * k, np.int32)
    src = np.empty(T * k, np.int32)
    flags = load().orc_permute(_p(ids), T, k, E, _p(counts), _p(offsets), _p(dest), _p(src))
    return counts, offsets, dest, src, int(flags)


def gather(x, src):
    x = _bf16(x)
    src = _c(src, np.int32)
    rows = src.shape[0]
    d = x.shape[1]
    out = np.zeros((rows, d), np.uint16)
    load().orc_gather(_p(x), _p(src), rows, d, _p(out))
    return out


def expert_ffn(a, offsets, w_gate, w_up, w_down, clamp_limit, clamp_mode=0):
    """Grouped FFN. Returns (h[rows,F] uint16 bf16 bits, y[rows,d] float64)."""
    a = _bf16(a)
    offsets = _c(offsets, np.int32)
    w_gate, w_up, w_down = _bf16(w_gate), _bf16(w_up), _bf16(w_down)
    G = offsets.shape[0] - 1
    rows, d = a.shape
    F = w_gate.shape[-2]
    h = np.zeros((rows, F), np.uint16)
    y = np.zeros((rows, d), np.float64)
    load().orc_expert_ffn(_p(a), _p(offsets), G, d, F, _p(w_gate), _p(w_up), _p(w_down),
                          float(clamp_limit), int(clamp_mode), _p(h), _p(y))
    return h, y


def expert_ffn_rows(a, rows, experts, w_gate, w_up, w_down, clamp_limit, clamp_mode=0):
    """FFN of a[rows[i]] through expert experts[i]; returns packed (h, y)."""
    a = _bf16(a)
    rows = _c(rows, np.int64)
    experts = _c(experts, np.int32)
    w_gate, w_up, w_down = _bf16(w_gate), _bf16(w_up), _bf16(w_down)
    n = rows.shape[0]
    d = a.shape[1]
    F = w_gate.shape[-2]
    h = np.zeros((n, F), np.uint16)
    y = np.zeros((n, d), np.float64)
    load().orc_expert_ffn_rows(_p(a), _p(rows), _p(experts), n, d, F, _p(w_gate), _p(w_up),
                               _p(w_down), float(clamp_limit), int(clamp_mode), _p(h), _p(y))
    return h, y


def combine_backward(dy, y_perm, dest, w, dy_perm=None):
    """Backward of the combine (orc_combine_backward): returns
    (dy_perm[rows,d] float64, dw[T,k] float64); rows no pair maps to keep the
    values of `dy_perm` (zeros if None)."""
    dy = _c(dy, np.float32)
    y_perm = _c(y_perm, np.float32)
    dest = _c(dest, np.int32)
    w = _c(w, np.float32)
    T, k = w.shape
    rows, d = y_perm.shape
    assert dy.shape == (T, d) and dest.size == T * k
    out = np.zeros((rows, d), np.float64) if dy_perm is None else _c(dy_perm, np.float64).copy()
    dw = np.empty((T, k), np.float64)
    load().orc_combine_backward(_p(dy), _p(y_perm), _p(dest), _p(w), T, d, k, rows, _p(out),
                                _p(dw))
    return out, dw


def grouped_gemm(a, offsets, w, out=None):
    """out[r] = a[r] @ w[g].T for the rows of group g (bf16 bits in, fp64
    out); rows outside every group keep `out`'s values (zeros if None)."""
    a = _bf16(a)
    offsets = _c(offsets, np.int32)
    w = _bf16(w)
    G, N, K = w.shape
    rows = a.shape[0]
    assert a.shape[1] == K and offsets.shape == (G + 1,)
    res = np.zeros((rows, N), np.float64) if out is None else _c(out, np.float64).copy()
    load().orc_grouped_gemm(_p(a), _p(offsets), G, K, N, _p(w), _p(res))
    return res


def router_backward(dl, x, wg):
    """(dx[T,d], dwg[E,d]) float64: gradients of l = x w_g^T for dl[T,E]."""
    dl = _c(dl, np.float64)
    x, wg = _bf16(x), _bf16(wg)
    T, E = dl.shape
    d = x.shape[1]
    dx = np.empty((T, d), np.float64)
    dwg = np.empty((E, d), np.float64)
    load().orc_router_backward(_p(dl), _p(x), _p(wg), T, d, E, _p(dx), _p(dwg))
    return dx, dwg


def round_bf16(v):
    """float64 values rounded to bf16 (nearest even), returned as bits."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    load().orc_round_bf16_array(_p(v), v.size, _p(out))
    return out


def add(a, b):
    """a + b (float64), elementwise."""
    a, b = _c(a, np.float64), _c(b, np.float64)
    assert a.shape == b.shape
    out = np.empty(a.shape, np.float64)
    load().orc_add_f64(_p(a), _p(b), a.size, _p(out))
    return out


def _t(w):
    """[G, N, K] bf16 bits -> [G, K, N] (the transposed matrices; data movement)."""
    return np.ascontiguousarray(np.swapaxes(_bf16(w), -1, -2))


def layer_backward(x, logits, k, scale, w_g, w_gate, w_up, w_down, s_gate, s_up, s_down, dy,
                   clamp_limit=10.0, clamp_mode=0, bias=None, modality=None, input_ids=None,
                   tid2eid=None, mode=MODE_TOPK, weight_grads=True):
    """Gradients of the whole layer for an output gradient dy[T,d] (fp32),
    chaining the pinned backward pieces in the reverse order of the forward.
    The forward's values come from `forward` (routes from the given logits).
    Gradients enter the matrix products as bf16 (round_bf16) and the fp32
    intermediates of the GPU path (expert outputs, pre-activations, their
    gradients, the routing-weight gradient) are passed as fp32, so the chain
    follows the precision at which each product is taken.  Returns a dict:
    dx, dw_g, dw_gate, dw_up, dw_down, ds_gate, ds_up, ds_down (float64) and
    dx_routed, dx_shared, dx_router (the three parts of dx).  With
    weight_grads=False the expert weight gradients are skipped (each token's
    dx depends only on that token, so dx can be checked on a token subset)."""
    x = _bf16(x)
    T, d = x.shape
    f = forward(x, logits, k, scale, w_gate, w_up, w_down, s_gate, s_up, s_down, clamp_limit,
                clamp_mode, bias, modality, input_ids, tid2eid, mode)
    w_gate, w_up, w_down = _bf16(w_gate), _bf16(w_up), _bf16(w_down)
    offs, dest, h, xp = f["offsets"], f["dest"], f["h"], f["x_perm"]
    dy = _c(dy, np.float32)
    out = {}
    # combine: y = ysh + sum_j w_j y_perm[dest_j]
    dyp, dtw = combine_backward(dy, f["y_perm"], dest, f["w"])
    dyp16 = round_bf16(dyp)
    # down projection y_perm = h W_down^T
    if weight_grads:
        out["dw_down"] = grouped_wgrad(dyp16, h, offs)
    dh = grouped_gemm(dyp16, offs, _t(w_down))
    # clamped SwiGLU h = silu(cg(G)) cu(U), G = x_perm W_gate^T, U = x_perm W_up^T
    G = grouped_gemm(xp, offs, w_gate)
    U = grouped_gemm(xp, offs, w_up)
    dG, dU = swiglu_backward(G, U, dh, clamp_limit, clamp_mode)
    dG16, dU16 = round_bf16(dG), round_bf16(dU)
    if weight_grads:
        out["dw_gate"] = grouped_wgrad(dG16, xp, offs)
        out["dw_up"] = grouped_wgrad(dU16, xp, offs)
    dxp = grouped_gemm(np.concatenate([dG16, dU16], axis=1), offs,
                       _t(np.concatenate([w_gate, w_up], axis=1)))
    # dispatch: x_perm[row] = x[src[row]]; its backward sums each token's rows
    out["dx_routed"] = combine(dxp, dest, np.ones((T, k), np.float32))
    # routing weights -> logits -> router projection
    dl, _ = route_backward(logits, f["ids"], dtw, scale)
    out["dx_router"], out["dw_g"] = router_backward(dl, x, w_g)
    # shared expert on x (none: no shared gradients, no dx part)
    if s_gate is None:
        out["dx_shared"] = np.zeros((T, d), np.float64)
        out["dx"] = add(out["dx_routed"], out["dx_router"])
        return out
    sg, su, sd = _bf16(s_gate), _bf16(s_up), _bf16(s_down)
    one = np.array([0, T], np.int32)
    hs, _ = expert_ffn(x, one, sg[None], su[None], sd[None], clamp_limit, clamp_mode)
    dy16 = round_bf16(dy)
    if weight_grads:
        out["ds_down"] = grouped_wgrad(dy16, hs, one)[0]
    dhs = grouped_gemm(dy16, one, _t(sd[None]))
    Gs = grouped_gemm(x, one, sg[None])
    Us = grouped_gemm(x, one, su[None])
    dGs, dUs = swiglu_backward(Gs, Us, dhs, clamp_limit, clamp_mode)
    dGs16, dUs16 = round_bf16(dGs), round_bf16(dUs)
    if weight_grads:
        out["ds_gate"] = grouped_wgrad(dGs16, x, one)[0]
        out["ds_up"] = grouped_wgrad(dUs16, x, one)[0]
    out["dx_shared"] = grouped_gemm(np.concatenate([dGs16, dUs16], axis=1), one,
                                    _t(np.concatenate([sg, su], axis=0)[None]))
    out["dx"] = add(add(out["dx_routed"], out["dx_shared"]), out["dx_router"])
    return out


def grouped_wgrad(dy, a, offsets):
    """dw[g] = dy[rows of g]^T a[rows of g] (fp64) for bf16 dy [rows, M] and
    a [rows, K]: the weight gradient of out = a W_g^T per group."""
    dy, a = _bf16(dy), _bf16(a)
    offsets = _c(offsets, np.int32)
    G = offsets.shape[0] - 1
    M, K = dy.shape[1], a.shape[1]
    dw = np.empty((G, M, K), np.float64)
    load().orc_grouped_wgrad(_p(dy), _p(a), _p(offsets), G, M, K, _p(dw))
    return dw


def grouped_wgrad_entries(dy, a, offsets, g, m, k):
    """grouped_wgrad at the listed entries (g[i], m[i], k[i]) only."""
    dy, a = _bf16(dy), _bf16(a)
    offsets = _c(offsets, np.int32)
    g, m, k = _c(g, np.int32), _c(m, np.int32), _c(k, np.int32)
    out = np.empty(g.shape[0], np.float64)
    load().orc_grouped_wgrad_entries(_p(dy), _p(a), _p(offsets), dy.shape[1], a.shape[1], _p(g),
                                     _p(m), _p(k), g.shape[0], _p(out))
    return out


def swiglu_backward(gate, up, dh, clamp_limit, clamp_mode=0):
    """Backward of the clamped SwiGLU (orc_swiglu_backward): returns
    (dgate, dup) float64 arrays of the inputs' shape."""
    gate = _c(gate, np.float32)
    up = _c(up, np.float32)
    dh = _c(dh, np.float32)
    assert gate.shape == up.shape == dh.shape
    dg = np.empty(gate.shape, np.float64)
    du = np.empty(gate.shape, np.float64)
    load().orc_swiglu_backward(_p(gate), _p(up), _p(dh), gate.size, float(clamp_limit),
                               int(clamp_mode), _p(dg), _p(du))
    return dg, du


def combine(y_perm, dest, w, ysh=None):
    y_perm = _c(y_perm, np.float64)
    dest = _c(dest, np.int32)
    w = _c(w, np.float32)
    T, k = w.shape
    d = y_perm.shape[1]
    ysh = _c(ysh, np.float64)
    y = np.empty((T, d), np.float64)
    load().orc_combine(_p(y_perm), _p(dest), _p(w), _p(ysh), T, d, k, _p(y))
    return y


def tokens_forward(x, tokens, ids, w, w_gate, w_up, w_down, s_gate, s_up, s_down,
                   clamp_limit, clamp_mode=0):
    """Layer output for the listed tokens from their routing (ids, w)."""
    x = _bf16(x)
    tokens = _c(tokens, np.int64)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    w_gate, w_up, w_down = _bf16(w_gate), _bf16(w_up), _bf16(w_down)
    s_gate, s_up, s_down = _bf16(s_gate), _bf16(s_up), _bf16(s_down)
    n = tokens.shape[0]
    d = x.shape[1]
    k = ids.shape[1]
    F = w_gate.shape[-2]
    Fs = 0 if s_gate is None else s_gate.shape[0]
    y = np.empty((n, d), np.float64)
    load().orc_tokens_forward(_p(x), _p(tokens), n, d, F, k, _p(ids), _p(w), _p(w_gate),
                              _p(w_up), _p(w_down), _p(s_gate), _p(s_up), _p(s_down), Fs,
                              float(clamp_limit), int(clamp_mode), _p(y))
    return y


def forward(x, logits, k, scale, w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None,
            clamp_limit=10.0, clamp_mode=0, bias=None, modality=None, input_ids=None,
            tid2eid=None, mode=MODE_TOPK):
    """Whole layer from given router logits, step by step.

    Returns a dict with ids, w, counts, offsets, dest, src, x_perm, h, y_perm,
    ysh, y (y and y_perm in fp64, h in bf16 bits) and the flag word.
    """
    x = _bf16(x)
    E = np.asarray(logits).shape[1]
    ids, w, f1 = route(logits, k, scale, bias, modality, input_ids, tid2eid, mode)
    counts, offsets, dest, src, f2 = permute(ids, E)
    x_perm = gather(x, src)
    h, y_perm = expert_ffn(x_perm, offsets, w_gate, w_up, w_down, clamp_limit, clamp_mode)
    ysh = None
    if s_gate is not None:
        T = x.shape[0]
        _, ysh = expert_ffn(x, np.array([0, T], np.int32), _bf16(s_gate)[None],
                            _bf16(s_up)[None], _bf16(s_down)[None], clamp_limit, clamp_mode)
    y = combine(y_perm, dest, w, ysh)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, dest=dest, src=src,
                x_perm=x_perm, h=h, y_perm=y_perm, ysh=ysh, y=y, flags=f1 | f2)


def quant_dequant_mxfp8(a):
    """bf16 bits [..., K] -> their MXFP8 values (quantise along K in blocks of
    32, then dequantise) as bf16 bits; exact (see orc_quant_mxfp8)."""
    q, x = quant_mxfp8(a)
    return dequant_mxfp8(q, x)


def forward_a8w4(x, logits, k, scale, w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None,
                 clamp_limit=10.0, clamp_mode=0, bias=None, modality=None, input_ids=None,
                 tid2eid=None, mode=MODE_TOPK):
    """Whole layer in the A8W4 reading ("CANN DeepSeek-V4 training
    optimisation", outlook, functional-expansion bullets: FP8 and A8W4
    low-precision training on MxFP8 / MxFP4): the routed experts' weights are
    given as their (dequantised) MXFP4 values and both routed expert matmuls
    take MXFP8 activations: each token's row of x is quantised along d before
    gate/up, each row of h (the bf16 SwiGLU output) along F before down.  The
    router, routing, dispatch, the shared expert (bf16, on x itself) and the
    combine are those of forward().  Returns forward()'s dict plus x8 (the
    quantised x, bf16 bits) and h8 (the quantised h)."""
    x = _bf16(x)
    E = np.asarray(logits).shape[1]
    ids, w, f1 = route(logits, k, scale, bias, modality, input_ids, tid2eid, mode)
    counts, offsets, dest, src, f2 = permute(ids, E)
    x8 = quant_dequant_mxfp8(x)
    x_perm = gather(x8, src)
    h, _ = expert_ffn(x_perm, offsets, w_gate, w_up, w_down, clamp_limit, clamp_mode)
    h8 = quant_dequant_mxfp8(h)
    y_perm = grouped_gemm(h8, offsets, w_down)
    ysh = None
    if s_gate is not None:
        T = x.shape[0]
        _, ysh = expert_ffn(x, np.array([0, T], np.int32), _bf16(s_gate)[None],
                            _bf16(s_up)[None], _bf16(s_down)[None], clamp_limit, clamp_mode)
    y = combine(y_perm, dest, w, ysh)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, dest=dest, src=src,
                x_perm=x_perm, x8=x8, h=h, h8=h8, y_perm=y_perm, ysh=ysh, y=y, flags=f1 | f2)


def tokens_forward_a8w4(x, tokens, ids, w, w_gate, w_up, w_down, s_gate, s_up, s_down,
                        clamp_limit, clamp_mode=0):
    """forward_a8w4's output for the listed tokens from their routing (ids,
    w): the token's quantised row through each of its k experts, h quantised,
    the down products combined with the routing weights in slot order in
    fp64, plus the shared expert on the unquantised row."""
    x = _bf16(x)
    tokens = _c(tokens, np.int64)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    n, k = tokens.shape[0], ids.shape[1]
    E = _bf16(w_gate).shape[0]
    x8 = quant_dequant_mxfp8(x[tokens])
    # (token, slot) pairs grouped by expert (valid ids only)
    pt = np.repeat(np.arange(n), k)
    pe = ids[tokens].reshape(-1)
    ok = (pe >= 0) & (pe < E)
    order = np.argsort(np.where(ok, pe, E), kind="stable")[: int(ok.sum())]
    counts = np.bincount(pe[order], minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = x8[pt[order]]
    h, _ = expert_ffn(a, offsets, w_gate, w_up, w_down, clamp_limit, clamp_mode)
    yp = grouped_gemm(quant_dequant_mxfp8(h), offsets, w_down)
    y_pair = np.zeros((n * k, x.shape[1]), np.float64)
    y_pair[order] = yp
    wt = np.where(ok, w[tokens].reshape(-1).astype(np.float64), 0.0)
    y = np.zeros((n, x.shape[1]), np.float64)
    for j in range(k):
        y += wt[j::k, None] * y_pair[j::k]
    if s_gate is not None:
        _, ysh = expert_ffn(x[tokens], np.array([0, n], np.int32), _bf16(s_gate)[None],
                            _bf16(s_up)[None], _bf16(s_down)[None], clamp_limit, clamp_mode)
        y += ysh
    return y


def e4m3_decode(code):
    """Value of an E4M3 code (float; NaN for S.1111.111)."""
    return float(load().orc_e4m3_decode(int(code)))


def e4m3_encode(v):
    """E4M3 code of v (round to nearest even, saturating)."""
    return int(load().orc_e4m3_encode(float(v)))


def quant_mxfp8(w):
    """bf16 bits [..., K] -> (codes uint8 [..., K], block exponents int32 [..., K/32])."""
    w = _c(w, np.uint16)
    K = w.shape[-1]
    R = w.size // K
    q = np.empty(w.shape, np.uint8)
    x = np.empty(w.shape[:-1] + (K // 32,), np.int32)
    load().orc_quant_mxfp8(_p(w), R, K, _p(q), _p(x))
    return q, x


def dequant_mxfp8(q, x):
    """(codes [..., K], block exponents [..., K/32]) -> dequantised weights as bf16 bits."""
    q = _c(q, np.uint8)
    x = _c(x, np.int32)
    K = q.shape[-1]
    w = np.empty(q.shape, np.uint16)
    load().orc_dequant_mxfp8(_p(q), _p(x), q.size // K, K, _p(w))
    return w


def e2m1_decode(code):
    """Value of an E2M1 code (0..15)."""
    return float(load().orc_e2m1_decode(int(code)))


def e2m1_encode(v):
    """E2M1 code of v (nearest, ties to the even code, saturating)."""
    return int(load().orc_e2m1_encode(float(v)))


def quant_mxfp4(w):
    """bf16 bits [..., K] -> (codes uint8 [..., K], block exponents int32 [..., K/32])."""
    w = _c(w, np.uint16)
    K = w.shape[-1]
    q = np.empty(w.shape, np.uint8)
    x = np.empty(w.shape[:-1] + (K // 32,), np.int32)
    load().orc_quant_mxfp4(_p(w), w.size // K, K, _p(q), _p(x))
    return q, x


def dequant_mxfp4(q, x):
    """(codes [..., K], block exponents [..., K/32]) -> dequantised weights as bf16 bits."""
    q = _c(q, np.uint8)
    x = _c(x, np.int32)
    K = q.shape[-1]
    w = np.empty(q.shape, np.uint16)
    load().orc_dequant_mxfp4(_p(q), _p(x), q.size // K, K, _p(w))
    return w
