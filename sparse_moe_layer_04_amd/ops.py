"""Python binding of the C-ABI MoE library (``libmoe_hip.so``).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory and the current HIP stream.  There is
no fallback: if the library is missing or a call fails, an exception is
raised.
"""
import ctypes
import os
import re

import torch

MODE_TOPK = 0
MODE_HASH = 1
OUT_BF16 = 0
OUT_F32 = 1
CLAMP_SYMMETRIC = 0
CLAMP_GATE_UPPER = 1
FLAG_BAD_INPUT_ID = 1
FLAG_BAD_EXPERT_ID = 2
FORWARD_STAGES = 8
STAGE_NAMES = ("router_gemm", "route", "permute", "gate_up_routed", "gate_up_shared",
               "down_routed", "down_shared", "combine")

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
HEADER = os.path.join(_ROOT, "include", "moe.h")
# the in-tree build; MOE_HIP_LIBRARY may point at another build of the same sources
LIBRARY = os.environ.get("MOE_HIP_LIBRARY", os.path.join(_HERE, "libmoe_hip.so"))

_lib = None


class MoeError(RuntimeError):
    pass


class MoeCfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int), ("d", ctypes.c_int), ("E", ctypes.c_int),
                ("k", ctypes.c_int), ("F", ctypes.c_int), ("F_shared", ctypes.c_int),
                ("mode", ctypes.c_int), ("n_bias", ctypes.c_int), ("V", ctypes.c_int),
                ("scale", ctypes.c_float), ("clamp_limit", ctypes.c_float),
                ("clamp_mode", ctypes.c_int), ("out_dtype", ctypes.c_int)]


WEIGHT_NAMES = ("w_g", "logit_offset", "score_bias", "tid2eid", "w_gate", "w_up", "w_down",
                "s_gate", "s_up", "s_down", "w_gate_scale", "w_up_scale", "w_down_scale")
# moe_weights.packed values of MXFP8 / MXFP4 routed-expert weights
WEIGHTS_FP8 = 2
WEIGHTS_FP4 = 3
WEIGHTS_A8W4 = 4
MATRIX_NAMES = ("w_g", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")


class MoeWeights(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_int)] + [(n, ctypes.c_void_p) for n in WEIGHT_NAMES]


BWD_WEIGHT_NAMES = ("w_g", "w_down_t", "w_gu_t", "s_down_t", "s_gu_t")
GRAD_NAMES = ("dx", "dw_g", "dw_gate", "dw_up", "dw_down", "ds_gate", "ds_up", "ds_down")


class MoeBwdWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BWD_WEIGHT_NAMES]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_NAMES]


def declared_functions():
    """Names of the functions include/moe.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise MoeError(f"{LIBRARY} is missing: build it with sparse_moe_layer_04_amd/build.py")
    L = ctypes.CDLL(LIBRARY)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.moe_status_string.argtypes = [I]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_gate_logits.argtypes = [P, P, P, I, I, I, P, P]
    L.moe_route.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, P, P, P, P]
    L.moe_route_backward.argtypes = [P, P, P, I, I, I, F, P, P, P]
    L.moe_combine_backward.argtypes = [P, P, P, P, I, I, I, I, P, P, P]
    L.moe_swiglu_backward.argtypes = [P, P, P, ctypes.c_int64, F, I, P, P, P]
    L.moe_grouped_gemm_packed.argtypes = [P, P, I, I, I, I, P, P, P]
    L.moe_grouped_wgrad.argtypes = [P, P, P, I, I, I, I, P, P]
    L.moe_permute_workspace_size.argtypes = [I, I, I]
    L.moe_permute_workspace_size.restype = S
    L.moe_permute.argtypes = [P, P, I, I, I, I, P, P, P, P, P, P, P, S, P]
    L.moe_permute_noalloc.argtypes = [P, P, I, I, I, I, P, P, P, P, P, P, P]
    L.moe_expert_ffn.argtypes = [P, P, I, I, I, I, P, P, P, F, I, P, P, P]
    L.moe_expert_ffn_packed.argtypes = L.moe_expert_ffn.argtypes
    L.moe_combine.argtypes = [P, P, P, P, I, I, I, I, I, P, P]
    L.moe_packed_weight_bytes.argtypes = [I, I, I, I]
    L.moe_packed_weight_bytes.restype = S
    L.moe_pack_weights.argtypes = [P, I, I, I, I, P, P]
    L.moe_packed_fp8_weight_bytes.argtypes = [I, I, I, I]
    L.moe_packed_fp8_weight_bytes.restype = S
    L.moe_packed_fp8_scale_bytes.argtypes = [I, I, I, I]
    L.moe_packed_fp8_scale_bytes.restype = S
    L.moe_pack_weights_fp8.argtypes = [P, I, I, I, I, P, P, P]
    L.moe_packed_fp4_weight_bytes.argtypes = [I, I, I, I]
    L.moe_packed_fp4_weight_bytes.restype = S
    L.moe_pack_weights_fp4.argtypes = [P, I, I, I, I, P, P, P]
    L.moe_quantize_mxfp8.argtypes = [P, ctypes.c_longlong, I, P, P, P]
    L.moe_expert_ffn_a8w4.argtypes = [P, P, P, I, I, I, I, P, P, P, P, P, P, F, I, P, P, P, P]
    L.moe_forward_workspace_size.argtypes = [ctypes.POINTER(MoeCfg)]
    L.moe_forward_workspace_size.restype = S
    L.moe_workspace_size.argtypes = [ctypes.POINTER(MoeCfg)]
    L.moe_workspace_size.restype = S
    L.moe_read_error_flags.argtypes = [P, P, ctypes.POINTER(ctypes.c_uint32)]
    L.moe_forward.argtypes = [ctypes.POINTER(MoeCfg), ctypes.POINTER(MoeWeights), P, P, P, P,
                              P, P, P, P, P, S, P]
    L.moe_forward_timed.argtypes = L.moe_forward.argtypes + [P]
    L.moe_backward_workspace_size.argtypes = [ctypes.POINTER(MoeCfg)]
    L.moe_backward_workspace_size.restype = S
    L.moe_backward.argtypes = [ctypes.POINTER(MoeCfg), ctypes.POINTER(MoeWeights),
                               ctypes.POINTER(MoeBwdWeights), P, P, P, P,
                               ctypes.POINTER(MoeGrads), P, P, S, P]
    for name in ("moe_gate_logits", "moe_route", "moe_permute", "moe_expert_ffn",
                 "moe_expert_ffn_packed",
                 "moe_combine", "moe_forward", "moe_forward_timed", "moe_pack_weights",
                 "moe_pack_weights_fp8", "moe_pack_weights_fp4", "moe_quantize_mxfp8",
                 "moe_expert_ffn_a8w4"):
        getattr(L, name).restype = I
    _lib = L
    return L


def read_error_flags(flags):
    """The device error-flag word (MOE_FLAG_* bits) after the work queued on
    the current stream so far (moe_read_error_flags: synchronises with the
    stream)."""
    _need(flags, torch.int32, "flags", shape=(1,))
    out = ctypes.c_uint32(0)
    _check(lib().moe_read_error_flags(_ptr(flags), _stream(), ctypes.byref(out)),
           "moe_read_error_flags")
    return int(out.value)


def _check(status, what):
    if status != 0:
        msg = lib().moe_status_string(status).decode()
        raise MoeError(f"{what} failed: {msg} ({status})")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _need(t, dtype, name, dims=None, shape=None):
    """Checks a tensor handed to the library as a raw pointer: device,
    dtype, contiguity, rank and (None entries match any size) shape.  The
    kernels trust these sizes, so a mismatch is an error here rather than an
    out-of-bounds access on the device."""
    if t is None:
        raise MoeError(f"{name} is required")
    if not t.is_cuda:
        raise MoeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise MoeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    if dims is not None and t.dim() != dims:
        raise MoeError(f"{name} must have {dims} dims")
    if shape is not None and (t.dim() != len(shape) or
                              any(s is not None and s != n for s, n in zip(shape, t.shape))):
        want = "[" + ", ".join("*" if s is None else str(s) for s in shape) + "]"
        raise MoeError(f"{name} must be {want}, got {list(t.shape)}")
    return t


def _opt(t, dtype, name, shape=None):
    return None if t is None else _need(t, dtype, name, shape=shape)


def _out(t, dtype, name, shape, device):
    """An output tensor: allocated when None, else checked like an input."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _need(t, dtype, name, shape=shape)


def _flags(flags):
    return _opt(flags, torch.int32, "flags", shape=(1,))


def gate_logits(x, w_g, logit_offset=None, out=None):
    """logits[T,E] fp32 = x[T,d] @ w_g[E,d]^T (+ logit_offset[E])."""
    _need(x, torch.bfloat16, "x", 2)
    T, d = x.shape
    _need(w_g, torch.bfloat16, "w_g", shape=(None, d))
    E = w_g.shape[0]
    _opt(logit_offset, torch.float32, "logit_offset", shape=(E,))
    out = _out(out, torch.float32, "out", (T, E), x.device)
    _check(lib().moe_gate_logits(_ptr(x), _ptr(w_g), _ptr(logit_offset), T, d, E, _ptr(out),
                                 _stream()), "moe_gate_logits")
    return out


def route(logits, k, scale, score_bias=None, modality=None, input_ids=None, tid2eid=None,
          mode=MODE_TOPK, flags=None, ids=None, w=None):
    """Returns (topk_ids[T,k] int32, topk_w[T,k] fp32)."""
    _need(logits, torch.float32, "logits", 2)
    T, E = logits.shape
    if score_bias is not None and score_bias.dim() == 1:
        if score_bias.numel() % E:
            raise MoeError(f"score_bias must hold whole rows of E = {E} values")
        score_bias = score_bias.view(-1, E)
    _opt(score_bias, torch.float32, "score_bias", shape=(None, E))
    _opt(modality, torch.uint8, "modality", shape=(T,))
    _opt(input_ids, torch.int32, "input_ids", shape=(T,))
    _opt(tid2eid, torch.int32, "tid2eid", shape=(None, k))
    _flags(flags)
    n_bias = 0 if score_bias is None else score_bias.shape[0]
    V = 0 if tid2eid is None else tid2eid.shape[0]
    ids = _out(ids, torch.int32, "ids", (T, k), logits.device)
    w = _out(w, torch.float32, "w", (T, k), logits.device)
    _check(lib().moe_route(_ptr(logits), _ptr(score_bias), _ptr(modality), _ptr(input_ids),
                           _ptr(tid2eid), T, E, k, n_bias, V, mode, float(scale), _ptr(ids),
                           _ptr(w), _ptr(flags), _stream()), "moe_route")
    return ids, w


def route_backward(logits, ids, dw, scale, flags=None, out=None):
    """Gradient of the routing weights with respect to the logits
    (moe_route_backward): returns d_logits[T,E] fp32 for dw[T,k]."""
    _need(logits, torch.float32, "logits", 2)
    T, E = logits.shape
    _need(ids, torch.int32, "ids", 2)
    k = ids.shape[1]
    _need(ids, torch.int32, "ids", shape=(T, k))
    _need(dw, torch.float32, "dw", shape=(T, k))
    _flags(flags)
    out = _out(out, torch.float32, "out", (T, E), logits.device)
    _check(lib().moe_route_backward(_ptr(logits), _ptr(ids), _ptr(dw), T, E, k, float(scale),
                                    _ptr(out), _ptr(flags), _stream()), "moe_route_backward")
    return out


def permute_workspace_size(T, k, E):
    return int(lib().moe_permute_workspace_size(T, k, E))


def permute(topk_ids, x, E, flags=None, workspace=None):
    """Returns dict(counts, offsets, dest, src, x_perm)."""
    _need(topk_ids, torch.int32, "topk_ids", 2)
    T, k = topk_ids.shape
    _need(x, torch.bfloat16, "x", shape=(T, None))
    _flags(flags)
    d = x.shape[1]
    dev = x.device
    ws_bytes = permute_workspace_size(T, k, E)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _need(workspace, torch.uint8, "workspace", 1)
    out = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               dest=torch.empty(T * k, dtype=torch.int32, device=dev),
               src=torch.empty(T * k, dtype=torch.int32, device=dev),
               x_perm=torch.empty((T * k, d), dtype=torch.bfloat16, device=dev))
    _check(lib().moe_permute(_ptr(topk_ids), _ptr(x), T, d, E, k, _ptr(out["counts"]),
                             _ptr(out["offsets"]), _ptr(out["dest"]), _ptr(out["src"]),
                             _ptr(out["x_perm"]), _ptr(flags), _ptr(workspace),
                             workspace.numel(), _stream()), "moe_permute")
    return out


def permute_noalloc(topk_ids, x, E, flags=None, out=None):
    """moe_permute_noalloc (the permutation with its scratch in the library's
    static device array): returns dict(counts, offsets, dest, src, x_perm).
    `out` may hold preallocated outputs (a dict of the same keys), so that the
    call itself allocates nothing."""
    _need(topk_ids, torch.int32, "topk_ids", 2)
    T, k = topk_ids.shape
    _need(x, torch.bfloat16, "x", shape=(T, None))
    _flags(flags)
    d = x.shape[1]
    dev = x.device
    out = dict(out or {})
    out["counts"] = _out(out.get("counts"), torch.int32, "counts", (E,), dev)
    out["offsets"] = _out(out.get("offsets"), torch.int32, "offsets", (E + 1,), dev)
    out["dest"] = _out(out.get("dest"), torch.int32, "dest", (T * k,), dev)
    out["src"] = _out(out.get("src"), torch.int32, "src", (T * k,), dev)
    out["x_perm"] = _out(out.get("x_perm"), torch.bfloat16, "x_perm", (T * k, d), dev)
    _check(lib().moe_permute_noalloc(_ptr(topk_ids), _ptr(x), T, d, E, k, _ptr(out["counts"]),
                                     _ptr(out["offsets"]), _ptr(out["dest"]), _ptr(out["src"]),
                                     _ptr(out["x_perm"]), _ptr(flags), _stream()),
           "moe_permute_noalloc")
    return out


def expert_ffn(a, offsets, w_gate, w_up, w_down, clamp_limit=10.0, clamp_mode=CLAMP_SYMMETRIC,
               h=None, y=None):
    """Grouped FFN: returns (h[rows,F] bf16, y[rows,d] fp32)."""
    _need(a, torch.bfloat16, "a", 2)
    _need(offsets, torch.int32, "offsets", 1)
    rows, d = a.shape
    _need(w_gate, torch.bfloat16, "w_gate", shape=(None, None, d))
    G, F, _ = w_gate.shape
    _need(w_up, torch.bfloat16, "w_up", shape=(G, F, d))
    _need(w_down, torch.bfloat16, "w_down", shape=(G, d, F))
    if offsets.numel() != G + 1:
        raise MoeError("offsets must have G + 1 entries")
    h = _out(h, torch.bfloat16, "h", (rows, F), a.device)
    y = _out(y, torch.float32, "y", (rows, d), a.device)
    _check(lib().moe_expert_ffn(_ptr(a), _ptr(offsets), G, rows, d, F, _ptr(w_gate), _ptr(w_up),
                                _ptr(w_down), float(clamp_limit), int(clamp_mode), _ptr(h),
                                _ptr(y), _stream()), "moe_expert_ffn")
    return h, y


def expert_ffn_packed(a, offsets, w_gate_p, w_up_p, w_down_p, G, F, clamp_limit=10.0,
                      clamp_mode=CLAMP_SYMMETRIC, h=None, y=None):
    """Grouped FFN on packed weights (pack_weights with PANEL_ROWS): returns
    (h[rows,F] bf16, y[rows,d] fp32)."""
    _need(a, torch.bfloat16, "a", 2)
    _need(offsets, torch.int32, "offsets", 1)
    rows, d = a.shape
    for name, t, n, k, p in (("w_gate", w_gate_p, F, d, 128), ("w_up", w_up_p, F, d, 128),
                             ("w_down", w_down_p, d, F, 256)):
        _need(t, torch.bfloat16, name, 1)
        if t.numel() * 2 != lib().moe_packed_weight_bytes(G, n, k, p):
            raise MoeError(f"{name} is not a packed [{G},{n},{k}] matrix (panel_rows {p})")
    if offsets.numel() != G + 1:
        raise MoeError("offsets must have G + 1 entries")
    h = _out(h, torch.bfloat16, "h", (rows, F), a.device)
    y = _out(y, torch.float32, "y", (rows, d), a.device)
    _check(lib().moe_expert_ffn_packed(_ptr(a), _ptr(offsets), G, rows, d, F, _ptr(w_gate_p),
                                       _ptr(w_up_p), _ptr(w_down_p), float(clamp_limit),
                                       int(clamp_mode), _ptr(h), _ptr(y), _stream()),
           "moe_expert_ffn_packed")
    return h, y


def combine(y_perm, dest, topk_w, y_shared=None, out_dtype=OUT_BF16, y=None):
    """y[T,d] = y_shared + sum_j topk_w[t,j] * y_perm[dest[t,j]]."""
    _need(y_perm, torch.float32, "y_perm", 2)
    _need(topk_w, torch.float32, "topk_w", 2)
    T, k = topk_w.shape
    rows, d = y_perm.shape
    _need(dest, torch.int32, "dest")
    if dest.numel() != T * k:
        raise MoeError(f"dest must have T k = {T * k} entries")
    _opt(y_shared, torch.float32, "y_shared", shape=(T, d))
    dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
    y = _out(y, dt, "y", (T, d), y_perm.device)
    _check(lib().moe_combine(_ptr(y_perm), _ptr(dest), _ptr(topk_w), _ptr(y_shared), T, d, k,
                             rows, int(out_dtype), _ptr(y), _stream()), "moe_combine")
    return y


def combine_backward(dy, y_perm, dest, topk_w, dy_perm=None, d_topk_w=None):
    """Backward of the combine (moe_combine_backward): returns
    (dy_perm[rows,d] fp32, d_topk_w[T,k] fp32).  A new dy_perm starts at
    zero, so rows no pair maps to are 0."""
    _need(topk_w, torch.float32, "topk_w", 2)
    T, k = topk_w.shape
    _need(y_perm, torch.float32, "y_perm", 2)
    rows, d = y_perm.shape
    _need(dy, torch.float32, "dy", shape=(T, d))
    _need(dest, torch.int32, "dest")
    if dest.numel() != T * k:
        raise MoeError(f"dest must have T k = {T * k} entries")
    if dy_perm is None:
        dy_perm = torch.zeros((rows, d), dtype=torch.float32, device=dy.device)
    _need(dy_perm, torch.float32, "dy_perm", shape=(rows, d))
    d_topk_w = _out(d_topk_w, torch.float32, "d_topk_w", (T, k), dy.device)
    _check(lib().moe_combine_backward(_ptr(dy), _ptr(y_perm), _ptr(dest), _ptr(topk_w), T, d, k,
                                      rows, _ptr(dy_perm), _ptr(d_topk_w), _stream()),
           "moe_combine_backward")
    return dy_perm, d_topk_w


def grouped_gemm_packed(a, offsets, w_packed, G, N, out=None):
    """out[r] = a[r] @ W[g].T for the rows of group g (moe_grouped_gemm_packed;
    w_packed = pack_weights(W [G, N, K], 256)); a new `out` starts at zero."""
    _need(a, torch.bfloat16, "a", 2)
    rows, K = a.shape
    _need(offsets, torch.int32, "offsets", shape=(G + 1,))
    _need(w_packed, torch.bfloat16, "w_packed", 1)
    if w_packed.numel() * 2 != lib().moe_packed_weight_bytes(G, N, K, 256):
        raise MoeError(f"w_packed is not a packed [{G},{N},{K}] matrix (panel_rows 256)")
    if out is None:
        out = torch.zeros((rows, N), dtype=torch.float32, device=a.device)
    _need(out, torch.float32, "out", shape=(rows, N))
    _check(lib().moe_grouped_gemm_packed(_ptr(a), _ptr(offsets), G, rows, K, N, _ptr(w_packed),
                                         _ptr(out), _stream()), "moe_grouped_gemm_packed")
    return out


def grouped_wgrad(dy, a, offsets, G=None, out=None):
    """dw[g] = dy[rows of g]^T a[rows of g] (fp32 [G, M, K]) for bf16 dy
    [rows, M] and a [rows, K]: the weight gradient of a grouped matmul.
    offsets [G+1] int32 (device) or None for one group of all rows."""
    _need(dy, torch.bfloat16, "dy", 2)
    rows, M = dy.shape
    _need(a, torch.bfloat16, "a", shape=(rows, None))
    K = a.shape[1]
    if offsets is None:
        G = 1
    else:
        _need(offsets, torch.int32, "offsets", 1)
        G = offsets.numel() - 1
    out = _out(out, torch.float32, "out", (G, M, K), dy.device)
    _check(lib().moe_grouped_wgrad(_ptr(dy), _ptr(a), _ptr(offsets), G, rows, M, K, _ptr(out),
                                   _stream()), "moe_grouped_wgrad")
    return out


def swiglu_backward(gate, up, dh, clamp_limit=10.0, clamp_mode=CLAMP_SYMMETRIC, dgate=None,
                    dup=None):
    """Backward of the clamped SwiGLU (moe_swiglu_backward): returns
    (dgate, dup), fp32 tensors of gate's shape."""
    _need(gate, torch.float32, "gate")
    shape = tuple(gate.shape)
    _need(up, torch.float32, "up", shape=shape)
    _need(dh, torch.float32, "dh", shape=shape)
    dgate = _out(dgate, torch.float32, "dgate", shape, gate.device)
    dup = _out(dup, torch.float32, "dup", shape, gate.device)
    _check(lib().moe_swiglu_backward(_ptr(gate), _ptr(up), _ptr(dh), gate.numel(),
                                     float(clamp_limit), int(clamp_mode), _ptr(dgate), _ptr(dup),
                                     _stream()), "moe_swiglu_backward")
    return dgate, dup


# panel height each matrix is packed with for moe_forward
PANEL_ROWS = dict(w_g=256, w_gate=128, w_up=128, w_down=256, s_gate=128, s_up=128, s_down=256)


def pack_weights(w, panel_rows):
    """Packed copy (moe_pack_weights layout, panels of `panel_rows` rows) of
    bf16 weights [G,N,K] or [N,K]."""
    _need(w, torch.bfloat16, "w")
    shape = tuple(w.shape)
    G, N, K = (1,) + shape if w.dim() == 2 else shape
    nbytes = int(lib().moe_packed_weight_bytes(G, N, K, panel_rows))
    if nbytes == 0:
        raise MoeError(f"cannot pack weights of shape {shape} in panels of {panel_rows}")
    out = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=w.device)
    _check(lib().moe_pack_weights(_ptr(w), G, N, K, panel_rows, _ptr(out), _stream()),
           "moe_pack_weights")
    return out


def pack_weights_fp8(w, panel_rows):
    """MXFP8 copy (moe_pack_weights_fp8: E4M3 codes in the packed layout, one
    power-of-two scale per 32 values of K) of bf16 weights [G,N,K] or [N,K];
    returns (codes uint8 tensor, scale bytes uint8 tensor)."""
    _need(w, torch.bfloat16, "w")
    shape = tuple(w.shape)
    G, N, K = (1,) + shape if w.dim() == 2 else shape
    nbytes = int(lib().moe_packed_fp8_weight_bytes(G, N, K, panel_rows))
    if nbytes == 0:
        raise MoeError(f"cannot pack weights of shape {shape} in panels of {panel_rows}")
    codes = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    scales = torch.empty(int(lib().moe_packed_fp8_scale_bytes(G, N, K, panel_rows)),
                         dtype=torch.uint8, device=w.device)
    _check(lib().moe_pack_weights_fp8(_ptr(w), G, N, K, panel_rows, _ptr(codes), _ptr(scales),
                                      _stream()), "moe_pack_weights_fp8")
    return codes, scales


def quantize_mxfp8(a, codes=None, scales=None):
    """MXFP8 quantisation of bf16 rows a [rows, K] along K (moe_quantize_mxfp8):
    returns (codes uint8 [rows, K], scale bytes X + 127 uint8 [rows, K/32])."""
    _need(a, torch.bfloat16, "a", 2)
    rows, K = a.shape
    codes = _out(codes, torch.uint8, "codes", (rows, K), a.device)
    scales = _out(scales, torch.uint8, "scales", (rows, K // 32), a.device)
    _check(lib().moe_quantize_mxfp8(_ptr(a), rows, K, _ptr(codes), _ptr(scales), _stream()),
           "moe_quantize_mxfp8")
    return codes, scales


def expert_ffn_a8w4(a8, a_scale, offsets, w_gate, w_up, w_down, G, F, clamp_limit=10.0,
                    clamp_mode=CLAMP_SYMMETRIC):
    """Grouped FFN in the A8W4 mode (moe_expert_ffn_a8w4): a8 / a_scale from
    quantize_mxfp8, w_* = (codes, scales) pairs from pack_weights_fp4
    (panel rows 128, 128, 256).  Returns (h8 uint8 [rows, F], h_scale uint8
    [rows, F/32], y fp32 [rows, d])."""
    _need(a8, torch.uint8, "a8", 2)
    rows, d = a8.shape
    _need(a_scale, torch.uint8, "a_scale", shape=(rows, d // 32))
    _need(offsets, torch.int32, "offsets", shape=(G + 1,))
    dev = a8.device
    h8 = torch.empty((rows, F), dtype=torch.uint8, device=dev)
    hs = torch.empty((rows, F // 32), dtype=torch.uint8, device=dev)
    y = torch.zeros((rows, d), dtype=torch.float32, device=dev)
    (cg, sg), (cu, su), (cd, sd) = w_gate, w_up, w_down
    _check(lib().moe_expert_ffn_a8w4(_ptr(a8), _ptr(a_scale), _ptr(offsets), G, rows, d, F,
                                     _ptr(cg), _ptr(cu), _ptr(cd), _ptr(sg), _ptr(su), _ptr(sd),
                                     float(clamp_limit), int(clamp_mode), _ptr(h8), _ptr(hs),
                                     _ptr(y), _stream()), "moe_expert_ffn_a8w4")
    return h8, hs, y


def pack_weights_fp4(w, panel_rows):
    """MXFP4 copy (moe_pack_weights_fp4: E2M1 codes in the packed layout, one
    power-of-two scale per 32 values of K) of bf16 weights [G,N,K] or [N,K];
    returns (codes uint8 tensor, scale bytes uint8 tensor)."""
    _need(w, torch.bfloat16, "w")
    shape = tuple(w.shape)
    G, N, K = (1,) + shape if w.dim() == 2 else shape
    nbytes = int(lib().moe_packed_fp4_weight_bytes(G, N, K, panel_rows))
    if nbytes == 0:
        raise MoeError(f"cannot pack weights of shape {shape} in panels of {panel_rows}")
    codes = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    scales = torch.empty(int(lib().moe_packed_fp8_scale_bytes(G, N, K, panel_rows)),
                         dtype=torch.uint8, device=w.device)
    _check(lib().moe_pack_weights_fp4(_ptr(w), G, N, K, panel_rows, _ptr(codes), _ptr(scales),
                                      _stream()), "moe_pack_weights_fp4")
    return codes, scales


class MoeLayer:
    """One fine-grained MoE layer on the device: holds the weights, the config
    and a preallocated workspace; ``forward`` is one C-ABI call."""

    def __init__(self, T, d, E, k, F, F_shared, weights, mode=MODE_TOPK, n_bias=0, V=0,
                 scale=1.0, clamp_limit=10.0, clamp_mode=CLAMP_SYMMETRIC, out_dtype=OUT_BF16,
                 packed=False):
        self.cfg = MoeCfg(T=T, d=d, E=E, k=k, F=F, F_shared=F_shared, mode=mode, n_bias=n_bias,
                          V=V, scale=float(scale), clamp_limit=float(clamp_limit),
                          clamp_mode=int(clamp_mode), out_dtype=int(out_dtype))
        self.weights = dict(weights)
        self.plain = dict(weights)     # the [out, in] matrices (for the backward's layouts)
        self.bw = None
        _need(self.weights["w_g"], torch.bfloat16, "w_g", shape=(E, d))
        _need(self.weights["w_gate"], torch.bfloat16, "w_gate", shape=(E, F, d))
        _need(self.weights["w_up"], torch.bfloat16, "w_up", shape=(E, F, d))
        _need(self.weights["w_down"], torch.bfloat16, "w_down", shape=(E, d, F))
        if F_shared > 0:
            _need(self.weights["s_gate"], torch.bfloat16, "s_gate", shape=(F_shared, d))
            _need(self.weights["s_up"], torch.bfloat16, "s_up", shape=(F_shared, d))
            _need(self.weights["s_down"], torch.bfloat16, "s_down", shape=(d, F_shared))
        _opt(self.weights.get("logit_offset"), torch.float32, "logit_offset", shape=(E,))
        if mode == MODE_TOPK and n_bias > 0:
            _need(self.weights.get("score_bias"), torch.float32, "score_bias",
                  shape=(n_bias, E))
        if mode == MODE_HASH:
            _need(self.weights.get("tid2eid"), torch.int32, "tid2eid", shape=(V, k))
        fp8 = packed == "fp8"
        a8w4 = packed == "a8w4"
        fp4 = packed == "fp4" or a8w4
        if packed:
            # one-time layout change at load time (moe_pack_weights; with
            # packed="fp8" / "fp4" the routed expert matrices are quantised to
            # MXFP8 / MXFP4 by moe_pack_weights_fp8 / _fp4 instead; "a8w4":
            # MXFP4 weights and MXFP8 activations)
            for key in MATRIX_NAMES:
                if self.weights.get(key) is None:
                    continue
                if (fp8 or fp4) and key in ("w_gate", "w_up", "w_down"):
                    pack = pack_weights_fp8 if fp8 else pack_weights_fp4
                    self.weights[key], self.weights[key + "_scale"] = pack(
                        self.weights[key], PANEL_ROWS[key])
                else:
                    self.weights[key] = pack_weights(self.weights[key], PANEL_ROWS[key])
        self.packed = (WEIGHTS_FP8 if fp8 else WEIGHTS_A8W4 if a8w4 else WEIGHTS_FP4 if fp4
                       else int(bool(packed)))
        self.cw = MoeWeights(packed=self.packed,
                             **{n: _ptr(self.weights.get(n)) for n in WEIGHT_NAMES})
        self.device = self.weights["w_g"].device
        self.ws_bytes = int(lib().moe_forward_workspace_size(ctypes.byref(self.cfg)))
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.flags = torch.zeros(1, dtype=torch.int32, device=self.device)

    def backward_weights(self):
        """The weights in the layouts of the backward's input-gradient
        products (moe_bwd_weights): packed once per weight update from the
        [out, in] matrices (transposed and concatenated copies, then
        moe_pack_weights with 256-row panels)."""
        if self.bw is None:
            p = self.plain
            bw = dict(w_g=p["w_g"].contiguous(),
                      w_down_t=pack_weights(p["w_down"].transpose(1, 2).contiguous(), 256),
                      w_gu_t=pack_weights(torch.cat([p["w_gate"], p["w_up"]], dim=1)
                                          .transpose(1, 2).contiguous(), 256))
            if self.cfg.F_shared > 0:
                bw["s_down_t"] = pack_weights(p["s_down"].t().contiguous(), 256)
                bw["s_gu_t"] = pack_weights(torch.cat([p["s_gate"], p["s_up"]], dim=0)
                                            .t().contiguous(), 256)
            self.bw = bw
            self.cbw = MoeBwdWeights(**{n: _ptr(bw.get(n)) for n in BWD_WEIGHT_NAMES})
            self.bws_bytes = int(lib().moe_backward_workspace_size(ctypes.byref(self.cfg)))
            self.bworkspace = torch.empty(self.bws_bytes, dtype=torch.uint8, device=self.device)
        return self.bw

    def backward(self, x, dy, input_ids=None, modality=None, grads=None):
        """Gradients of the layer output for an output gradient dy [T, d]
        fp32 (one moe_backward call): dict with dx, dw_g, dw_gate, dw_up,
        dw_down and, with a shared expert, ds_gate, ds_up, ds_down (fp32)."""
        c = self.cfg
        if self.packed != 1:
            raise MoeError("moe_backward takes bf16 packed weights (packed=True)")
        _need(x, torch.bfloat16, "x", shape=(c.T, c.d))
        _need(dy, torch.float32, "dy", shape=(c.T, c.d))
        _opt(input_ids, torch.int32, "input_ids", shape=(c.T,))
        _opt(modality, torch.uint8, "modality", shape=(c.T,))
        self.backward_weights()
        shapes = dict(dx=(c.T, c.d), dw_g=(c.E, c.d), dw_gate=(c.E, c.F, c.d),
                      dw_up=(c.E, c.F, c.d), dw_down=(c.E, c.d, c.F))
        if c.F_shared > 0:
            shapes.update(ds_gate=(c.F_shared, c.d), ds_up=(c.F_shared, c.d),
                          ds_down=(c.d, c.F_shared))
        grads = dict(grads or {})
        for n, shp in shapes.items():
            grads[n] = _out(grads.get(n), torch.float32, n, shp, x.device)
        cg = MoeGrads(**{n: _ptr(grads.get(n)) for n in GRAD_NAMES})
        _check(lib().moe_backward(ctypes.byref(c), ctypes.byref(self.cw), ctypes.byref(self.cbw),
                                  _ptr(x), _ptr(input_ids), _ptr(modality), _ptr(dy),
                                  ctypes.byref(cg), _ptr(self.flags), _ptr(self.bworkspace),
                                  self.bws_bytes, _stream()), "moe_backward")
        return grads

    @classmethod
    def from_workload(cls, w, inputs, out_dtype=OUT_BF16, packed=False):
        n_bias = 0 if inputs.get("score_bias") is None else inputs["score_bias"].shape[0]
        return cls(w.T, w.d, w.E, w.k, w.F, w.Fs, inputs, mode=w.mode, n_bias=n_bias, V=w.V,
                   scale=w.scale, clamp_limit=w.clamp_limit, clamp_mode=w.clamp_mode,
                   out_dtype=out_dtype, packed=packed)

    def forward(self, x, input_ids=None, modality=None, y=None, logits=None, ids=None, w=None,
                events=None):
        """One layer forward (one C-ABI call).  `events`: optional list of
        FORWARD_STAGES + 1 recorded torch.cuda.Event objects, re-recorded
        around the stages."""
        c = self.cfg
        _need(x, torch.bfloat16, "x", 2)
        if tuple(x.shape) != (c.T, c.d):
            raise MoeError(f"x must be [{c.T}, {c.d}]")
        _opt(input_ids, torch.int32, "input_ids", shape=(c.T,))
        _opt(modality, torch.uint8, "modality", shape=(c.T,))
        _opt(logits, torch.float32, "logits", shape=(c.T, c.E))
        _opt(ids, torch.int32, "ids", shape=(c.T, c.k))
        _opt(w, torch.float32, "w", shape=(c.T, c.k))
        dt = torch.float32 if c.out_dtype == OUT_F32 else torch.bfloat16
        y = _out(y, dt, "y", (c.T, c.d), x.device)
        ev = None
        if events is not None:
            if len(events) != FORWARD_STAGES + 1:
                raise MoeError(f"need {FORWARD_STAGES + 1} events")
            ev = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        _check(lib().moe_forward_timed(ctypes.byref(c), ctypes.byref(self.cw), _ptr(x),
                                       _ptr(input_ids), _ptr(modality), _ptr(y), _ptr(logits),
                                       _ptr(ids), _ptr(w), _ptr(self.flags),
                                       _ptr(self.workspace), self.ws_bytes, _stream(), ev),
               "moe_forward")
        return y
